"""Host logic of bench.py that runs without a GPU: the one-GPU refusal, the
HBM-counter summary (calibration by the copy kernel's known bytes) and the
digest check that ties stored counter data to the decode sources."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _counter_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, value in KiB) as rocprofv3 writes them."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, k, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": counter,
                        "Counter_Value": v})
        # a counter of another pass in the same file is ignored
        w.writerow({"Dispatch_Id": 99, "Kernel_Name": "void pa::move_blocks_kernel(...)",
                    "Counter_Name": "SQ_WAVES", "Counter_Value": 1.0})


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_summarize_counters_scales_by_the_calibration_copy(tmp_path):
    copy = "void pa::move_blocks_kernel(...)"
    dec = "void pa::decode_balanced_mfma_kernel<pa::BF16, pa::BF16, 16, 4>(...)"
    red = "void pa::balanced_reduce_wave_kernel<pa::BF16, 128, 4>(...)"
    true_kib = 256.0 * 1024  # the calibration copy moves 256 MiB each way
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # The fetch counter reads half the copy's true bytes, the write counter all of them.
    _counter_csv(fetch, "FETCH_SIZE", [(1, copy, true_kib / 2), (2, dec, 1000.0), (3, dec, 3000.0),
                                       (4, dec, 2000.0), (5, red, 10.0)])
    _counter_csv(write, "WRITE_SIZE", [(1, copy, true_kib), (2, dec, 7.0), (3, dec, 9.0),
                                       (4, dec, 8.0), (5, red, 4.0)])
    out = tmp_path / "counters.json"
    d = bench.summarize_counters(str(fetch), str(write), "wl", str(out))
    assert d["fetch_scale"] == pytest.approx(2.0)
    assert d["write_scale"] == pytest.approx(1.0)
    k = d["kernels"]
    # medians per dispatch, KiB -> bytes, times the scale
    assert k["decode_balanced"]["fetch_bytes"] == pytest.approx(2000.0 * 1024 * 2.0)
    assert k["decode_balanced"]["write_bytes"] == pytest.approx(8.0 * 1024)
    assert k["balanced_reduce"]["fetch_bytes"] == pytest.approx(10.0 * 1024 * 2.0)
    assert k["balanced_reduce"]["write_bytes"] == pytest.approx(4.0 * 1024)
    assert d["hbm_bytes_per_launch"] == round((2000.0 * 2 + 8.0 + 10.0 * 2 + 4.0) * 1024)
    assert d["source_digest"] == bench.kernel_source_digest()
    assert json.loads(out.read_text()) == d


def test_stored_traffic_is_null_unless_the_sources_match(tmp_path, monkeypatch):
    digest = bench.kernel_source_digest()  # the decode sources of this tree
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: digest)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("wl") is None  # no stored counters
    (tmp_path / "profiles").mkdir()
    path = tmp_path / "profiles" / "decode_kernel_wl_counters.json"
    rec = {"source_digest": "0" * 16,
           "kernels": {"decode_balanced": {"fetch_bytes": 100.4, "write_bytes": 20.3}}}
    path.write_text(json.dumps(rec))
    assert bench.stored_traffic("wl") is None  # taken on other sources
    rec["source_digest"] = digest
    path.write_text(json.dumps(rec))
    assert bench.stored_traffic("wl") == round(100.4 + 20.3)
