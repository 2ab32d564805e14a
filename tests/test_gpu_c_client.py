"""The device calls from plain C: tests/c_client/pa_device_client (built by
__graft_entry__.build() from pa_device_client.c) places three sequences
with the block manager, writes their K/V with pa_cache_write, decodes with
split-K, then forks one, appends with copy-on-write through pa_copy_blocks
and decodes again, all through the C ABI with hipMalloc'd buffers.  Its
inputs come from a 32-bit LCG repeated here; its outputs are compared with
the oracle."""
import os
import subprocess

import numpy as np
import pytest

import pa_gpu as G
from oracle import block_manager as obm
from oracle import paged as opg

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_client", "pa_device_client")
HQ, HKV, D, BS, NB, MAXB = 8, 2, 64, 16, 24, 8


class Lcg:
    """x <- 1664525 x + 1013904223 (mod 2^32); value (x >> 8) * 2^-23 - 1."""

    def __init__(self, seed):
        self.x = seed

    def values(self, n):
        out = np.empty(n, dtype=np.float32)
        x = self.x
        for i in range(n):
            x = (x * 1664525 + 1013904223) & 0xFFFFFFFF
            out[i] = (x >> 8) * 2.0 ** -23 - 1.0
        self.x = x
        return out


def padded(bm, sids):
    t = np.full((len(sids), MAXB), -1, dtype=np.int32)
    for i, s in enumerate(sids):
        row = bm.table(s)
        t[i, :len(row)] = row
    return t


def test_device_calls_from_c():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built (run __graft_entry__.build())")
    G.say("[c client] running pa_device_client")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"client failed:\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"
    o = {}
    for line in r.stdout.splitlines():
        name, *vals = line.split(" ")
        o[name] = vals

    rng = Lcg(12345)
    bm = obm.BlockManager(NB, BS)
    lens0 = [1, 37, 100]
    slots = np.concatenate([bm.add(s, n) for s, n in enumerate(lens0)]).astype(np.int64)
    assert [int(v) for v in o["slots"]] == slots.tolist()
    T = int(sum(lens0))
    k0 = rng.values(T * HKV * D).reshape(T, HKV, D)
    v0 = rng.values(T * HKV * D).reshape(T, HKV, D)
    q1 = rng.values(3 * HQ * D).reshape(3, HQ, D)
    kp = np.zeros((NB, HKV, BS, D))
    vp = np.zeros((NB, HKV, BS, D))
    opg.cache_write(kp, vp, "f32", k0, v0, "f32", slots)
    ref1 = opg.paged_decode(q1, kp, vp, padded(bm, [0, 1, 2]), np.array(lens0), 0.125)
    got1 = np.array([float(v) for v in o["out1"]]).reshape(3, HQ, D)
    G.assert_close(got1, ref1, "f32", "C client: split-K decode")

    bm.fork(2, 3)
    slots2, cow = bm.append([2, 3])
    assert [int(v) for v in o["slots2"]] == list(slots2)
    assert [int(v) for v in o["cow"]] == [x for p in cow for x in p] and len(cow) == 1
    kn = rng.values(2 * HKV * D).reshape(2, HKV, D)
    vn = rng.values(2 * HKV * D).reshape(2, HKV, D)
    q2 = rng.values(2 * HQ * D).reshape(2, HQ, D)
    opg.copy_blocks(kp, vp, cow)
    opg.cache_write(kp, vp, "f32", kn, vn, "f32", np.asarray(slots2, dtype=np.int64))
    ref2 = opg.paged_decode(q2, kp, vp, padded(bm, [2, 3]), np.array([101, 101]), 0.125)
    got2 = np.array([float(v) for v in o["out2"]]).reshape(2, HQ, D)
    G.assert_close(got2, ref2, "f32", "C client: decode after fork and copy-on-write")
    # The fork shares all but the last block, and the two last tokens differ.
    assert not np.allclose(ref2[0], ref2[1])
