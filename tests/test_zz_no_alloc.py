"""pa_decode_no_alloc (the decode entry point that allocates nothing: its
split-K partials live in the library's static per-device scratch) against
pa_decode with a caller workspace, through the C ABI: two calls in a row,
the second on a smaller batch, in the balanced split and with fixed
partitions.  The two entry points run the same kernels on the same inputs,
so their outputs must agree bit for bit; the first call is also checked
against the oracle."""
import numpy as np
import pytest
import torch

import pa_gpu as G
from paged_kv_cache_11_amd import binding as pa
from paged_kv_cache_11_amd import workloads as wl

pytestmark = pytest.mark.gpu
BAL = pa.PA_PARTITION_BALANCED


@pytest.fixture(scope="module")
def llama():
    b = wl.llama3_8b_decode()
    G.say(f"[no-alloc] {b.num_seqs} seqs, {b.num_blocks} blocks")
    kp, vp = G.gpu_pool(b)
    G.gpu_fill(b, kp, vp)
    qt = G.query_tensor(b)
    return b, kp, vp, qt


def _both(b, kp, vp, qt, lens, ps, flags):
    tables = torch.from_numpy(np.ascontiguousarray(b.block_tables)).to(G.DEV)
    dlens = torch.from_numpy(np.ascontiguousarray(lens)).to(G.DEV)
    msl = int(lens.max())
    pa.validate_decode(b.block_tables, lens, msl, b.num_blocks, b.block_size)
    ref = torch.empty_like(qt)
    pa.pa_decode(ref, qt, kp, vp, tables, dlens, msl, b.scale, partition_size=ps, flags=flags)
    got = torch.full_like(qt, float("nan"))
    pa.pa_decode_no_alloc(got, qt, kp, vp, tables, dlens, msl, b.scale, partition_size=ps,
                          flags=flags)
    torch.cuda.synchronize()
    return got.float().cpu().numpy(), ref.float().cpu().numpy()


@pytest.mark.parametrize("ps,flags", [(BAL, pa.PA_DECODE_READ_ONCE), (BAL, pa.PA_DECODE_SHARED),
                                      (512, 0)])
def test_no_alloc_matches_pa_decode_twice(llama, ps, flags):
    b, kp, vp, qt = llama
    G.say(f"[no-alloc] partition {ps}, flags {flags}: full batch")
    got, ref = _both(b, kp, vp, qt, b.seq_lens, ps, flags)
    assert np.array_equal(got, ref)
    okp, ovp = G.oracle_pool(b)
    seqs = list(range(0, b.num_seqs, 4))
    oref = G.oracle_decode(b, okp, ovp, G.query_f64(qt), seqs=seqs)
    G.assert_close(got.astype(np.float64), oref, "bf16", "no-alloc decode", rows=seqs)
    # A second call on a smaller batch: shorter contexts, some empty.  The
    # scratch still holds the first call's states; nothing of them may leak.
    G.say(f"[no-alloc] partition {ps}, flags {flags}: smaller batch")
    small = np.where(np.arange(b.num_seqs) % 3 == 0, 0, b.seq_lens // 4).astype(np.int32)
    got2, ref2 = _both(b, kp, vp, qt, small, ps, flags)
    assert np.array_equal(got2, ref2)
    assert np.all(got2[small == 0] == 0)


def test_no_alloc_refuses_a_split_past_its_scratch():
    # 64 sequences of up to 32768 tokens in 512-token partitions need
    # 64 * 32 heads * 64 partitions * (128 + 2) floats = 68 MB of partials.
    need = pa.pa_decode_workspace_size(64, 32, 8, 128, 32768, 512)
    assert need > 48 * 1024 * 1024
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device=G.DEV)
    pool = torch.zeros((2048, 8, 16, 128), dtype=torch.bfloat16, device=G.DEV)
    tables = torch.zeros((64, 2048), dtype=torch.int32, device=G.DEV)
    lens = torch.ones(64, dtype=torch.int32, device=G.DEV)
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.pa_decode_no_alloc(q, q, pool, pool, tables, lens, 32768, 0.1, partition_size=512)
    assert e.value.code == pa.PA_ERR_WORKSPACE and "scratch" in str(e.value)
