"""CPU checks of the C ABI: the library loads, exports every function
include/pa.h declares, and rejects bad host arguments before any launch
(these paths never touch a GPU)."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_11_amd import binding as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pa.h"), encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = pa.load()
    names = _declared()
    assert names and "pa_decode" in names and "pa_prefill_chunk" in names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(pa.exported_symbols()) == names


def test_version_and_strerror():
    assert pa.pa_version() >= 100
    lib = pa.load()
    for c in (0, -1, -2, -3, -4, 7):
        assert lib.pa_strerror(c)


def test_pool_bytes_and_workspace_sizes():
    assert pa.pa_pool_bytes(10, 8, 16, 128, pa.PA_BF16) == 10 * 8 * 16 * 128 * 2
    assert pa.pa_pool_bytes(10, 8, 32, 128, pa.PA_FP8_E4M3) == 10 * 8 * 32 * 128
    assert pa.pa_pool_bytes(0, 8, 16, 128, pa.PA_BF16) == 0
    assert pa.pa_decode_workspace_size(64, 32, 8, 128, 4096, 0) == 0
    assert pa.pa_decode_workspace_size(64, 32, 8, 128, 512, 512) == 0
    n = 8 * 32 * 64
    want = ((n * 128 * 4 + 255) // 256) * 256 + ((n * 2 * 4 + 255) // 256) * 256
    assert pa.pa_decode_workspace_size(8, 32, 8, 128, 32768, 512) == want
    nb = 4096 * 2 * 4  # two partial states of 4 heads per wavefront of the largest grid
    want_b = (((nb * 128 * 4 + 255) // 256) * 256 + ((nb * 2 * 4 + 255) // 256) * 256
              + 4096 * 2 * 4    # + a two-word merge task per wavefront
              + ((64 * 8 * 8 + 255) // 256) * 256)   # + a two-word cut record per (seq, KV head)
    assert pa.pa_decode_workspace_size(64, 32, 8, 128, 4096, pa.PA_PARTITION_BALANCED) == want_b
    assert pa.pa_decode_workspace_size(64, 30, 8, 128, 4096, 0) == 0


P = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first


def _decode(**kw):
    a = dict(out=P, query=P, q_dtype=pa.PA_BF16, num_seqs=4, num_heads=32, head_size=128,
             k_cache=P, v_cache=P, cache_dtype=pa.PA_BF16, num_blocks=100, block_size=16,
             num_kv_heads=8, block_tables=P, max_blocks_per_seq=8, seq_lens=P, max_seq_len=128,
             scale=0.1, k_scale=1.0, v_scale=1.0, partition_size=0, flags=0, workspace=None,
             workspace_bytes=0, stream=None)
    a.update(kw)
    return pa.load().pa_decode(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(k_cache=None), pa.PA_ERR_INVALID),
    (dict(num_heads=30), pa.PA_ERR_INVALID),
    (dict(partition_size=24), pa.PA_ERR_INVALID),
    (dict(max_seq_len=200), pa.PA_ERR_INVALID),
    (dict(head_size=96), pa.PA_ERR_UNSUPPORTED),
    (dict(block_size=8, max_seq_len=64), pa.PA_ERR_UNSUPPORTED),
    (dict(num_heads=48, num_kv_heads=3), pa.PA_ERR_UNSUPPORTED),
    (dict(q_dtype=pa.PA_F32), pa.PA_ERR_UNSUPPORTED),
    (dict(q_dtype=pa.PA_F32, cache_dtype=pa.PA_F32), pa.PA_ERR_UNSUPPORTED),
    (dict(cache_dtype=9), pa.PA_ERR_INVALID),
    (dict(scale=float("nan")), pa.PA_ERR_INVALID),
    (dict(partition_size=32), pa.PA_ERR_WORKSPACE),
    (dict(partition_size=32, workspace=P, workspace_bytes=100), pa.PA_ERR_WORKSPACE),
    (dict(partition_size=pa.PA_PARTITION_BALANCED), pa.PA_ERR_WORKSPACE),
    (dict(partition_size=-2), pa.PA_ERR_INVALID),
    (dict(out=None), pa.PA_ERR_INVALID),
    # flags: unknown bits, contradictory hints, two engines, an engine not built
    (dict(flags=0x10), pa.PA_ERR_INVALID),
    (dict(flags=pa.PA_DECODE_READ_ONCE | pa.PA_DECODE_SHARED), pa.PA_ERR_INVALID),
    (dict(flags=pa.PA_DECODE_ENGINE_VALU | pa.PA_DECODE_ENGINE_MFMA), pa.PA_ERR_INVALID),
    (dict(flags=pa.PA_DECODE_ENGINE_MFMA, head_size=64, max_seq_len=128), pa.PA_ERR_UNSUPPORTED),
    # misaligned arrays (the kernels move 16-byte vectors)
    (dict(query=ctypes.c_void_p(24)), pa.PA_ERR_INVALID),
    (dict(out=ctypes.c_void_p(40)), pa.PA_ERR_INVALID),
    (dict(block_tables=ctypes.c_void_p(18)), pa.PA_ERR_INVALID),
    (dict(k_cache=ctypes.c_void_p(8)), pa.PA_ERR_INVALID),
    # fixed partitions put sequences on a grid axis of at most 65535
    (dict(num_seqs=70000), pa.PA_ERR_INVALID),
])
def test_decode_rejects_bad_host_arguments(kw, code):
    assert _decode(**kw) == code
    assert pa.load().pa_last_error()


def _append(**kw):
    a = dict(out=P, query=P, q_dtype=pa.PA_BF16, num_seqs=4, num_heads=32, head_size=128,
             k_new=P, v_new=P, k_cache=P, v_cache=P, cache_dtype=pa.PA_BF16, num_blocks=100,
             block_size=16, num_kv_heads=8, block_tables=P, max_blocks_per_seq=8, seq_lens=P,
             max_seq_len=128, scale=0.1, k_scale=1.0, v_scale=1.0, flags=0, workspace=None,
             workspace_bytes=0, stream=None)
    a.update(kw)
    return pa.load().pa_decode_append(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(k_new=None), pa.PA_ERR_INVALID),
    (dict(v_new=None), pa.PA_ERR_INVALID),
    (dict(k_new=ctypes.c_void_p(24)), pa.PA_ERR_INVALID),
    # the fused append runs on the matrix-core engine only
    (dict(flags=pa.PA_DECODE_ENGINE_VALU), pa.PA_ERR_UNSUPPORTED),
    (dict(head_size=64), pa.PA_ERR_UNSUPPORTED),
    (dict(num_heads=16), pa.PA_ERR_UNSUPPORTED),
    (dict(q_dtype=pa.PA_F32, cache_dtype=pa.PA_F32, head_size=64), pa.PA_ERR_UNSUPPORTED),
    (dict(cache_dtype=pa.PA_FP8_E4M3, k_scale=0.0),
     pa.PA_ERR_INVALID),
    (dict(), pa.PA_ERR_WORKSPACE),
])
def test_decode_append_rejects_bad_host_arguments(kw, code):
    assert _append(**kw) == code
    assert pa.load().pa_last_error()


def test_decode_append_with_no_sequences_is_a_noop():
    assert _append(num_seqs=0, out=None, query=None, k_new=None, v_new=None) == pa.PA_OK


def test_decode_with_no_sequences_is_a_noop():
    assert _decode(num_seqs=0, out=None, query=None) == pa.PA_OK


def test_cache_write_and_copy_validation():
    lib = pa.load()
    # fp32 source into a bf16 cache is not a supported conversion.
    assert lib.pa_cache_write(P, P, pa.PA_F32, 4, P, P, pa.PA_BF16, 10, 16, 8, 128, P, 1.0, 1.0,
                              None) == pa.PA_ERR_UNSUPPORTED
    # fp8 quantisation needs positive finite scales.
    assert lib.pa_cache_write(P, P, pa.PA_BF16, 4, P, P, pa.PA_FP8_E4M3, 10, 16, 8, 128, P, 0.0,
                              1.0, None) == pa.PA_ERR_INVALID
    assert lib.pa_cache_write(P, P, pa.PA_BF16, -1, P, P, pa.PA_BF16, 10, 16, 8, 128, P, 1.0, 1.0,
                              None) == pa.PA_ERR_INVALID
    assert lib.pa_cache_write(None, None, pa.PA_BF16, 0, P, P, pa.PA_BF16, 10, 16, 8, 128, None,
                              1.0, 1.0, None) == pa.PA_OK
    assert lib.pa_cache_write(P, P, pa.PA_BF16, 2, P, P, pa.PA_BF16, 10, 16, 8, 4, P, 1.0, 1.0,
                              None) == pa.PA_ERR_UNSUPPORTED  # 8-byte head rows
    assert lib.pa_copy_blocks(P, P, pa.PA_BF16, 10, 16, 8, 128, None, 0, None) == pa.PA_OK
    assert lib.pa_copy_blocks(P, P, pa.PA_BF16, 10, 16, 8, 128, None, 3, None) == pa.PA_ERR_INVALID
    assert lib.pa_copy_blocks(None, P, pa.PA_BF16, 10, 16, 8, 128, P, 3, None) == pa.PA_ERR_INVALID
    # misaligned key / value / slot_mapping / block_mapping
    assert lib.pa_cache_write(ctypes.c_void_p(8), P, pa.PA_BF16, 2, P, P, pa.PA_BF16, 10, 16, 8,
                              128, P, 1.0, 1.0, None) == pa.PA_ERR_INVALID
    assert lib.pa_cache_write(P, ctypes.c_void_p(20), pa.PA_BF16, 2, P, P, pa.PA_BF16, 10, 16, 8,
                              128, P, 1.0, 1.0, None) == pa.PA_ERR_INVALID
    assert lib.pa_cache_write(P, P, pa.PA_BF16, 2, P, P, pa.PA_BF16, 10, 16, 8, 128,
                              ctypes.c_void_p(12), 1.0, 1.0, None) == pa.PA_ERR_INVALID
    assert lib.pa_copy_blocks(P, P, pa.PA_BF16, 10, 16, 8, 128, ctypes.c_void_p(4), 3,
                              None) == pa.PA_ERR_INVALID


def test_prefill_validation():
    lib = pa.load()
    args = [P, P, pa.PA_BF16, 512, 64, 128, P, 1, 512, P, P, pa.PA_FP8_E4M3, 100, 32, 8, P, 64, P,
            0.1, 1.0, 1.0, None]
    bad = list(args)
    bad[4] = 60  # 60 % 8 != 0
    assert lib.pa_prefill_chunk(*bad) == pa.PA_ERR_INVALID
    bad = list(args)
    bad[5] = 96
    assert lib.pa_prefill_chunk(*bad) == pa.PA_ERR_UNSUPPORTED
    bad = list(args)
    bad[1] = ctypes.c_void_p(8)  # misaligned query
    assert lib.pa_prefill_chunk(*bad) == pa.PA_ERR_INVALID
    bad = list(args)
    bad[7] = 70000  # chunks on a grid axis of at most 65535
    assert lib.pa_prefill_chunk(*bad) == pa.PA_ERR_INVALID


def _shared(**kw):
    a = dict(out=P, query=P, q_dtype=pa.PA_BF16, num_seqs=4, num_heads=32, head_size=128,
             k_cache=P, v_cache=P, cache_dtype=pa.PA_BF16, num_blocks=100, block_size=16,
             num_kv_heads=8, block_tables=P, max_blocks_per_seq=8, seq_lens=P, max_seq_len=128,
             prefix_len=64, scale=0.1, k_scale=1.0, v_scale=1.0, flags=0, workspace=None,
             workspace_bytes=0, stream=None)
    a.update(kw)
    return pa.load().pa_decode_shared_prefix(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(prefix_len=40), pa.PA_ERR_INVALID),          # not whole blocks
    (dict(prefix_len=144), pa.PA_ERR_INVALID),         # past max_seq_len
    (dict(prefix_len=-16), pa.PA_ERR_INVALID),
    (dict(head_size=64), pa.PA_ERR_UNSUPPORTED),        # the prefix product takes head size 128
    (dict(q_dtype=pa.PA_F32, cache_dtype=pa.PA_F32), pa.PA_ERR_UNSUPPORTED),
    (dict(num_seqs=70000), pa.PA_ERR_WORKSPACE),       # any number of sequences
    (dict(), pa.PA_ERR_WORKSPACE),
    (dict(workspace=P, workspace_bytes=1000), pa.PA_ERR_WORKSPACE),
])
def test_shared_prefix_rejects_bad_host_arguments(kw, code):
    assert _shared(**kw) == code
    assert pa.load().pa_last_error()


def test_shared_prefix_checks_decode_arguments_before_any_launch():
    # With a large enough (never touched) workspace, the decode checks still
    # run before the prefix product is enqueued: contradictory flags fail.
    need = pa.pa_decode_shared_prefix_workspace_size(4, 32, 8, 128, 64)
    assert need > pa.pa_decode_workspace_size(4, 32, 8, 128, 128, pa.PA_PARTITION_BALANCED)
    rc = _shared(workspace=P, workspace_bytes=need,
                 flags=pa.PA_DECODE_READ_ONCE | pa.PA_DECODE_SHARED)
    assert rc == pa.PA_ERR_INVALID
    assert _shared(workspace=P, workspace_bytes=need, out=None) == pa.PA_ERR_INVALID
    assert _shared(num_seqs=0) == pa.PA_OK
