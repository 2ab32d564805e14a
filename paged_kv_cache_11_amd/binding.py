"""ctypes binding of ``libpa.so`` (the C ABI in include/pa.h).

Argument marshalling only: each function takes torch tensors that already
live on the GPU, reads their data pointers and shapes, and calls the C entry
point of the same name on the current HIP stream.  Every step of the path
runs in the library's kernels; there is no fallback.  If the library is not
built, loading it raises ``PagedAttentionError``.

Tensor conventions (all contiguous, on the same device):
  K/V pools      [num_blocks, num_kv_heads, block_size, head_size];
                 float32, bfloat16, or uint8 / float8_e4m3fn for fp8 E4M3FN
  queries, out   [num_tokens, num_heads, head_size]
  block_tables   int32 [num_seqs, max_blocks_per_seq]
  seq_lens       int32 [num_seqs]
  slot_mapping   int64 [num_tokens]
  block_mapping  int64 [num_pairs, 2]
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_PARTITION_BALANCED = -1
# pa_decode flags (include/pa.h)
PA_DECODE_READ_ONCE, PA_DECODE_SHARED = 0x1, 0x2
PA_DECODE_ENGINE_VALU, PA_DECODE_ENGINE_MFMA = 0x4, 0x8
PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = 0, -1, -2, -3, -4
PA_ERR_NO_BLOCKS = -5

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

_c_int, _c_f, _c_p, _c_sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGNATURES = {
    "pa_version": ([], _c_int),
    "pa_strerror": ([_c_int], ctypes.c_char_p),
    "pa_last_error": ([], ctypes.c_char_p),
    "pa_pool_bytes": ([_c_int, _c_int, _c_int, _c_int, _c_int], _c_sz),
    "pa_cache_write": ([_c_p, _c_p, _c_int, _c_int, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int,
                        _c_int, _c_p, _c_f, _c_f, _c_p], _c_int),
    "pa_copy_blocks": ([_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p],
                       _c_int),
    "pa_swap_blocks": ([_c_p, _c_p, _c_int, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                        _c_p, _c_int, _c_p], _c_int),
    "pa_decode_workspace_size": ([_c_int, _c_int, _c_int, _c_int, _c_int, _c_int], _c_sz),
    "pa_decode": ([_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_p, _c_int, _c_int, _c_int,
                   _c_int, _c_p, _c_int, _c_p, _c_int, _c_f, _c_f, _c_f, _c_int, _c_int, _c_p,
                   _c_sz, _c_p], _c_int),
    "pa_decode_append": ([_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_p, _c_p, _c_p,
                          _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p, _c_int, _c_f, _c_f,
                          _c_f, _c_int, _c_p, _c_sz, _c_p], _c_int),
    "pa_prefill_chunk": ([_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_int, _c_p,
                          _c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p, _c_f, _c_f,
                          _c_f, _c_p], _c_int),
    "pa_decode_no_alloc": ([_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_p, _c_int, _c_int,
                            _c_int, _c_int, _c_p, _c_int, _c_p, _c_int, _c_f, _c_f, _c_f, _c_int,
                            _c_int, _c_p], _c_int),
    "pa_decode_shared_prefix_workspace_size": ([_c_int, _c_int, _c_int, _c_int, _c_int], _c_sz),
    "pa_decode_shared_prefix": ([_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_p, _c_p, _c_int,
                                 _c_int, _c_int, _c_int, _c_p, _c_int, _c_p, _c_int, _c_int, _c_f,
                                 _c_f, _c_f, _c_int, _c_p, _c_sz, _c_p], _c_int),
    "pa_profile_next_decode": ([_c_p, _c_p], _c_int),
    # host-side validation of the data arrays (host pointers)
    "pa_validate_decode": ([_c_p, _c_int, _c_int, _c_p, _c_int, _c_int, _c_int, _c_p], _c_int),
    "pa_validate_prefill": ([_c_p, _c_int, _c_int, _c_int, _c_p, _c_int, _c_p, _c_int, _c_int,
                             _c_p], _c_int),
    "pa_validate_slots": ([_c_p, _c_int, _c_int, _c_int, _c_p], _c_int),
    "pa_validate_block_pairs": ([_c_p, _c_int, _c_int, _c_int, _c_int, _c_p], _c_int),
    "pa_validate_shared_prefix": ([_c_p, _c_int, _c_int, _c_p, _c_int, _c_int, _c_int, _c_p],
                                  _c_int),
    # host block manager
    "pa_bm_create": ([_c_int, _c_int], _c_p),
    "pa_bm_destroy": ([_c_p], None),
    "pa_bm_num_free": ([_c_p], _c_int),
    "pa_bm_add": ([_c_p, ctypes.c_int64, _c_int, _c_p], _c_int),
    "pa_bm_append": ([_c_p, _c_int, _c_p, _c_p, _c_p, _c_p], _c_int),
    "pa_bm_fork": ([_c_p, ctypes.c_int64, ctypes.c_int64], _c_int),
    "pa_bm_free": ([_c_p, ctypes.c_int64], _c_int),
    "pa_bm_seq_len": ([_c_p, ctypes.c_int64], _c_int),
    "pa_bm_block_tables": ([_c_p, _c_int, _c_p, _c_int, _c_p, _c_p], _c_int),
    "pa_bm_ref_count": ([_c_p, _c_int], _c_int),
    "pa_bm_create_swap": ([_c_int, _c_int, _c_int], _c_p),
    "pa_bm_swap_out": ([_c_p, _c_int, _c_p, _c_p, _c_int, _c_p], _c_int),
    "pa_bm_swap_in": ([_c_p, _c_int, _c_p, _c_p, _c_int, _c_p], _c_int),
    "pa_bm_num_free_host": ([_c_p], _c_int),
    "pa_bm_is_swapped": ([_c_p, ctypes.c_int64], _c_int),
    "pa_bm_block_hash": ([ctypes.c_uint64, _c_p, _c_int, ctypes.c_uint64], ctypes.c_uint64),
    "pa_bm_enable_prefix_caching": ([_c_p], _c_int),
    "pa_bm_add_prompt": ([_c_p, ctypes.c_int64, _c_p, _c_int, ctypes.c_uint64, _c_p, _c_p], _c_int),
    "pa_bm_append_tokens": ([_c_p, _c_int, _c_p, _c_p, _c_p, _c_p, _c_p], _c_int),
    "pa_bm_num_cached_blocks": ([_c_p], _c_int),
}


class PagedAttentionError(RuntimeError):
    """A library call returned an error code (message from pa_last_error)."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} [{code}]")
        self.code = code


_lib = None


def load(path: Optional[str] = None):
    """Load the HIP library (once) and declare its C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise PagedAttentionError(PA_ERR_HIP, f"HIP library not built: {p} is missing "
                                  "(run __graft_entry__.build() or paged_kv_cache_11_amd/build.py)")
    lib = ctypes.CDLL(p)
    for name, (args, res) in _SIGNATURES.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, res
    if path is None:
        _lib = lib
    return lib


def exported_symbols():
    return sorted(_SIGNATURES)


def _check(code: int):
    if code != PA_OK:
        raise PagedAttentionError(code, load().pa_last_error().decode() or
                                  load().pa_strerror(code).decode())


def dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_FP8_E4M3
    raise PagedAttentionError(PA_ERR_UNSUPPORTED, f"no pa dtype for {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise PagedAttentionError(PA_ERR_INVALID, "tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _pool_dims(k_cache, v_cache):
    if k_cache.dim() != 4 or tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.dtype != v_cache.dtype:
        raise PagedAttentionError(PA_ERR_INVALID, "k_cache and v_cache must be equal 4-D pools "
                                  "[num_blocks, num_kv_heads, block_size, head_size]")
    nb, hkv, bs, d = (int(x) for x in k_cache.shape)
    return nb, hkv, bs, d


def pa_version() -> int:
    return int(load().pa_version())


def pa_pool_bytes(num_blocks, num_kv_heads, block_size, head_size, cache_dtype) -> int:
    return int(load().pa_pool_bytes(num_blocks, num_kv_heads, block_size, head_size, cache_dtype))


def pa_cache_write(key, value, k_cache, v_cache, slot_mapping, k_scale: float = 1.0,
                   v_scale: float = 1.0, stream=None) -> None:
    """Write key/value [num_tokens, num_kv_heads, head_size] into their slots."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    if _validating():
        validate_slots(slot_mapping, nb, bs)
    _check(load().pa_cache_write(_ptr(key), _ptr(value), dtype_code(key), int(key.shape[0]),
                                 _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), nb, bs, hkv, d,
                                 _ptr(slot_mapping), float(k_scale), float(v_scale), _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> None:
    """Copy whole physical blocks (src, dst) in both pools."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    n = int(block_mapping.shape[0]) if block_mapping is not None else 0
    if _validating() and n:
        validate_block_pairs(block_mapping, nb, nb, True)
    _check(load().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), nb, bs, hkv, d,
                                 _ptr(block_mapping) if n else None, n, _stream(stream)))


def block_hash(parent_hash: int, tokens, extra_hash: int = 0) -> int:
    """The library's chained hash of one full block of token ids."""
    import numpy as np

    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    return int(load().pa_bm_block_hash(int(parent_hash) & (2 ** 64 - 1), toks.ctypes.data,
                                       toks.size, int(extra_hash) & (2 ** 64 - 1)))


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, block_mapping, stream=None) -> None:
    """Move whole blocks (src, dst) from the source pools into the
    destination pools; one side is usually pinned host memory (a tensor made
    with pin_memory=True), the other the device pool.  block_mapping lives
    in device or pinned host memory."""
    snb, hkv, bs, d = _pool_dims(src_k, src_v)
    dnb, dhkv, dbs, dd = _pool_dims(dst_k, dst_v)
    if (hkv, bs, d) != (dhkv, dbs, dd) or src_k.dtype != dst_k.dtype:
        raise PagedAttentionError(PA_ERR_INVALID, "source and destination pools differ in geometry")
    n = int(block_mapping.shape[0]) if block_mapping is not None else 0
    _check(load().pa_swap_blocks(_ptr(src_k), _ptr(src_v), snb, _ptr(dst_k), _ptr(dst_v), dnb,
                                 dtype_code(src_k), bs, hkv, d,
                                 _ptr(block_mapping) if n else None, n, _stream(stream)))


def pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len,
                             partition_size) -> int:
    return int(load().pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_size,
                                               max_seq_len, partition_size))


def pa_decode(out, query, k_cache, v_cache, block_tables, seq_lens, max_seq_len: int,
              scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
              partition_size: int = 0, workspace=None, stream=None, flags: int = 0) -> None:
    """Decode attention of query [num_seqs, num_heads, head_size] into out.

    partition_size: 0 (no split), a multiple of the block size (fixed
    partitions), or PA_PARTITION_BALANCED (equal block runs per wavefront).
    flags: PA_DECODE_READ_ONCE / PA_DECODE_SHARED (how blocks are shared)
    and PA_DECODE_ENGINE_VALU / _MFMA (engine pin), as in include/pa.h.

    With ``workspace=None`` and a split that needs one, a workspace tensor
    is taken from torch's allocator."""
    import torch

    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    S, H = int(query.shape[0]), int(query.shape[1])
    if _validating():
        validate_decode(block_tables, seq_lens, max_seq_len, nb, bs)
    need = pa_decode_workspace_size(S, H, hkv, d, max_seq_len, partition_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pa_decode(_ptr(out), _ptr(query), dtype_code(query), S, H, d, _ptr(k_cache),
                            _ptr(v_cache), dtype_code(k_cache), nb, bs, hkv, _ptr(block_tables),
                            int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len),
                            float(scale), float(k_scale), float(v_scale), int(partition_size),
                            int(flags), _ptr(workspace), ws_bytes, _stream(stream)))


def pa_decode_append(out, query, k_new, v_new, k_cache, v_cache, block_tables, seq_lens,
                     max_seq_len: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                     workspace=None, stream=None, flags: int = 0) -> None:
    """One decode step in one call: each sequence's newest token (position
    seq_len - 1), given as bf16 rows k_new / v_new [num_seqs, num_kv_heads,
    head_size], is written into the slot its block table gives and attended
    to with the rest (the balanced split, as pa_decode).  The same pool and
    output as pa_cache_write with those slots followed by pa_decode."""
    import torch

    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    S, H = int(query.shape[0]), int(query.shape[1])
    if _validating():
        validate_decode(block_tables, seq_lens, max_seq_len, nb, bs)
    need = pa_decode_workspace_size(S, H, hkv, d, max_seq_len, PA_PARTITION_BALANCED)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pa_decode_append(_ptr(out), _ptr(query), dtype_code(query), S, H, d,
                                   _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                   dtype_code(k_cache), nb, bs, hkv, _ptr(block_tables),
                                   int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len),
                                   float(scale), float(k_scale), float(v_scale), int(flags),
                                   _ptr(workspace), ws_bytes, _stream(stream)))


def pa_decode_no_alloc(out, query, k_cache, v_cache, block_tables, seq_lens, max_seq_len: int,
                       scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                       partition_size: int = 0, stream=None, flags: int = 0) -> None:
    """pa_decode whose split-K partials live in the library's static
    per-device scratch (no workspace, no allocation); calls on one GPU must
    not overlap."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    S, H = int(query.shape[0]), int(query.shape[1])
    if _validating():
        validate_decode(block_tables, seq_lens, max_seq_len, nb, bs)
    _check(load().pa_decode_no_alloc(_ptr(out), _ptr(query), dtype_code(query), S, H, d,
                                     _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), nb, bs,
                                     hkv, _ptr(block_tables), int(block_tables.shape[1]),
                                     _ptr(seq_lens), int(max_seq_len), float(scale),
                                     float(k_scale), float(v_scale), int(partition_size),
                                     int(flags), _stream(stream)))


def pa_decode_shared_prefix_workspace_size(num_seqs, num_heads, num_kv_heads, head_size,
                                           prefix_len) -> int:
    return int(load().pa_decode_shared_prefix_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                             head_size, prefix_len))


def pa_decode_shared_prefix(out, query, k_cache, v_cache, block_tables, seq_lens,
                            max_seq_len: int, prefix_len: int, scale: float, k_scale: float = 1.0,
                            v_scale: float = 1.0, workspace=None, stream=None,
                            flags: int = PA_DECODE_READ_ONCE) -> None:
    """pa_decode for sequences that share their first prefix_len tokens
    (the same blocks, read from table row 0): the prefix attention once per
    KV head for all sequences on the matrix cores, the suffixes through the
    balanced split, a log-sum-exp merge of the two."""
    import torch

    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    S, H = int(query.shape[0]), int(query.shape[1])
    if _validating():
        validate_decode(block_tables, seq_lens, max_seq_len, nb, bs)
        validate_shared_prefix(block_tables, seq_lens, prefix_len, nb, bs)
    need = pa_decode_shared_prefix_workspace_size(S, H, hkv, d, prefix_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pa_decode_shared_prefix(
        _ptr(out), _ptr(query), dtype_code(query), S, H, d, _ptr(k_cache), _ptr(v_cache),
        dtype_code(k_cache), nb, bs, hkv, _ptr(block_tables), int(block_tables.shape[1]),
        _ptr(seq_lens), int(max_seq_len), int(prefix_len), float(scale), float(k_scale),
        float(v_scale), int(flags), _ptr(workspace), ws_bytes, _stream(stream)))


def pa_profile_next_decode(start_event, stop_event) -> None:
    """Record these torch.cuda.Event objects (timing enabled, already
    created by one record()) around the main kernel of the next decode call
    on this thread; None, None cancels."""
    h = [ctypes.c_void_p(e.cuda_event) if e is not None else None
         for e in (start_event, stop_event)]
    _check(load().pa_profile_next_decode(*h))


# --- host-side validation ---------------------------------------------------
# PA_VALIDATE=1 in the environment makes every device call of this binding
# copy its index arrays to the host and check them first (a debug mode: it
# synchronises).  The validate_* functions can also be called directly on
# numpy arrays or tensors.

def _validating() -> bool:
    return os.environ.get("PA_VALIDATE", "0") not in ("", "0")


def _host(a, dtype):
    import numpy as np

    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _validated(code):
    if code != PA_OK:
        raise PagedAttentionError(code, load().pa_last_error().decode())


def validate_decode(block_tables, seq_lens, max_seq_len: int, num_blocks: int,
                    block_size: int) -> None:
    """Raise PagedAttentionError naming the first table entry or length a
    pa_decode call with these arrays would read out of bounds."""
    import numpy as np

    t = _host(block_tables, np.int32)
    ln = _host(seq_lens, np.int32).reshape(-1)
    if t.ndim != 2 or t.shape[0] != ln.size:
        raise PagedAttentionError(PA_ERR_INVALID, "block_tables must be [num_seqs, max_blocks]")
    _validated(load().pa_validate_decode(t.ctypes.data, ln.size, t.shape[1], ln.ctypes.data,
                                         int(max_seq_len), int(num_blocks), int(block_size), None))


def validate_prefill(query_start_loc, num_tokens: int, max_query_len: int, block_tables,
                     seq_lens, num_blocks: int, block_size: int) -> None:
    import numpy as np

    q = _host(query_start_loc, np.int32).reshape(-1)
    t = _host(block_tables, np.int32)
    ln = _host(seq_lens, np.int32).reshape(-1)
    if q.size != ln.size + 1 or t.ndim != 2 or t.shape[0] != ln.size:
        raise PagedAttentionError(PA_ERR_INVALID, "query_start_loc / block_tables / seq_lens "
                                  "disagree on the number of chunks")
    _validated(load().pa_validate_prefill(q.ctypes.data, ln.size, int(num_tokens),
                                          int(max_query_len), t.ctypes.data, t.shape[1],
                                          ln.ctypes.data, int(num_blocks), int(block_size), None))


def validate_slots(slot_mapping, num_blocks: int, block_size: int) -> None:
    import numpy as np

    s = _host(slot_mapping, np.int64).reshape(-1)
    _validated(load().pa_validate_slots(s.ctypes.data, s.size, int(num_blocks), int(block_size),
                                        None))


def validate_shared_prefix(block_tables, seq_lens, prefix_len: int, num_blocks: int,
                           block_size: int) -> None:
    import numpy as np

    t = _host(block_tables, np.int32)
    ln = _host(seq_lens, np.int32).reshape(-1)
    _validated(load().pa_validate_shared_prefix(t.ctypes.data, ln.size, t.shape[1],
                                                ln.ctypes.data, int(prefix_len), int(num_blocks),
                                                int(block_size), None))


def validate_block_pairs(block_mapping, src_num_blocks: int, dst_num_blocks: int,
                         same_pool: bool) -> None:
    import numpy as np

    m = _host(block_mapping, np.int64).reshape(-1, 2)
    _validated(load().pa_validate_block_pairs(m.ctypes.data, m.shape[0], int(src_num_blocks),
                                              int(dst_num_blocks), int(bool(same_pool)), None))


def pa_prefill_chunk(out, query, query_start_loc, max_query_len: int, k_cache, v_cache,
                     block_tables, seq_lens, scale: float, k_scale: float = 1.0,
                     v_scale: float = 1.0, stream=None) -> None:
    """Causal attention of chunk queries [num_tokens, num_heads, head_size]."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    T, H = int(query.shape[0]), int(query.shape[1])
    if _validating():
        validate_prefill(query_start_loc, T, max_query_len, block_tables, seq_lens, nb, bs)
    _check(load().pa_prefill_chunk(_ptr(out), _ptr(query), dtype_code(query), T, H, d,
                                   _ptr(query_start_loc), int(seq_lens.shape[0]),
                                   int(max_query_len), _ptr(k_cache), _ptr(v_cache),
                                   dtype_code(k_cache), nb, bs, hkv, _ptr(block_tables),
                                   int(block_tables.shape[1]), _ptr(seq_lens), float(scale),
                                   float(k_scale), float(v_scale), _stream(stream)))


class BlockManager:
    """The host block manager of the library (pa_bm_*): a first-in first-out
    free list of physical blocks, reference counts, and fork / append / free
    with copy-on-write.  Arrays are numpy host arrays; copy them to the
    device for pa_cache_write, pa_copy_blocks and pa_decode."""

    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0,
                 prefix_caching: bool = False):
        self._lib = load()
        self._h = self._lib.pa_bm_create_swap(int(num_blocks), int(num_host_blocks), int(block_size))
        if not self._h:
            raise PagedAttentionError(PA_ERR_INVALID, self._lib.pa_last_error().decode())
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.num_host_blocks = int(num_host_blocks)
        if prefix_caching:
            _check(self._lib.pa_bm_enable_prefix_caching(self._h))

    def add_prompt(self, seq_id: int, tokens, extra_hash: int = 0):
        """A new sequence from its prompt token ids, reusing cached blocks;
        returns (slots int64 [n], num_cached: leading tokens already in the pool)."""
        import numpy as np

        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        slots = np.empty(max(toks.size, 1), dtype=np.int64)
        nc = ctypes.c_int32(0)
        _check(self._lib.pa_bm_add_prompt(self._h, int(seq_id), toks.ctypes.data, toks.size,
                                          int(extra_hash) & (2 ** 64 - 1), slots.ctypes.data,
                                          ctypes.byref(nc)))
        return slots[:toks.size], int(nc.value)

    def append_tokens(self, seq_ids, tokens):
        """``append`` with each sequence's new token id (full blocks enter the cache)."""
        import numpy as np

        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        if toks.size != ids.size:
            raise PagedAttentionError(PA_ERR_INVALID, "one token per listed sequence")
        n = ids.size
        slots = np.empty(max(n, 1), dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int64)
        nc = ctypes.c_int32(0)
        _check(self._lib.pa_bm_append_tokens(self._h, n, ids.ctypes.data, toks.ctypes.data,
                                             slots.ctypes.data, pairs.ctypes.data, ctypes.byref(nc)))
        return slots[:n], pairs[:nc.value]

    def num_cached_blocks(self) -> int:
        return int(self._lib.pa_bm_num_cached_blocks(self._h))

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.pa_bm_destroy(h)

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def add(self, seq_id: int, num_tokens: int):
        """A new sequence of num_tokens tokens; returns their slots (int64)."""
        import numpy as np

        slots = np.empty(max(int(num_tokens), 1), dtype=np.int64)
        _check(self._lib.pa_bm_add(self._h, int(seq_id), int(num_tokens), slots.ctypes.data))
        return slots[:int(num_tokens)]

    def append(self, seq_ids):
        """One token for each id (in order); returns (slots int64 [n],
        copy-on-write pairs int64 [c, 2])."""
        import numpy as np

        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        n = ids.size
        slots = np.empty(max(n, 1), dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int64)
        nc = ctypes.c_int32(0)
        _check(self._lib.pa_bm_append(self._h, n, ids.ctypes.data, slots.ctypes.data,
                                      pairs.ctypes.data, ctypes.byref(nc)))
        return slots[:n], pairs[:nc.value]

    def _swap(self, fn, seq_ids, max_pairs):
        import numpy as np

        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        cap = int(max_pairs) if max_pairs is not None else max(self.num_blocks, self.num_host_blocks)
        pairs = np.empty((max(cap, 1), 2), dtype=np.int64)
        n = ctypes.c_int32(0)
        _check(fn(self._h, ids.size, ids.ctypes.data, pairs.ctypes.data, cap, ctypes.byref(n)))
        return pairs[:n.value]

    def swap_out(self, seq_ids, max_pairs=None):
        """Move these sequences to host blocks; returns (device block, host
        block) pairs int64 [n, 2] for pa_swap_blocks."""
        return self._swap(self._lib.pa_bm_swap_out, seq_ids, max_pairs)

    def swap_in(self, seq_ids, max_pairs=None):
        """Move swapped-out sequences back; returns (host block, device block) pairs."""
        return self._swap(self._lib.pa_bm_swap_in, seq_ids, max_pairs)

    def num_free_host(self) -> int:
        return int(self._lib.pa_bm_num_free_host(self._h))

    def is_swapped(self, seq_id: int) -> bool:
        r = int(self._lib.pa_bm_is_swapped(self._h, int(seq_id)))
        if r < 0:
            _check(r)
        return bool(r)

    def fork(self, parent_id: int, child_id: int) -> None:
        _check(self._lib.pa_bm_fork(self._h, int(parent_id), int(child_id)))

    def release(self, seq_id: int) -> None:
        _check(self._lib.pa_bm_free(self._h, int(seq_id)))

    def seq_len(self, seq_id: int) -> int:
        r = int(self._lib.pa_bm_seq_len(self._h, int(seq_id)))
        if r < 0:
            _check(r)
        return r

    def ref_count(self, block: int) -> int:
        r = int(self._lib.pa_bm_ref_count(self._h, int(block)))
        if r < 0:
            _check(r)
        return r

    def block_tables(self, seq_ids, max_blocks_per_seq: int):
        """(int32 [n, max_blocks_per_seq] tables padded with -1, int32 [n] lengths)."""
        import numpy as np

        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        n = ids.size
        tables = np.empty((max(n, 1), max(int(max_blocks_per_seq), 1)), dtype=np.int32)
        lens = np.empty(max(n, 1), dtype=np.int32)
        _check(self._lib.pa_bm_block_tables(self._h, n, ids.ctypes.data, int(max_blocks_per_seq),
                                            tables.ctypes.data, lens.ctypes.data))
        return tables[:n, :int(max_blocks_per_seq)], lens[:n]
