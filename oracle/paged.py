"""Paged K/V cache semantics and attention, in float64 — the oracle.

Sources (the pages, by title and section):
  [LIB]  "vLLM：大语言模型推理与服务库", §4 "vLLM核心——PagedAttention":
         §4.2 item 1 (physical block of a fixed number of tokens), item 2
         (per-sequence block table, logical -> physical block id, worked
         example of a 50-token sequence at block size 16 in 4 blocks),
         §4.3 (a new token's K/V is written into the last block, a new block
         is taken when it is full), §4.4 item 3 (for each query: walk the
         sequence's physical blocks, score q·k, softmax, weight V).
  [EVAL] "vLLM 高性能大语言模型推理引擎深度技术评估与分布式架构展望":
         "逻辑块到物理块的映射转换" step 4 (the kernel gathers K/V through
         the block table in place, with no copy into a contiguous tensor);
         "束搜索与并行采样的三大调度原语" (fork shares blocks; append copies
         only the block that changes; free drops reference counts);
         "分块预填充克服队头阻塞" (a long prompt is processed in chunks).
  [DEEP] "vLLM 深度解析：从 PagedAttention 到生产部署", §3.1 (block table
         figure for two interleaved requests; prefix sharing and
         copy-on-write).
  [ESSAY] the openeuler.csdn.net vLLM essay, section
         "PagedAttention：把操作系统的分页搬上 GPU" (kernel grid over heads,
         sequences and partitions).

The formula the pages print for the block-level computation did not survive
text extraction; paging is an addressing scheme and changes no arithmetic, so
the oracle is plain softmax(q·Kᵀ·scale)·V over the gathered tokens.

Pool layout (the library's documented contract, restated here independently):
each of the K pool and the V pool is an array
``[num_blocks, num_kv_heads, block_size, head_size]`` of storage words, head
dimension fastest.  Slot ``b * block_size + o`` is offset ``o`` of block
``b``.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from . import codecs


# ----------------------------------------------------------------------------
# addressing
# ----------------------------------------------------------------------------
def slots_of(table_row, length: int, block_size: int) -> np.ndarray:
    """Slot of each token 0..length-1 of a sequence: the physical block of its
    logical block (t // block_size) times block_size plus its offset in the
    block ([LIB] §4.2 item 2)."""
    t = np.arange(length, dtype=np.int64)
    blocks = np.asarray(table_row, dtype=np.int64)[t // block_size]
    if length and (blocks < 0).any():
        raise ValueError("block table entry < 0 inside the sequence")
    return blocks * block_size + t % block_size


def gather(pool, table_row, length: int):
    """K (or V) of one sequence as a contiguous ``[length, num_kv_heads, D]``
    array, read token by token through the block table ([EVAL] step 4).
    Only logical blocks 0..ceil(length / block_size)-1 are touched."""
    pool = np.asarray(pool)
    bs = pool.shape[2]
    out = np.empty((length, pool.shape[1], pool.shape[3]), dtype=pool.dtype)
    for t in range(length):
        b = int(table_row[t // bs])
        if b < 0 or b >= pool.shape[0]:
            raise ValueError(f"token {t}: block id {b} outside the pool")
        out[t] = pool[b, :, t % bs, :]
    return out


def pool_values(raw_pool, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Raw pool words -> float64 values (fp8 scaled by its per-tensor scale)."""
    return codecs.decode(raw_pool, dtype, scale)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def _kv_head(h: int, num_heads: int, num_kv_heads: int) -> int:
    """Query head h reads KV head h // (Hq / Hkv): contiguous GQA groups."""
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return h // (num_heads // num_kv_heads)


def attend(q, K, V, scale: float, visible=None):
    """softmax(scale · K·q) · V for one query vector, float64.

    q: [D]; K, V: [L, D]; ``visible``: optional boolean mask [L] of keys the
    query may see.  With no visible key the result is the zero vector."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if visible is not None:
        K = K[visible]
        V = V[visible]
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = (K @ q) * float(np.float32(scale))
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def _seq_kv(k_pool, v_pool, table_row, L, kv_dtype, k_scale, v_scale):
    """Gathered K and V of one sequence as float64 [L, Hkv, D].  With
    ``kv_dtype`` the pools hold raw storage words, decoded after the gather."""
    K = gather(k_pool, table_row, L)
    V = gather(v_pool, table_row, L)
    if kv_dtype is not None:
        K = pool_values(K, kv_dtype, k_scale)
        V = pool_values(V, kv_dtype, v_scale)
    return K, V


def paged_decode(q, k_pool, v_pool, block_tables, seq_lens, scale: float, kv_dtype=None,
                 k_scale: float = 1.0, v_scale: float = 1.0, seqs=None):
    """One query token per sequence against its whole paged context.

    q: [S, Hq, D]; k_pool, v_pool: pools ``[num_blocks, Hkv, block_size, D]``
    of float64 values, or of raw storage words of ``kv_dtype`` (fp8 scaled by
    k_scale / v_scale); block_tables: [S, MB]; seq_lens: [S] (the context
    includes the token just written).  ``seqs`` restricts the work to some
    sequences (other rows stay zero).  Returns float64 [S, Hq, D]."""
    q = np.asarray(q, dtype=np.float64)
    S, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(seq_lens[s])
        K, V = _seq_kv(k_pool, v_pool, block_tables[s], L, kv_dtype, k_scale, v_scale)
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            out[s, h] = attend(q[s, h], K[:, g, :], V[:, g, :], scale)
    return out


def paged_prefill(q, query_start, k_pool, v_pool, block_tables, seq_lens, scale: float,
                  kv_dtype=None, k_scale: float = 1.0, v_scale: float = 1.0, rows=None):
    """Causal attention for chunks of queries appended to paged sequences.

    Chunk c owns query rows query_start[c]:query_start[c+1]; it has
    n_c = query_start[c+1] - query_start[c] queries and seq_lens[c] keys in
    the cache, its own included.  Query i of the chunk sits at position
    seq_lens[c] - n_c + i and sees keys 0..that position.  Pools as in
    ``paged_decode``; ``rows`` restricts the work to some query rows."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.zeros((T, Hq, D), dtype=np.float64)
    want = None if rows is None else set(int(r) for r in rows)
    for c in range(len(seq_lens)):
        a, b = int(query_start[c]), int(query_start[c + 1])
        L = int(seq_lens[c])
        n = b - a
        if n > L:
            raise ValueError("a chunk cannot hold more queries than keys")
        if want is not None and not any(a <= r < b for r in want):
            continue
        K, V = _seq_kv(k_pool, v_pool, block_tables[c], L, kv_dtype, k_scale, v_scale)
        keys = np.arange(L)
        for i in range(n):
            if want is not None and a + i not in want:
                continue
            pos = L - n + i
            for h in range(Hq):
                g = _kv_head(h, Hq, Hkv)
                out[a + i, h] = attend(q[a + i, h], K[:, g, :], V[:, g, :], scale,
                                       visible=keys <= pos)
    return out


# ----------------------------------------------------------------------------
# split-K partitions and their merge
# ----------------------------------------------------------------------------
def partition_state(q, K, V, scale: float):
    """Softmax state of one query over one partition of keys:
    m = max score, l = sum exp(score - m), o = sum exp(score - m)·v / l."""
    s = (np.asarray(K, np.float64) @ np.asarray(q, np.float64)) * float(np.float32(scale))
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return m, l, (p @ np.asarray(V, np.float64)) / l


def lse_merge(states):
    """Combine partition states (m_p, l_p, o_p) into the full softmax output:
    weights w_p = exp(m_p - max m) · l_p, result sum w_p o_p / sum w_p.
    This is the exact identity softmax over a union of key sets satisfies."""
    M = max(m for m, _, _ in states)
    w = np.array([np.exp(m - M) * l for m, l, _ in states])
    o = np.stack([o for _, _, o in states])
    return (w[:, None] * o).sum(0) / w.sum()


def split_attend(q, K, V, scale: float, partition_size: int):
    """Attention of one query computed partition by partition and merged."""
    L = K.shape[0]
    states = [partition_state(q, K[a:a + partition_size], V[a:a + partition_size], scale)
              for a in range(0, L, partition_size)]
    return lse_merge(states)


# ----------------------------------------------------------------------------
# cache write and block copy
# ----------------------------------------------------------------------------
def cache_write(k_pool, v_pool, pool_dtype: str, k_src, v_src, src_dtype: str,
                slot_mapping, k_scale: float = 1.0, v_scale: float = 1.0):
    """Write each token's K and V rows into its slot ([LIB] §4.3: the new
    token's K/V goes into the sequence's current block).

    k_pool, v_pool: raw pools [num_blocks, Hkv, block_size, D] (updated in
    place and returned).  k_src, v_src: raw source words [T, Hkv, D] in
    ``src_dtype``.  A negative slot is a padding token and is skipped; two
    tokens may not share a slot.
    Matching dtypes copy bits; an fp8 pool quantises the float32 value of the
    source by its per-tensor scale (``codecs.quantize_e4m3fn``)."""
    nb, Hkv, bs, D = k_pool.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = np.nonzero(slots >= 0)[0]
    if len(np.unique(slots[live])) != len(live):
        raise ValueError("two tokens map to the same slot")
    b, off = slots[live] // bs, slots[live] % bs
    if live.size and b.max() >= nb:
        raise ValueError("a slot is past the pool's last block")
    for pool, src, sc in ((k_pool, k_src, k_scale), (v_pool, v_src, v_scale)):
        rows = np.asarray(src)[live]                      # [n, Hkv, D]
        if pool_dtype == src_dtype:
            words = rows
        elif pool_dtype == "fp8":
            x32 = codecs.decode(rows, src_dtype).astype(np.float32)
            words = codecs.quantize_e4m3fn(x32, sc)
        else:
            raise ValueError(f"no cache write from {src_dtype} into {pool_dtype}")
        pool[b, :, off, :] = words
    return k_pool, v_pool


def copy_blocks(k_pool, v_pool, pairs):
    """Copy-on-write block copy ([EVAL] fork/append/free primitives; [DEEP]
    §3.1 copy-on-write): for each (src, dst) pair, every K and V word of
    physical block src is copied into block dst.  Sources are read before
    any destination is written; a destination must not repeat and must not
    be the source of another pair."""
    pairs = _pairs_inside(pairs, k_pool.shape[0], k_pool.shape[0])
    srcs, dsts = pairs[:, 0], pairs[:, 1]
    if len(set(dsts.tolist())) != len(dsts) or set(dsts.tolist()) & set(srcs.tolist()):
        raise ValueError("destinations must be distinct and disjoint from sources")
    for pool in (k_pool, v_pool):
        snap = pool[srcs].copy()
        pool[dsts] = snap
    return k_pool, v_pool


def _pairs_inside(pairs, src_blocks: int, dst_blocks: int) -> np.ndarray:
    """The (src, dst) pairs whose blocks both exist; a pair naming a block
    outside its pool moves nothing (the pages say nothing of such a pair)."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    ok = ((pairs[:, 0] >= 0) & (pairs[:, 0] < src_blocks) &
          (pairs[:, 1] >= 0) & (pairs[:, 1] < dst_blocks))
    return pairs[ok]


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs):
    """SWAP preemption ([EVAL], its section on preemption; [DEEP] §3.2,
    preemption strategies): the K/V blocks of a preempted sequence move from
    the device pool to a pool in host memory, and back when it resumes.  For
    each (src, dst) pair every K and V word of block src of the source pools
    is copied into block dst of the destination pools, which have the same
    geometry and may hold any number of blocks.  Destinations must be
    distinct."""
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools differ in geometry")
    pairs = _pairs_inside(pairs, src_k.shape[0], dst_k.shape[0])
    if len(set(pairs[:, 1].tolist())) != len(pairs):
        raise ValueError("destinations must be distinct")
    for src, dst in ((src_k, dst_k), (src_v, dst_v)):
        for s, d in pairs:
            dst[d] = src[s]
    return dst_k, dst_v
