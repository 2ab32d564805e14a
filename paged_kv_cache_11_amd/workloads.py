"""Seeded synthetic workloads for the paged K/V cache path.

This module only draws numbers and lays out inputs: sequence lengths, block
allocation (block tables and slot mappings), and the N(0,1) query/key/value
values. It holds none of the attention arithmetic; both the HIP path (through
the binding) and the CPU oracle consume what it produces.

Input format it follows (the paged layout described by the pages):
  * a physical block holds ``block_size`` consecutive tokens of one sequence
    ("vLLM：大语言模型推理与服务库", §4.2 item 1 "物理块");
  * ``block_tables[s, j]`` is the physical block id of logical block ``j`` of
    sequence ``s`` (same page, §4.2 item 2 "块表"); entries past the last used
    logical block are -1;
  * the slot of token ``t`` of sequence ``s`` is
    ``block_tables[s, t // block_size] * block_size + t % block_size``; a
    negative slot marks a padding token that is not written.

Draw order for every workload is fixed: sequence lengths, block permutation,
Q, K, V, then any workload-specific extras.  Values are drawn in float32 from
``numpy.random.default_rng(seed)``; storage casts (bf16) are done by the caller
with torch's round-to-nearest-even cast.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DTYPES = ("f32", "bf16", "fp8")
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}

# Pool filler for slots no sequence owns: a quiet NaN in every storage type.
# Any read of an unowned slot that leaks into an output shows up as NaN.
POISON_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0, "fp8": 0x7F}


@dataclasses.dataclass
class PagedBatch:
    """One synthetic batch over one K/V pool.

    Shapes (T = number of cached tokens written into the pool):
      q            float32 [S, Hq, D]   decode queries (one token per sequence)
      k, v         float32 [T, Hkv, D]  every cached token's key/value
      slot_mapping int64   [T]          pool slot of each cached token
      seq_lens     int32   [S]          tokens each sequence attends to
      block_tables int32   [S, MB]      physical block ids, -1 padded
    Optional chunked-prefill part (one or more chunks appended to sequences
    that live in the same pool):
      chunk_q            float32 [C, Hq, D]
      chunk_query_start  int32   [n+1]
      chunk_seq_lens     int32   [n]     keys each chunk sees (incl. itself)
      chunk_block_tables int32   [n, MBc]
    """

    name: str
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    q_dtype: str
    kv_src_dtype: str
    kv_dtype: str
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    slot_mapping: np.ndarray
    seq_lens: np.ndarray
    block_tables: np.ndarray
    k_scale: float = 1.0
    v_scale: float = 1.0
    partition_size: int = 0
    chunk_q: Optional[np.ndarray] = None
    chunk_query_start: Optional[np.ndarray] = None
    chunk_seq_lens: Optional[np.ndarray] = None
    chunk_block_tables: Optional[np.ndarray] = None
    copy_pairs: Optional[np.ndarray] = None
    notes: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    def kv_bytes_per_token(self) -> int:
        """Bytes of K plus V for one token over all KV heads, in the pool."""
        return 2 * self.num_kv_heads * self.head_size * ELEM_BYTES[self.kv_dtype]

    def decode_kv_bytes(self) -> int:
        """Algorithmic K/V bytes one decode call reads: sum of seq_lens x bytes/token."""
        return int(self.seq_lens.astype(np.int64).sum()) * self.kv_bytes_per_token()


def _tables_from_lengths(lengths, block_size, perm, start=0):
    """Hand out consecutive slices of ``perm`` as block tables."""
    nblk = [(int(L) + block_size - 1) // block_size for L in lengths]
    mb = max(nblk) if nblk else 0
    tables = np.full((len(lengths), max(mb, 1)), -1, dtype=np.int32)
    cur = start
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[cur:cur + n]
        cur += n
    return tables, cur


def _slots_for(table_row, length, block_size, first=0):
    t = np.arange(first, length, dtype=np.int64)
    return table_row[t // block_size].astype(np.int64) * block_size + t % block_size


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _pool_blocks(needed: int, factor: float = 1.25) -> int:
    return int(math.ceil(factor * needed))


def tiny_decode(seed: int = 1235) -> PagedBatch:
    """Tiny fp32 decode: 4 sequences of 1, 16, 17 and 50 tokens, block 16,
    8 query heads over 2 KV heads, head size 64, a 64-block pool whose tables
    are consecutive slices of a seeded permutation of all 64 block ids."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs, nb = 8, 2, 64, 16, 64
    seq_lens = np.array([1, 16, 17, 50], dtype=np.int32)
    perm = rng.permutation(nb).astype(np.int32)
    tables, _ = _tables_from_lengths(seq_lens, bs, perm)
    q = _normal(rng, (len(seq_lens), Hq, D))
    T = int(seq_lens.sum())
    k = _normal(rng, (T, Hkv, D))
    v = _normal(rng, (T, Hkv, D))
    slots = np.concatenate([_slots_for(tables[s], seq_lens[s], bs) for s in range(len(seq_lens))])
    return PagedBatch("tiny_fp32", Hq, Hkv, D, bs, nb, "f32", "f32", "f32",
                      1.0 / math.sqrt(D), q, k, v, slots, seq_lens, tables)


def _uniform_lengths(rng, num_seqs: int, min_len: int, max_len: int) -> np.ndarray:
    return rng.integers(min_len, max_len + 1, size=num_seqs, dtype=np.int64).astype(np.int32)


def llama3_8b_lengths(seed: int = 1236, num_seqs: int = 64, min_len: int = 512,
                      max_len: int = 4096) -> np.ndarray:
    """The context lengths of ``llama3_8b_decode`` alone (same seed, same draw)."""
    return _uniform_lengths(np.random.default_rng(seed), num_seqs, min_len, max_len)


def llama3_8b_decode(seed: int = 1236, num_seqs: int = 64, min_len: int = 512,
                     max_len: int = 4096, kv_dtype: str = "bf16",
                     block_size: int = 16) -> PagedBatch:
    """Llama-3-8B-shape decode: 64 sequences with lengths uniform in
    [512, 4096], 32 query heads over 8 KV heads, head size 128, block 16
    (64 and 128 are the larger blocks of the same workload: same lengths and
    values, fewer and larger table entries), pool sized 1.25x the blocks
    needed, tables drawn from a shuffled pool."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 32, 8, 128, block_size
    seq_lens = _uniform_lengths(rng, num_seqs, min_len, max_len)
    needed = int(sum((int(L) + bs - 1) // bs for L in seq_lens))
    nb = _pool_blocks(needed)
    perm = rng.permutation(nb).astype(np.int32)
    tables, _ = _tables_from_lengths(seq_lens, bs, perm)
    q = _normal(rng, (num_seqs, Hq, D))
    T = int(seq_lens.sum())
    k = _normal(rng, (T, Hkv, D))
    v = _normal(rng, (T, Hkv, D))
    slots = np.concatenate([_slots_for(tables[s], seq_lens[s], bs) for s in range(num_seqs)])
    name = "llama3_8b_decode_bf16" if bs == 16 else f"llama3_8b_decode_bf16_bs{bs}"
    return PagedBatch(name, Hq, Hkv, D, bs, nb, "bf16", "bf16", kv_dtype,
                      1.0 / math.sqrt(D), q, k, v, slots, seq_lens, tables)


def continuous_batching_decode(seed: int = 1241, num_seqs: int = 768, min_len: int = 64,
                               max_len: int = 1024, block_size: int = 16) -> PagedBatch:
    """A continuous-batching decode step, Llama-3-8B shape: many sequences
    at every stage of generation in one batch ("vLLM：大语言模型推理与服务库"
    §4.5: requests join and leave the running batch each step), here 768
    sequences with lengths uniform in [64, 1024], 32 query heads over 8 KV
    heads, head size 128, bf16, block 16, pool 1.25x the blocks needed,
    tables from a shuffled pool."""
    b = llama3_8b_decode(seed=seed, num_seqs=num_seqs, min_len=min_len, max_len=max_len,
                         block_size=block_size)
    b.name = "continuous_batching_decode_bf16"
    return b


def long_context_decode(seed: int = 1237, num_seqs: int = 8, seq_len: int = 32768,
                        partition_size: int = 512, outlier_frac: float = 0.01,
                        outlier_gain: float = 8.0) -> PagedBatch:
    """Long-context split-K decode: 8 sequences of 32768 tokens, 32/8 heads,
    head size 128, block 16, 512-token partitions; 1% of the (token, KV head)
    key rows are multiplied by 8 to widen the softmax range."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 32, 8, 128, 16
    seq_lens = np.full(num_seqs, seq_len, dtype=np.int32)
    needed = num_seqs * ((seq_len + bs - 1) // bs)
    nb = _pool_blocks(needed)
    perm = rng.permutation(nb).astype(np.int32)
    tables, _ = _tables_from_lengths(seq_lens, bs, perm)
    q = _normal(rng, (num_seqs, Hq, D))
    T = int(seq_lens.sum())
    k = _normal(rng, (T, Hkv, D))
    v = _normal(rng, (T, Hkv, D))
    n_rows = T * Hkv
    n_out = int(round(outlier_frac * n_rows))
    rows = rng.choice(n_rows, size=n_out, replace=False)
    k.reshape(n_rows, D)[rows] *= np.float32(outlier_gain)
    slots = np.concatenate([_slots_for(tables[s], seq_lens[s], bs) for s in range(num_seqs)])
    return PagedBatch("long_context_splitk_bf16", Hq, Hkv, D, bs, nb, "bf16", "bf16", "bf16",
                      1.0 / math.sqrt(D), q, k, v, slots, seq_lens, tables,
                      partition_size=partition_size)


def shared_prefix_decode(seed: int = 1238, num_forks: int = 256, prefix_len: int = 2048,
                         max_suffix: int = 512, pool_factor: float = 1.25) -> PagedBatch:
    """Parallel sampling from one shared prefix: 256 sequences forked from a
    2048-token prefix whose blocks every fork shares, then distinct suffixes
    of uniform [0, 512] tokens plus one new decode token each.

    Forking copies the parent's block table so children point at the same
    physical blocks ("vLLM 高性能大语言模型推理引擎深度技术评估与分布式架构展望",
    section on the fork/append/free primitives).  A prefix whose last block is
    partly filled cannot take a child's tokens in place: each child gets a
    private copy of that block first (copy-on-write), listed in
    ``copy_pairs`` as (shared block, private block).  With a 2048-token prefix
    at block 16 no prefix block is partial and ``copy_pairs`` is empty; pass
    ``prefix_len=2040`` for the variant where all 256 forks copy.
    ``pool_factor`` sizes the pool against the blocks in use (1.25 by
    default; a serving pool sized to memory is several times larger).
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 32, 8, 128, 16
    suffix = rng.integers(0, max_suffix + 1, size=num_forks, dtype=np.int64)
    seq_lens = (prefix_len + suffix + 1).astype(np.int32)
    n_prefix_blocks = (prefix_len + bs - 1) // bs
    partial = prefix_len % bs != 0
    full_prefix = prefix_len // bs  # fully filled, shared read-only
    # Blocks each fork owns privately: everything past the full prefix blocks.
    own = [(int(L) + bs - 1) // bs - full_prefix for L in seq_lens]
    needed = n_prefix_blocks + sum(own)
    nb = _pool_blocks(needed, pool_factor)
    perm = rng.permutation(nb).astype(np.int32)
    prefix_blocks = perm[:n_prefix_blocks]
    cur = n_prefix_blocks
    mb = max((int(L) + bs - 1) // bs for L in seq_lens)
    tables = np.full((num_forks, mb), -1, dtype=np.int32)
    copy_pairs = []
    for s in range(num_forks):
        tables[s, :full_prefix] = prefix_blocks[:full_prefix]
        tables[s, full_prefix:full_prefix + own[s]] = perm[cur:cur + own[s]]
        if partial:
            copy_pairs.append((int(prefix_blocks[full_prefix]), int(tables[s, full_prefix])))
        cur += own[s]
    q = _normal(rng, (num_forks, Hq, D))
    # Prefix tokens are written once into the shared blocks; each fork's own
    # tokens (suffix + decode token) are written into its private blocks.
    n_own_tokens = [int(L) - prefix_len for L in seq_lens]
    T = prefix_len + sum(n_own_tokens)
    k = _normal(rng, (T, Hkv, D))
    v = _normal(rng, (T, Hkv, D))
    prefix_table = np.full(mb, -1, dtype=np.int32)
    prefix_table[:n_prefix_blocks] = prefix_blocks
    slots = [_slots_for(prefix_table, prefix_len, bs)]
    for s in range(num_forks):
        slots.append(_slots_for(tables[s], int(seq_lens[s]), bs, first=prefix_len))
    slots = np.concatenate(slots)
    pairs = np.array(copy_pairs, dtype=np.int64).reshape(-1, 2)
    b = PagedBatch("shared_prefix_bf16", Hq, Hkv, D, bs, nb, "bf16", "bf16", "bf16",
                   1.0 / math.sqrt(D), q, k, v, slots, seq_lens, tables, copy_pairs=pairs,
                   notes=f"prefix_len={prefix_len}")
    b.prefix_len = prefix_len
    b.prefix_blocks = prefix_blocks
    return b


def mixed_fp8_step(seed: int = 1239, num_decode: int = 32, min_len: int = 1024,
                   max_len: int = 8192, prompt_len: int = 2048, chunk_len: int = 512,
                   chunk_start: int = 1536) -> PagedBatch:
    """Mixed chunked-prefill + decode step over one fp8 (E4M3) pool with
    per-tensor scales: 70B-shape GQA (64 query heads over 8 KV heads), head
    size 128, block 32; 32 decode sequences with lengths uniform in
    [1024, 8192] plus one 512-query chunk at offset 1536 of a 2048-token
    prompt.  Keys/values are drawn in float32, stored as bf16 source tokens
    and quantised into the pool by the cache write; each scale is the
    largest magnitude of its bf16 source tensor divided by 448."""
    import torch  # storage casts only

    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 64, 8, 128, 32
    seq_lens = rng.integers(min_len, max_len + 1, size=num_decode, dtype=np.int64).astype(np.int32)
    dec_blocks = [(int(L) + bs - 1) // bs for L in seq_lens]
    chunk_blocks = (prompt_len + bs - 1) // bs
    needed = sum(dec_blocks) + chunk_blocks
    nb = _pool_blocks(needed)
    perm = rng.permutation(nb).astype(np.int32)
    tables, cur = _tables_from_lengths(seq_lens, bs, perm)
    ctable = np.full((1, chunk_blocks), -1, dtype=np.int32)
    ctable[0] = perm[cur:cur + chunk_blocks]
    q = _normal(rng, (num_decode, Hq, D))
    T = int(seq_lens.sum()) + prompt_len
    k = _normal(rng, (T, Hkv, D))
    v = _normal(rng, (T, Hkv, D))
    chunk_q = _normal(rng, (chunk_len, Hq, D))
    slots = [_slots_for(tables[s], int(seq_lens[s]), bs) for s in range(num_decode)]
    slots.append(_slots_for(ctable[0], prompt_len, bs))
    slots = np.concatenate(slots)

    def amax_scale(x):
        xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32)
        return float(np.float32(xb.abs().max().item()) / np.float32(448.0))

    b = PagedBatch("mixed_prefill_decode_fp8", Hq, Hkv, D, bs, nb, "bf16", "bf16", "fp8",
                   1.0 / math.sqrt(D), q, k, v, slots, seq_lens, tables,
                   k_scale=amax_scale(k), v_scale=amax_scale(v),
                   chunk_q=chunk_q,
                   chunk_query_start=np.array([0, chunk_len], dtype=np.int32),
                   chunk_seq_lens=np.array([chunk_start + chunk_len], dtype=np.int32),
                   chunk_block_tables=ctable)
    b.prompt_len = prompt_len
    return b


def budget_chunks(prompt_lens, budget: int, step: int):
    """The chunks of one scheduler step of chunked prefill under a token
    budget: prompts are served in order, each step takes up to ``budget``
    tokens, a prompt that does not fit is cut and continues at the next
    step.  Returns [(prompt index, first position, chunk length)] of step
    ``step`` (0-based); empty once every prompt is done."""
    done = [0] * len(prompt_lens)
    p = 0
    for s in range(step + 1):
        left, chunks = budget, []
        while left > 0 and p < len(prompt_lens):
            n = min(int(prompt_lens[p]) - done[p], left)
            chunks.append((p, done[p], n))
            done[p] += n
            left -= n
            if done[p] == int(prompt_lens[p]):
                p += 1
        if s == step:
            return chunks
    return []


def chunked_prefill_step(seed: int = 1240, budget: int = 2048, step: int = 3,
                         num_prompts: int = 24, min_len: int = 256, max_len: int = 2048,
                         block_size: int = 16) -> PagedBatch:
    """One step of varlen chunked prefill under a token budget (512 or 2048
    batched tokens), Llama-3-8B shape: 32 query heads over 8 KV heads, head
    size 128, bf16 pool, block 16.  Prompt lengths are uniform in
    [256, 2048]; the step's chunks are what ``budget_chunks`` gives for step
    ``step`` (a continued prompt first, then new ones, the last one cut).
    Each prompt's pool holds its tokens up to the end of its chunk (earlier
    chunks and the chunk's own K/V already written)."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 32, 8, 128, block_size
    prompt_lens = _uniform_lengths(rng, num_prompts, min_len, max_len)
    chunks = budget_chunks(prompt_lens, budget, step)
    if not chunks:
        raise ValueError("the step is past the last prompt")
    ends = np.array([first + n for _, first, n in chunks], dtype=np.int32)
    nblk = [(int(L) + bs - 1) // bs for L in ends]
    nb = _pool_blocks(sum(nblk))
    perm = rng.permutation(nb).astype(np.int32)
    tables, _ = _tables_from_lengths(ends, bs, perm)
    T = int(ends.sum())
    k = _normal(rng, (T, Hkv, D))
    v = _normal(rng, (T, Hkv, D))
    n_q = [n for _, _, n in chunks]
    chunk_q = _normal(rng, (sum(n_q), Hq, D))
    slots = np.concatenate([_slots_for(tables[c], int(ends[c]), bs) for c in range(len(chunks))])
    b = PagedBatch(f"chunked_prefill_budget{budget}_bf16", Hq, Hkv, D, bs, nb, "bf16", "bf16",
                   "bf16", 1.0 / math.sqrt(D), chunk_q[:1], k, v, slots, ends, tables,
                   chunk_q=chunk_q,
                   chunk_query_start=np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32),
                   chunk_seq_lens=ends, chunk_block_tables=tables,
                   notes=f"chunks (prompt, first, len): {chunks}")
    b.chunks = chunks
    return b


WORKLOADS = {
    "tiny_fp32": tiny_decode,
    "llama3_8b_decode_bf16": llama3_8b_decode,
    "long_context_splitk_bf16": long_context_decode,
    "shared_prefix_bf16": shared_prefix_decode,
    "continuous_batching_decode_bf16": continuous_batching_decode,
    "mixed_prefill_decode_fp8": mixed_fp8_step,
    "chunked_prefill_budget2048_bf16": chunked_prefill_step,
    "chunked_prefill_budget512_bf16": lambda **kw: chunked_prefill_step(**{"budget": 512, **kw}),
}


def make(name: str, **kw) -> PagedBatch:
    return WORKLOADS[name](**kw)


def storage_tensor(x: np.ndarray, dtype: str):
    """float32 draws -> a CPU torch tensor in the storage dtype (torch's RNE cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(f"no source storage for dtype {dtype!r}")


def storage_bits(t) -> np.ndarray:
    """Raw storage of a CPU tensor as unsigned integers (uint32 / uint16 / uint8)."""
    import torch

    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.uint8, torch.int8) or str(t.dtype).startswith("torch.float8"):
        return t.view(torch.uint8).numpy()
    raise ValueError(f"unsupported tensor dtype {t.dtype}")


def poisoned_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_size: int,
                  dtype: str) -> np.ndarray:
    """A pool ``[num_blocks, num_kv_heads, block_size, head_size]`` of raw storage
    words, every slot set to the dtype's quiet NaN."""
    np_t = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}[dtype]
    return np.full((num_blocks, num_kv_heads, block_size, head_size), POISON_BITS[dtype], dtype=np_t)
