/*
 * pa.h — paged K/V cache attention for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The library implements the data-parallel path of PagedAttention as the
 * pages describe it:
 *   [LIB]  "vLLM：大语言模型推理与服务库", §4 "vLLM核心——PagedAttention"
 *          (§4.2 physical blocks, block table, block pool; §4.3 writing a
 *          new token's K/V; §4.4 the attention kernel's inputs and per-block
 *          computation);
 *   [EVAL] "vLLM 高性能大语言模型推理引擎深度技术评估与分布式架构展望"
 *          (logical-to-physical block mapping, step 4: the kernel gathers
 *          K/V in place through the block table; the fork/append/free
 *          primitives and copy-on-write; chunked prefill);
 *   [ESSAY] the openeuler.csdn.net vLLM essay, "PagedAttention：把操作系统
 *          的分页搬上 GPU" (kernel grid over heads, sequences and partitions);
 *   [DEEP] "vLLM 深度解析：从 PagedAttention 到生产部署", §3.1 (block table,
 *          prefix sharing, copy-on-write).
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every call
 * ---------------------------------------------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer owned by the caller.
 *   The library allocates no memory, keeps no per-call state and never
 *   synchronises: work is enqueued on `stream` (a hipStream_t; NULL = the
 *   default stream) and is complete only when the caller synchronises.
 *   Scalars (sizes, max lengths, scales) are host values, so no call reads
 *   device memory on the host.
 *
 * Element types (pa_dtype).  PA_F32 = IEEE binary32; PA_BF16 = bfloat16;
 *   PA_FP8_E4M3 = OCP FP8 E4M3FN (bias 7, no infinities, 0x7F/0xFF NaN,
 *   largest finite 448) holding value * scale with a per-tensor fp32 scale.
 *
 * K/V pool layout.  The K cache and the V cache are two separate pools with
 *   the same shape
 *       [num_blocks][num_kv_heads][block_size][head_size]
 *   head dimension fastest.  A (block, kv_head) tile of block_size tokens is
 *   contiguous (4 KiB for bf16 16x128, fp8 32x128 and f32 16x64), and one
 *   token row of one head is head_size contiguous elements.  Slot s of the
 *   pool is offset s % block_size of physical block s / block_size.
 *   Bytes of one pool: num_blocks * num_kv_heads * block_size * head_size *
 *   element size (pa_pool_bytes).
 *
 * Block tables.  block_tables is int32 [num_seqs][max_blocks_per_seq],
 *   row-major: entry j of row s is the physical block holding tokens
 *   j*block_size .. j*block_size+block_size-1 of sequence s ([LIB] §4.2
 *   item 2).  Entries at or past ceil(seq_len / block_size) are never read
 *   (callers usually fill them with -1).  Tables may share blocks (prefix
 *   sharing, [DEEP] §3.1).
 *
 * GQA.  num_heads query heads read num_kv_heads K/V heads in contiguous
 *   groups: query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Errors.  Every call validates its host arguments before enqueuing work
 *   and returns one of the PA_* codes below; on error nothing is enqueued.
 *   pa_strerror(code) names the code; pa_last_error() returns a message
 *   about the most recent failure on the calling thread.  Device-side
 *   data errors (a block id >= num_blocks, a sequence length past its
 *   table) cannot be seen by the device calls, which never read device
 *   memory on the host; they are undefined behaviour, like a bad
 *   page-table entry.  The pa_validate_* calls at the end of this header
 *   check host copies of those arrays and name the first bad entry.  Slots
 *   past the pool (cache write) and block pairs outside it (copy, swap)
 *   are skipped by the kernels.
 *
 * Alignment.  Query, output, key and value arrays and the pools must be
 *   16-byte aligned (the kernels move 16-byte vectors); int32 arrays 4-byte
 *   and int64 arrays 8-byte aligned.  Misaligned pointers are refused with
 *   PA_ERR_INVALID.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_F32 = 0,
  PA_BF16 = 1,
  PA_FP8_E4M3 = 2
} pa_dtype;

enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* null pointer, bad size, inconsistent arguments   */
  PA_ERR_UNSUPPORTED = -2, /* dtype / head_size / block_size / group not built */
  PA_ERR_WORKSPACE = -3,   /* workspace missing or too small                   */
  PA_ERR_HIP = -4,         /* the HIP runtime refused a launch                 */
  PA_ERR_NO_BLOCKS = -5    /* block manager: the free list cannot cover it     */
};

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t pa_version(void);

/* Name of an error code. Never NULL. */
const char* pa_strerror(int32_t code);

/* Detail of the most recent error on the calling thread ("" if none). */
const char* pa_last_error(void);

/* Bytes of ONE pool (K or V) in the layout above; 0 for invalid input. */
size_t pa_pool_bytes(int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                     int32_t head_size, int32_t cache_dtype);

/*
 * pa_cache_write — the slot-mapped cache write ("reshape and cache").
 *
 * [LIB] §4.3 item 2: each generated token's K/V is written into its
 * sequence's current block (a new block is taken from the pool when the
 * last one is full — that allocation is the caller's; it arrives here as
 * the slot).  For each token t with slot = slot_mapping[t] >= 0 and each KV
 * head h:
 *     k_cache[slot / block_size][h][slot % block_size][:] = enc(key[t][h][:])
 *     v_cache[...same...]                                  = enc(value[t][h][:])
 * A negative slot marks a padding token and is skipped; so is a slot at or
 * past num_blocks * block_size (no byte outside the pools is written).  Two
 * tokens must not share a slot.
 *
 *   key, value     [num_tokens][num_kv_heads][head_size] of src_dtype, contiguous
 *   src_dtype      PA_F32 or PA_BF16 (or PA_FP8_E4M3 into an fp8 cache)
 *   k_cache,v_cache  pools of cache_dtype, layout above
 *   slot_mapping   int64 [num_tokens]
 *   k_scale, v_scale  per-tensor scales, used only when cache_dtype is fp8
 *                  and src_dtype is not: enc(x) = E4M3FN(clamp(fp32(x) /
 *                  scale, -448, 448)) rounded to nearest, ties to even; NaN
 *                  stays NaN (0x7F with its sign).  Otherwise enc is a bit
 *                  copy (src_dtype must equal cache_dtype).
 * Supported: head_size * sizeof(cache element) a multiple of 16 bytes.
 * num_tokens == 0 is a valid no-op.
 */
int32_t pa_cache_write(const void* key, const void* value, int32_t src_dtype,
                       int32_t num_tokens,
                       void* k_cache, void* v_cache, int32_t cache_dtype,
                       int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                       int32_t head_size,
                       const int64_t* slot_mapping, float k_scale, float v_scale,
                       void* stream);

/*
 * pa_copy_blocks — the block copy behind copy-on-write.
 *
 * [EVAL] "束搜索与并行采样的三大调度原语": fork makes a child table point at
 * the parent's physical blocks; when a shared block is about to change, only
 * that block is copied into a fresh one ([DEEP] §3.1 copy-on-write).  For
 * each pair i, every K and V element of physical block block_mapping[2i]
 * (all heads, all offsets) is copied bit-exactly into block
 * block_mapping[2i+1].
 *
 *   block_mapping  int64 [num_pairs][2] = (src, dst), device memory
 * Destinations must be distinct and must not be the source of any pair
 * (all copies run concurrently); a pair naming a block outside the pool is
 * skipped.  num_pairs == 0 is a valid no-op.
 */
int32_t pa_copy_blocks(void* k_cache, void* v_cache, int32_t cache_dtype,
                       int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                       int32_t head_size,
                       const int64_t* block_mapping, int32_t num_pairs, void* stream);

/*
 * pa_swap_blocks — move whole blocks between two pools: the HBM pool and a
 * pool in pinned host memory, either way.
 *
 * The SWAP mode of preemption ([EVAL], its section on preemption; [DEEP]
 * §3.2, preemption strategies): when the HBM pool runs short, the physical
 * K/V blocks of a preempted sequence move to host memory over the host link
 * and come back when it resumes.  For each pair i, every K and V element of
 * block block_mapping[2i] of the source pools (all heads, all offsets) is
 * copied bit-exactly into block block_mapping[2i+1] of the destination
 * pools.
 *
 *   src_k, src_v  source pools [src_num_blocks][num_kv_heads][block_size][head_size]
 *   dst_k, dst_v  destination pools [dst_num_blocks][...] of the same geometry
 *   block_mapping int64 [num_pairs][2] = (source block, destination block)
 * Each of the five pointers is device memory or pinned host memory (from
 * hipHostMalloc, e.g. a torch tensor made with pin_memory=True); pinned host
 * memory is reached through its device mapping.  Pageable host memory is
 * refused with PA_ERR_INVALID before anything is enqueued.  All memory is
 * the caller's.  Destinations must be distinct; a pair naming a block
 * outside its pool is skipped.  The host must not touch a host pool between
 * the call and the completion of the work on the stream.  num_pairs == 0 is
 * a valid no-op (the pointers are still checked).
 */
int32_t pa_swap_blocks(const void* src_k, const void* src_v, int32_t src_num_blocks,
                       void* dst_k, void* dst_v, int32_t dst_num_blocks,
                       int32_t cache_dtype, int32_t block_size, int32_t num_kv_heads,
                       int32_t head_size, const int64_t* block_mapping, int32_t num_pairs,
                       void* stream);

/* partition_size value selecting the balanced split of pa_decode. */
#define PA_PARTITION_BALANCED (-1)

/* pa_decode flags (see pa_decode). */
#define PA_DECODE_READ_ONCE 0x1
#define PA_DECODE_SHARED 0x2
#define PA_DECODE_ENGINE_VALU 0x4
#define PA_DECODE_ENGINE_MFMA 0x8

/*
 * Workspace bytes pa_decode needs for split-K partials: 0 when
 * partition_size == 0 or one partition covers max_seq_len; for
 * PA_PARTITION_BALANCED two partial states and a two-word merge task per
 * wavefront of the largest balanced grid, plus a two-word cut record per
 * (sequence, KV head).
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_size, int32_t max_seq_len, int32_t partition_size);

/*
 * pa_decode — one query token per sequence against its paged context.
 *
 * [LIB] §4.4 items 1 and 3: with q, the K/V block pools, the block tables
 * and each sequence's context length, every query walks its sequence's
 * physical blocks, scores q·k, takes the softmax and weights V:
 *     out[s][h][:] = sum_t softmax_t(scale * q[s][h]·K_s[t][g]) * V_s[t][g]
 * over t < seq_lens[s], g = h / (num_heads / num_kv_heads), with K_s[t] read
 * from block block_tables[s][t / block_size], offset t % block_size, in place
 * ([EVAL] mapping step 4).  fp8 caches are dequantised as code * k_scale and
 * code * v_scale.  seq_lens[s] == 0 yields zeros.  The softmax runs in fp32
 * with a running maximum.
 *
 * Split-K ([ESSAY]: a grid axis over partitions of the context): with
 * partition_size > 0 (a multiple of block_size) each sequence's context is
 * cut into ceil(seq_len / partition_size) partitions processed in parallel;
 * each writes its (max score, exp-sum, normalised output) into `workspace`
 * and a second kernel merges them with log-sum-exp weights.  Sequences with
 * a single partition are finished by the first kernel.  partition_size == 0
 * processes each sequence in one partition and needs no workspace.
 * partition_size == PA_PARTITION_BALANCED cuts, per KV head, the blocks of
 * all sequences into equal contiguous runs, one per wavefront of a grid
 * sized to the device (so every wavefront streams the same number of
 * blocks whatever the length mix).  A wavefront finishes every sequence it
 * holds whole; a sequence cut between wavefronts leaves one partial state
 * per piece in `workspace`, and a second kernel merges them with the same
 * log-sum-exp weights.  The workspace needs no initialisation.
 *
 *   out            [num_seqs][num_heads][head_size] of q_dtype
 *   query          [num_seqs][num_heads][head_size] of q_dtype
 *   q_dtype/cache_dtype  (PA_F32, PA_F32), (PA_BF16, PA_BF16), (PA_BF16, PA_FP8_E4M3)
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens       int32 [num_seqs], each in [0, max_seq_len] and
 *                  ceil(seq_len / block_size) <= max_blocks_per_seq
 *   max_seq_len    host upper bound of seq_lens (sizes the grid)
 *   workspace      device buffer of >= pa_decode_workspace_size(...) bytes
 * Supported: head_size 64 or 128, block_size 16, 32, 64 or 128 (the range
 * [EVAL] gives for a physical block), num_heads / num_kv_heads in
 * {1, 2, 4, 8}, except f32 with head_size 128.
 * flags (a bitwise OR; 0 is always correct) tell the call how the K/V it
 * reads is shared, which it cannot see itself ([DEEP] §3.1: forks and
 * prefix sharing make several tables point at one physical block; the
 * caller's block manager knows the reference counts, pa_bm_tables_shared):
 *   PA_DECODE_READ_ONCE   no physical block appears twice among the blocks
 *                         the call reads (no sharing in the batch): K/V
 *                         lines are loaded evict-first, since none is read
 *                         again.  Wrong only in speed if the batch does
 *                         share blocks;
 *   PA_DECODE_SHARED      the tables share blocks: ordinary loads, and the
 *                         balanced split runs on the vector engine, whose
 *                         whole-row loads suit lines served from the caches;
 *   PA_DECODE_ENGINE_VALU pin the balanced split to the vector engine;
 *   PA_DECODE_ENGINE_MFMA pin it to the matrix-core engine (PA_ERR_UNSUPPORTED
 *                         where that engine is not built).
 * READ_ONCE with SHARED, or both engine bits, is PA_ERR_INVALID.
 * Engines (results agree within the bf16 rounding of P): by default, with
 * PA_PARTITION_BALANCED, head_size 128, groups of 4 or 8 and bf16 queries
 * run on the matrix cores; everything else on the vector ALUs.
 * Limits: with fixed partitions (partition_size >= 0) num_seqs and the
 * partition count are at most 65535; the balanced split has no limit on
 * num_seqs.
 */
int32_t pa_decode(void* out, const void* query, int32_t q_dtype,
                  int32_t num_seqs, int32_t num_heads, int32_t head_size,
                  const void* k_cache, const void* v_cache, int32_t cache_dtype,
                  int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* seq_lens, int32_t max_seq_len,
                  float scale, float k_scale, float v_scale,
                  int32_t partition_size, int32_t flags, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * pa_decode_append — a decode step's cache write and decode in one call:
 * each sequence's newest token is written into the pool and attended to.
 *
 * [LIB] §4.3 item 2 (each new token's K/V goes into the sequence's current
 * block, the slot the block table gives) followed by [LIB] §4.4 items 1
 * and 3 (pa_decode): for every sequence s with L = seq_lens[s] > 0, token
 * L - 1 is the new one.  Its K and V rows k_new[s] and v_new[s] (bf16,
 * [num_kv_heads][head_size] each) are stored at slot
 *     block_tables[s][(L - 1) / block_size] * block_size + (L - 1) % block_size
 * (an fp8 pool: quantised code = e4m3(x / k_scale) as pa_cache_write does),
 * and the attention over all L tokens is computed with them.  The pool
 * afterwards holds exactly what pa_cache_write with those slots leaves, and
 * `out` equals pa_cache_write followed by pa_decode with partition_size
 * PA_PARTITION_BALANCED and the same flags: the decode kernel writes the
 * token where it reads the sequence's last block and uses the new rows in
 * place of the slot's old contents, so the step needs no separate launch.
 *
 * Arguments as pa_decode (balanced split implied), plus
 *   k_new, v_new   bf16 [num_seqs][num_kv_heads][head_size], 16-byte aligned,
 *                  device memory; read only
 * Supported: the matrix-core engine's shapes (bf16 queries, bf16 or fp8 pool,
 * head_size 128, num_heads / num_kv_heads 4 or 8); elsewhere, or with
 * PA_DECODE_ENGINE_VALU, PA_ERR_UNSUPPORTED (use pa_cache_write and
 * pa_decode).  fp8 pools need k_scale, v_scale > 0.  Workspace: as pa_decode
 * with PA_PARTITION_BALANCED.  Two sequences whose last tokens map to one
 * slot are the caller's error (the writes race), as in pa_cache_write.
 */
int32_t pa_decode_append(void* out, const void* query, int32_t q_dtype,
                         int32_t num_seqs, int32_t num_heads, int32_t head_size,
                         const void* k_new, const void* v_new,
                         const void* k_cache, const void* v_cache, int32_t cache_dtype,
                         int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, int32_t max_seq_len,
                         float scale, float k_scale, float v_scale,
                         int32_t flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_shared_prefix — pa_decode for a batch whose sequences all begin
 * with the same prefix_len tokens held in the same physical blocks.
 *
 * [LIB] §4.2 item 2 and [DEEP] §3.1: parallel samples forked from one
 * prompt share the prompt's physical blocks (prefix sharing; copy-on-write
 * only for a block that changes).  pa_decode reads those blocks once per
 * sequence; here the attention to the shared prefix is computed once per
 * KV head for all the sequences' query heads together, as a dense product
 * on the matrix cores (S^T = K Q^T and O^T = V^T P^T over the prefix keys,
 * cut into splits across the chip), each sequence's own tokens past the
 * prefix run through the balanced split (from token prefix_len, with the
 * K/V reuse hints of `flags` as in pa_decode), and a log-sum-exp merge joins
 * the two.  The result is the same attention as pa_decode on the same
 * arguments (within the bf16 rounding of the probabilities).
 *
 * Arguments as pa_decode, plus
 *   prefix_len   tokens every sequence shares: a multiple of block_size,
 *                0 <= prefix_len <= every seq_lens[s]; the shared blocks are
 *                read from row 0 of block_tables, and every row must hold
 *                the same ids in its first prefix_len / block_size entries
 *                (pa_validate_shared_prefix checks a host copy)
 *   flags        PA_DECODE_* hints for the suffix part (usually
 *                PA_DECODE_READ_ONCE: the suffixes are private blocks)
 *   workspace    >= pa_decode_shared_prefix_workspace_size(...) bytes; needs
 *                no initialisation
 * Supported: bf16 queries, bf16 or fp8 cache, head_size 128, groups of 1,
 * 2, 4 or 8 (a prefix_len of 0 reduces to the balanced pa_decode and takes
 * its shapes).
 */
size_t pa_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_size,
                                              int32_t prefix_len);
int32_t pa_decode_shared_prefix(void* out, const void* query, int32_t q_dtype,
                                int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                const void* k_cache, const void* v_cache, int32_t cache_dtype,
                                int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t max_seq_len,
                                int32_t prefix_len, float scale, float k_scale, float v_scale,
                                int32_t flags, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * pa_decode_no_alloc — pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, meaning and results as pa_decode
 * without workspace / workspace_bytes: the split-K partials live in a
 * static device array of PA_DECODE_NO_ALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process ends.  A split that needs more
 * (pa_decode_workspace_size) is refused with PA_ERR_WORKSPACE before
 * anything is enqueued.  No call allocates or frees memory.  All calls on
 * one GPU share its array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.
 */
#define PA_DECODE_NO_ALLOC_SCRATCH_BYTES (48u * 1024u * 1024u)
int32_t pa_decode_no_alloc(void* out, const void* query, int32_t q_dtype,
                           int32_t num_seqs, int32_t num_heads, int32_t head_size,
                           const void* k_cache, const void* v_cache, int32_t cache_dtype,
                           int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t max_seq_len,
                           float scale, float k_scale, float v_scale,
                           int32_t partition_size, int32_t flags, void* stream);

/*
 * pa_profile_next_decode — measurement: the next decode call on the calling
 * thread (pa_decode, pa_decode_no_alloc or pa_decode_shared_prefix) records
 * start_event immediately before and stop_event immediately after its main
 * decode kernel on the call's stream (hipExtLaunchKernelGGL), so that the
 * kernel's own duration can be read with hipEventElapsedTime apart from
 * the reduce and merge kernels around it.  The events are hipEvent_t
 * created with timing enabled; they are used once and forgotten, also when
 * that call fails.  Passing NULL, NULL cancels; one NULL is PA_ERR_INVALID.
 */
int32_t pa_profile_next_decode(void* start_event, void* stop_event);

/*
 * pa_prefill_chunk — causal attention for chunks of prompt tokens whose K/V
 * are already in the paged cache.
 *
 * [EVAL] "分块预填充克服队头阻塞": a long prompt is processed in chunks so it
 * can share a step with decode.  Chunk c has query rows
 * query_start_loc[c] .. query_start_loc[c+1]-1 and seq_lens[c] keys in the
 * cache (earlier chunks and itself, written beforehand with
 * pa_cache_write).  Query i of a chunk of n queries sits at position
 * seq_lens[c] - n + i and attends keys 0..that position:
 *     out[r][h][:] = sum_{j <= pos} softmax_j(scale * q[r][h]·K_c[j][g]) * V_c[j][g]
 * QK^T and PV run on the matrix cores (bf16 operands, fp32 accumulation;
 * fp8 K/V widen exactly to bf16 and their scales are applied in fp32).
 *
 *   out, query     [num_tokens][num_heads][head_size] of q_dtype
 *   q_dtype/cache_dtype  (PA_BF16, PA_BF16) or (PA_BF16, PA_FP8_E4M3)
 *   query_start_loc int32 [num_chunks + 1], query_start_loc[num_chunks] == num_tokens
 *   max_query_len  host upper bound of the chunks' query counts
 *   block_tables   int32 [num_chunks][max_blocks_per_seq]
 *   seq_lens       int32 [num_chunks]; each >= its chunk's query count
 * Supported: head_size 128, block_size 16, 32, 64 or 128, group size in
 * {1, 2, 4, 8}.
 */
int32_t pa_prefill_chunk(void* out, const void* query, int32_t q_dtype,
                         int32_t num_tokens, int32_t num_heads, int32_t head_size,
                         const int32_t* query_start_loc, int32_t num_chunks,
                         int32_t max_query_len,
                         const void* k_cache, const void* v_cache, int32_t cache_dtype,
                         int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens,
                         float scale, float k_scale, float v_scale, void* stream);

/* ---------------------------------------------------------------------------
 * Host block manager ([LIB] §4.2 item 3 block pool, §4.3 item 2 new token;
 * [EVAL] the fork / append / free primitives and copy-on-write; [DEEP] §3.1)
 * ---------------------------------------------------------------------------
 * A host-side pool of num_blocks physical block ids, handed out first in,
 * first out (the order that reproduces [DEEP] §3.1's interleaved 9-block
 * figure), with a reference count per block and one block table per
 * sequence, keyed by a caller-chosen int64 id.  It produces the inputs of
 * the device calls: slot mappings for pa_cache_write, copy-on-write pairs
 * for pa_copy_blocks, block tables and lengths for pa_decode and
 * pa_prefill_chunk.  Unlike the device calls, every array argument here is
 * a HOST pointer owned by the caller; the manager owns its own host memory
 * (released by pa_bm_destroy) and no device memory.  Calls on one manager
 * must not overlap (no locking); each costs O(1) per token, block or
 * sequence it touches.
 * Errors: PA_ERR_INVALID (NULL pointer, negative size, unknown or
 * duplicate id), PA_ERR_NO_BLOCKS (the free list cannot cover the request;
 * the manager is left unchanged).  Running out of host memory is fatal.
 */
typedef struct pa_block_manager pa_block_manager;

/* A manager of blocks 0 .. num_blocks-1 of block_size tokens, all free.
 * Returns NULL (and sets pa_last_error) for non-positive sizes. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
/* The same with a second pool of num_host_blocks host blocks (>= 0) that
 * swapped-out sequences occupy (pa_bm_swap_out / pa_bm_swap_in). */
pa_block_manager* pa_bm_create_swap(int32_t num_blocks, int32_t num_host_blocks,
                                    int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);

/* Number of free blocks (>= 0), or PA_ERR_INVALID. */
int32_t pa_bm_num_free(const pa_block_manager* bm);

/* A new sequence of num_tokens tokens (its prompt): takes
 * ceil(num_tokens / block_size) blocks and writes the slot of every token to
 * slot_mapping[0 .. num_tokens-1]. */
int32_t pa_bm_add(pa_block_manager* bm, int64_t seq_id, int32_t num_tokens, int64_t* slot_mapping);

/* One new token for each of seq_ids[0 .. num_seqs-1], in order (a decode
 * step; an id may repeat).  slot_mapping[i] receives the slot of token i.
 * A sequence whose last block is full takes a new block; one whose last
 * block is shared and not full first copies it (copy-on-write): the pair
 * (shared block, fresh block) is written to cow_pairs[2c], cow_pairs[2c+1]
 * (int64 [num_seqs][2] capacity) and *num_cow counts the pairs.  The copies
 * must happen (pa_copy_blocks) before the new tokens are written
 * (pa_cache_write). */
int32_t pa_bm_append(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                     int64_t* slot_mapping, int64_t* cow_pairs, int32_t* num_cow);

/* child_id becomes a sequence sharing every block of parent_id (one more
 * reference each); nothing is copied. */
int32_t pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Releases a sequence: one reference less on each of its blocks; blocks at
 * zero return to the back of the free list, last block first. */
int32_t pa_bm_free(pa_block_manager* bm, int64_t seq_id);

/* Tokens of a sequence (>= 0), or PA_ERR_INVALID. */
int32_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id);

/* Block tables of seq_ids[0 .. num_seqs-1] into block_tables (int32
 * [num_seqs][max_blocks_per_seq], entries past a table's end set to -1) and
 * their lengths into seq_lens (int32 [num_seqs]); PA_ERR_INVALID (nothing
 * written) if a table is longer than max_blocks_per_seq. */
int32_t pa_bm_block_tables(const pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                           int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* seq_lens);

/* References held on a block of the device pool (0 = free), or PA_ERR_INVALID. */
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block);

/* Swap for preemption ([EVAL], its section on preemption: SWAP moves the
 * blocks of a preempted sequence to host memory and back when it resumes;
 * [DEEP] §3.2, preemption strategies).
 *
 * pa_bm_swap_out moves seq_ids[0 .. num_seqs-1] (distinct, not swapped out)
 * to host blocks.  The set must hold its blocks alone: a block also held by
 * a sequence outside the set cannot move (PA_ERR_INVALID), so forked
 * siblings go together.  Each distinct block moves once, in order of first
 * appearance (sequences in the given order, each table front to back), to a
 * host block taken from the front of the host free list; its reference
 * count moves with it and the device block returns to the back of the
 * device free list.  The pairs (device block, host block) are written to
 * pairs (int64 [max_pairs][2]) and *num_pairs counts them; they are the
 * block_mapping of the pa_swap_blocks call that must run before the freed
 * device blocks are written again.  PA_ERR_NO_BLOCKS (nothing changed) if
 * the host pool cannot hold the set, PA_ERR_INVALID if max_pairs is too
 * small.  A swapped-out sequence can be freed (its host blocks return to
 * the host free list) but not appended to, forked, or listed by
 * pa_bm_block_tables.
 *
 * pa_bm_swap_in is the reverse for swapped-out sequences: pairs are (host
 * block, device block) and PA_ERR_NO_BLOCKS means the device pool is short. */
int32_t pa_bm_swap_out(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                       int64_t* pairs, int32_t max_pairs, int32_t* num_pairs);
int32_t pa_bm_swap_in(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                      int64_t* pairs, int32_t max_pairs, int32_t* num_pairs);

/* Free host blocks (>= 0), or PA_ERR_INVALID. */
int32_t pa_bm_num_free_host(const pa_block_manager* bm);

/* 1 if the sequence is swapped out, 0 if not, or PA_ERR_INVALID. */
int32_t pa_bm_is_swapped(const pa_block_manager* bm, int64_t seq_id);

/* Automatic prefix caching ([EVAL], its section on prefix caching).
 *
 * Every full block gets a chained hash of the previous block's hash, the
 * block's token ids and an extra hash (e.g. an adapter id): 64-bit FNV-1a
 * over the little-endian bytes of parent_hash (8; 0 for a sequence's first
 * block), the token ids (4 each) and extra_hash (8) — pa_bm_block_hash
 * (which returns 0 for a negative num_tokens or NULL tokens; 0 is also a
 * possible hash, so callers validate their own input).  A
 * table maps hashes to device blocks.  Unreferenced cached blocks stay in
 * the free list, whose front block leaves the table when it is taken
 * (eviction): least recently released first and, since a freed sequence
 * returns its blocks last block first, the leaves of a chain before the
 * blocks near its root.  A swapped-out block leaves the cache.
 *
 * pa_bm_enable_prefix_caching turns the cache on; it must be called before
 * the first sequence (PA_ERR_INVALID otherwise).
 *
 * pa_bm_add_prompt adds a sequence with its prompt token ids
 * (tokens int32 [num_tokens]): the chain of its full blocks is looked up
 * block by block up to the first miss (a hit also compares the block's
 * stored token ids and extra hash); the hits join its table with one more
 * reference each (an unreferenced hit leaves the free list), the rest of
 * the blocks are taken from the free list, and the new full blocks enter
 * the table (a hash already in the table keeps its block).  slot_mapping
 * receives every token's slot and *num_cached_tokens the number of leading
 * tokens whose K/V is already in the pool (a multiple of block_size): the
 * caller writes K/V for tokens num_cached_tokens .. num_tokens-1 only.
 * PA_ERR_NO_BLOCKS (nothing changed) if the free list cannot cover the
 * blocks that missed.
 *
 * pa_bm_append_tokens is pa_bm_append with the new token id of each listed
 * sequence (tokens int32 [num_seqs]); a block that its token fills enters
 * the table.  Sequences added by pa_bm_add, or appended to by pa_bm_append,
 * have unknown token ids and commit nothing more. */
uint64_t pa_bm_block_hash(uint64_t parent_hash, const int32_t* tokens, int32_t num_tokens,
                          uint64_t extra_hash);
int32_t pa_bm_enable_prefix_caching(pa_block_manager* bm);
int32_t pa_bm_add_prompt(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                         int32_t num_tokens, uint64_t extra_hash, int64_t* slot_mapping,
                         int32_t* num_cached_tokens);
int32_t pa_bm_append_tokens(pa_block_manager* bm, int32_t num_seqs, const int64_t* seq_ids,
                            const int32_t* tokens, int64_t* slot_mapping, int64_t* cow_pairs,
                            int32_t* num_cow);
/* Blocks in the prefix cache's table (>= 0), or PA_ERR_INVALID. */
int32_t pa_bm_num_cached_blocks(const pa_block_manager* bm);

/* ---------------------------------------------------------------------------
 * Host-side validation of the device calls' data arrays
 * ---------------------------------------------------------------------------
 * The device calls never read device memory on the host, so a block id past
 * the pool or a length past its table reaches the kernels ([LIB] §4.2 item
 * 2: the block table is the only map from logical to physical blocks, as a
 * page table is).  These calls check HOST copies of those arrays before a
 * launch.  Each returns PA_OK, or PA_ERR_INVALID with pa_last_error naming
 * the first offending entry (array, index, value and the bound it breaks)
 * and, if bad_index is not NULL, that entry's flat index in its array
 * (-1 on PA_OK).  They touch no device state and cost O(entries read).
 *
 * pa_validate_decode: for every sequence s, 0 <= seq_lens[s] <=
 *   max_seq_len, ceil(seq_lens[s] / block_size) <= max_blocks_per_seq, and
 *   every table entry the sequence reads is a block of the pool
 *   (0 <= id < num_blocks).  block_tables is [num_seqs][max_blocks_per_seq].
 * pa_validate_prefill: query_start_loc[0] == 0, non-decreasing, ending at
 *   num_tokens; every chunk's query count <= max_query_len and <= its
 *   seq_lens entry; its table entries as for decode.
 * pa_validate_slots: every slot is negative (padding) or inside the pool
 *   (< num_blocks * block_size), and no slot repeats.
 * pa_validate_shared_prefix: every sequence holds at least prefix_len
 *   tokens (a multiple of block_size) and its first prefix_len / block_size
 *   table entries equal those of row 0, which are pool blocks.
 * pa_validate_block_pairs: every (src, dst) pair of block_mapping
 *   [num_pairs][2] names blocks inside the source (src_num_blocks) and
 *   destination (dst_num_blocks) pools, destinations are distinct, and, with
 *   same_pool != 0 (pa_copy_blocks), no destination is the source of a pair.
 */
int32_t pa_validate_decode(const int32_t* block_tables, int32_t num_seqs,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           int32_t max_seq_len, int32_t num_blocks, int32_t block_size,
                           int64_t* bad_index);
int32_t pa_validate_prefill(const int32_t* query_start_loc, int32_t num_chunks,
                            int32_t num_tokens, int32_t max_query_len,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t num_blocks, int32_t block_size,
                            int64_t* bad_index);
int32_t pa_validate_slots(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                          int32_t block_size, int64_t* bad_index);
int32_t pa_validate_shared_prefix(const int32_t* block_tables, int32_t num_seqs,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t prefix_len, int32_t num_blocks, int32_t block_size,
                                  int64_t* bad_index);
int32_t pa_validate_block_pairs(const int64_t* block_mapping, int32_t num_pairs,
                                int32_t src_num_blocks, int32_t dst_num_blocks,
                                int32_t same_pool, int64_t* bad_index);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
