// prefill_kernels.hip — causal chunked prefill over the paged K/V cache on
// the CDNA4 matrix cores.
//
// What it computes ("vLLM 高性能大语言模型推理引擎深度技术评估与分布式架构展望",
// "分块预填充克服队头阻塞": a long prompt is processed chunk by chunk): every
// query row of a chunk attends, causally, to the keys already in the cache
// (earlier chunks and the chunk itself, written beforehand by the cache
// write), gathered through the chunk's block table ("vLLM：大语言模型推理与
// 服务库" §4.2 item 2, §4.4 item 3).
//
// Shape of the work on gfx950:
//   * a workgroup takes 128 rows = (query, head) pairs of one KV head group
//     (128/G queries x G heads, so the G heads share every K/V tile) and
//     walks the keys 64 at a time; its 8 wavefronts are 4 row groups of 32
//     rows times 2 key halves: wavefront (r, h) computes rows 32r..32r+31
//     against keys 32h..32h+31 of every 64-key step, so two wavefronts per
//     SIMD interleave their matrix and softmax work, and the two halves'
//     states are merged through LDS at the end;
//   * the 64-key K tile and the transposed V tile are staged in LDS as
//     bf16 (fp8 E4M3 widens to bf16 exactly; the per-tensor scales are
//     applied in fp32, k_scale inside the score scale, v_scale on the
//     output); the next step's global loads are in flight while the current
//     one is computed;
//   * scores are computed transposed, S^T = K · Q^T, with
//     v_mfma_f32_32x32x16_bf16 (8 per 32-key tile), so each lane holds 16
//     keys of one query row: the row maximum needs one cross-lane step and
//     the probabilities are already in the B-operand layout of
//     O^T = V^T · P^T (8 more MFMAs), with the keys taken in a consistent
//     permuted order;
//   * online softmax in fp32 in the log2 domain, rescaling the accumulators
//     only when a score exceeds the running reference by 2^8;
//   * tiles that cross the diagonal are masked per element (key > position);
//     tiles past every row of a wavefront are skipped.
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kPD = 128;             // head size
constexpr int kKB = 32;              // keys per wavefront tile
constexpr int kStep = 2 * kKB;       // keys staged per step
constexpr int kRows = 128;           // rows per workgroup
constexpr int kRowGroups = kRows / 32;
constexpr int kPWaves = 2 * kRowGroups;
constexpr int kPThreads = kPWaves * kWave;
constexpr int kKStride = kPD + 8;    // LDS row stride of K (bf16 elements)
constexpr int kVStride = kPD + 32;   // LDS row stride of V (bf16 elements)
constexpr int kBufs = 4;             // LDS step buffers in rotation
constexpr float kPLog2e = 1.4426950408889634f;
constexpr float kPSlack = 8.0f;
static_assert(kPThreads / 8 == kStep, "the staging map covers one step exactly");
constexpr int kKBytes = kStep * kKStride * 2;
constexpr int kVBytes = kStep * kVStride * 2;
constexpr int kBufBytes = kKBytes + kVBytes;
// After the key walk: the two key halves trade half of their accumulators
// (kMergeFloats), then the finished tile goes through LDS row by row
// (kTileStride bytes per row of bf16 outputs) so that global stores cover
// whole rows.
constexpr int kMergeFloats = 2 * kRowGroups * (kPD / 4) * kWave + 4 * kRowGroups * kWave;
constexpr int kTileStride = kPD * 2 + 16;
constexpr int kTileOff = kMergeFloats * 4;
constexpr int kQStride = kPD * 2 + 16;  // LDS row stride of the query tile (bytes)
constexpr int kLdsBytes = kBufs * kBufBytes;
static_assert(kTileOff + kRows * kTileStride <= kLdsBytes, "the epilogue fits the step buffers");
static_assert(kRows * kQStride <= kBufBytes, "the query tile fits one step buffer");
static_assert(kLdsBytes <= 160 * 1024, "one workgroup's LDS fits a CU");

// How the query enters: the kernel's score scale is always positive, so a
// negative scale moves onto the query's sign and a zero scale zeroes the
// query (all scores 0, the same softmax as any positive scale on them).
constexpr int kQAsIs = 0, kQNegate = 1, kQZero = 2;

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ void fp8x4_to_bf16x2x2(uint32_t w, uint32_t& lo, uint32_t& hi) {
  // Exact: every E4M3 value is a bf16 value (scale 1).
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// max(x[lane], x[lane ^ 32]): v_permlane32_swap(x, x) returns the low
// half-wave's values in both halves and the high half-wave's in both.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return fmaxf(u2f(r[0]), u2f(r[1]));
}

// ds_read_b64_tr_b16 (gfx950): in each 16-lane group, lane t gives the
// address of 4 consecutive bf16 F[t][0..3], and lane j receives
// F[4k + j/4][j%4] for k = 0..3.
__device__ __forceinline__ u32x2 lds_tr16(const __bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

template <int N> struct Buf { static constexpr int value = N; };

// The prefix mode of the kernel (attention of many decode queries to one
// shared prefix): the rows are num_q queries (one per sequence), every row
// sees every key of the prefix (no causal mask), and the keys are cut into
// splits of split_len (grid z): split c covers keys c * split_len ..
// min(prefix_len, (c + 1) * split_len) - 1 of table row 0.  Each split
// leaves, per (query, head), its output normalised by its own exponent sum
// (no value scale), rounded to bf16 like any output, and its (reference
// maximum, exponent sum), log2 domain, in fp32, for a log-sum-exp merge:
// o[(c * num_q + q) * num_heads + h][head dim], ml[...][2].
struct PrefixStates {
  uint16_t* o;
  float* ml;
  int num_q;
  int split_len;   // a multiple of 128 keys: whole blocks and whole steps
  int prefix_len;
};

template <typename KV, int BS, int G, bool kPrefix>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(
    void* __restrict__ out, const void* __restrict__ query,
    const int32_t* __restrict__ query_start_loc, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int max_blocks_per_seq, const int32_t* __restrict__ seq_lens, int num_kv_heads,
    float qk_scale_log2, int q_mode, float v_scale, PrefixStates ps) {
  constexpr int EB = Elem<KV>::bytes;
  static_assert(kRows % G == 0, "rows hold whole queries");
  // Four LDS buffers, each one step's K tile and V tile (both key rows);
  // after the key walk the same bytes hold the merge of the two key halves.
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  auto k_lds = [&](int b) { return (__bf16*)(lds + b * kBufBytes); };
  auto v_lds = [&](int b) { return (__bf16*)(lds + b * kBufBytes + kKBytes); };

  const int tile = blockIdx.x, g = blockIdx.y, c = blockIdx.z;
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int rg = w % kRowGroups, kh = w / kRowGroups;
  const int half = lane / 32;
  // Chunk c: queries qs .. qs+n-1 over its L keys, query i at position
  // L - n + i.  Prefix mode: split c's L keys (positions relative to the
  // split's first key, whose table entries start at tbl), every query at
  // position L - 1.
  int qs, n, L;
  const int32_t* tbl;
  if constexpr (kPrefix) {
    qs = 0;
    n = ps.num_q;
    const int k_lo = c * ps.split_len;
    L = min(ps.prefix_len - k_lo, ps.split_len);
    tbl = block_tables + k_lo / BS;
  } else {
    qs = query_start_loc[c];
    n = query_start_loc[c + 1] - qs;
    L = seq_lens[c];
    tbl = block_tables + (int64_t)c * max_blocks_per_seq;
  }
  if (tile * kRows >= n * G) return;
  const int pos_shift = kPrefix ? L - 1 : L - n;  // position of query i: pos_shift + (kPrefix ? 0 : i)
  auto position = [&](int i) { return kPrefix ? pos_shift : pos_shift + i; };
  const int q_first = tile * kRows / G;
  const int q_last = min(q_first + kRows / G, n) - 1;
  const int min_pos = position(q_first), max_pos = position(q_last);
  const int nsteps = (max_pos + kStep) / kStep;
  const int nblk = (L + BS - 1) / BS;
  const int num_heads = num_kv_heads * G;

  // This lane's row: query qi, head hq.
  const int row = 32 * rg + (lane & 31);
  const int qi = q_first + row / G;
  const int hq = g * G + row % G;
  const bool row_ok = qi < n;
  const int pos = position(qi);
  // Last position among this wavefront's rows: later tiles are all masked.
  const int wave_max_pos = position(min(q_first + (32 * rg + 31) / G, q_last));

  // The tile's query rows arrive with whole-row loads (16 lanes per 256-byte
  // row, four rows per load instruction) and wait in the last step buffer,
  // which is first written two steps into the key walk.
  constexpr int kQPieces = kRows * kPD * 2 / 16 / kPThreads;  // 16-byte pieces per thread
  u32x4 qraw[kQPieces];
#pragma unroll
  for (int k = 0; k < kQPieces; ++k) {
    const int f = t + k * kPThreads, r = f / (kPD / 8), c = f % (kPD / 8);
    const int rq = q_first + r / G;
    qraw[k] = u32x4{0u, 0u, 0u, 0u};
    if (rq < n)
      qraw[k] = *(const u32x4*)((const uint16_t*)query +
                                 ((int64_t)(qs + rq) * num_heads + g * G + r % G) * kPD + 8 * c);
  }
  uint8_t* q_lds = lds + (kBufs - 1) * kBufBytes;
  // Q^T operand: k-step s holds dims 16 s + 8 half .. +8 of the row.
  bf16x8 qreg[kPD / 16];

  f32x16 oacc[kPD / 32];
#pragma unroll
  for (int mt = 0; mt < kPD / 32; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[mt][i] = 0.f;
  float m_ref = -INFINITY, l_part = 0.f;

  // Staging: thread t covers key t/8, dims 16 (t%8) .. +16, of K and of V.
  // Each step's loads are issued two steps ahead (two register stages), and
  // the block-table entries they need one step before that.
  const int kk = t / 8, kd = (t % 8) * 16;
  constexpr int KVEC = 16 * EB / 16;  // 16-byte vectors per 16 elements
  struct Stage {
    u32x4 k[KVEC];
    u32x4 v[KVEC];
  };
  const int64_t head_off = (int64_t)g * BS * kPD;  // element offset of head g in a block
  const int64_t block_elems = (int64_t)num_kv_heads * BS * kPD;

  // A wavefront stages keys 8w .. 8w+7 of a step, which lie in one block
  // (blocks hold a multiple of 8 keys, and a step is whole blocks or a
  // whole half or quarter of one): its physical block is one wave-uniform
  // table entry, read with a scalar load so that waiting for it never waits
  // for the vector loads in flight, and a thread's offset inside the block
  // depends on the step only through the step's offset in a block larger
  // than a step.  Past the last block the last one is re-read; keys at or
  // past L are zeroed when stored, so every step issues the same loads
  // unconditionally and the wait for a stage counts only later loads.
  static_assert((kStep % BS == 0 || BS % kStep == 0) && BS % 8 == 0,
                "steps and blocks nest, blocks are whole 8-key groups");
  const int wkey = __builtin_amdgcn_readfirstlane(8 * w);
  const int last_blk = nblk - 1;
  auto block_id = [&](int step) -> int { return tbl[min((step * kStep + wkey) / BS, last_blk)]; };
  const uint8_t* k_head = (const uint8_t*)k_cache + head_off * EB;
  const uint8_t* v_head = (const uint8_t*)v_cache + head_off * EB;
  const int kv_off = ((kk % BS) * kPD + kd) * EB;
  auto load_stage = [&](int bid, int step, Stage& S) {
    const int64_t base = (int64_t)bid * block_elems * EB +
                         (BS > kStep ? (int64_t)((step * kStep) % BS) * kPD * EB : 0);
    const u32x4* kp = (const u32x4*)(k_head + base + kv_off);
    const u32x4* vp = (const u32x4*)(v_head + base + kv_off);
#pragma unroll
    for (int v = 0; v < KVEC; ++v) S.k[v] = kp[v];
#pragma unroll
    for (int v = 0; v < KVEC; ++v) S.v[v] = vp[v];
  };
  // LDS layout of a buffer: K and V both as key rows of bf16, strides
  // kKStride and kVStride.  The two 8-dim halves of a 16-dim chunk are
  // stored swapped in chunks 4..7 of a K row and in every chunk of an odd V
  // row; either way the first 16-byte writes of a wavefront land on
  // distinct banks.  The V stride puts the 4 key rows of a transposing read
  // 16 banks apart.  Readers undo the swaps.
  const int k_wr_lo = kk * kKStride + kd + ((t % 8) >= 4 ? 8 : 0);  // bf16 elements
  const int k_wr_hi = kk * kKStride + kd + ((t % 8) >= 4 ? 0 : 8);
  const int v_wr_lo = kk * kVStride + kd + ((kk & 1) ? 8 : 0);
  const int v_wr_hi = kk * kVStride + kd + ((kk & 1) ? 0 : 8);
  auto widen = [&](const u32x4 (&x)[KVEC], uint32_t (&o)[8]) {
    if constexpr (std::is_same<KV, BF16>::value) {
      o[0] = x[0].x; o[1] = x[0].y; o[2] = x[0].z; o[3] = x[0].w;
      o[4] = x[1].x; o[5] = x[1].y; o[6] = x[1].z; o[7] = x[1].w;
    } else {
      fp8x4_to_bf16x2x2(x[0].x, o[0], o[1]);
      fp8x4_to_bf16x2x2(x[0].y, o[2], o[3]);
      fp8x4_to_bf16x2x2(x[0].z, o[4], o[5]);
      fp8x4_to_bf16x2x2(x[0].w, o[6], o[7]);
    }
  };
  // Zeroing keys past L happens here, where the stage is consumed, so the
  // wait for its loads stays two steps after their issue.
  auto store_stage = [&](int step, const Stage& S, int b) {
    const bool tail = step * kStep + kStep > L;  // some keys of the step are past L
    const bool ok = step * kStep + kk < L;
    uint32_t kw[8], vw[8];
    widen(S.k, kw);
    widen(S.v, vw);
    if (tail) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kw[i] = ok ? kw[i] : 0u;
        vw[i] = ok ? vw[i] : 0u;
      }
    }
    *(u32x4*)(k_lds(b) + k_wr_lo) = u32x4{kw[0], kw[1], kw[2], kw[3]};
    *(u32x4*)(k_lds(b) + k_wr_hi) = u32x4{kw[4], kw[5], kw[6], kw[7]};
    *(u32x4*)(v_lds(b) + v_wr_lo) = u32x4{vw[0], vw[1], vw[2], vw[3]};
    *(u32x4*)(v_lds(b) + v_wr_hi) = u32x4{vw[4], vw[5], vw[6], vw[7]};
  };

  auto active = [&](int step) { return step * kStep + kh * kKB <= wave_max_pos; };

  // S^T = K Q^T: lane holds keys m(i) = (i/4)*8 + 4 half + i%4 of its row.
  auto score_mfma = [&](f32x16& st, int b, int s) {
    const bf16x8 a = *(const bf16x8*)(k_lds(b) + (kh * kKB + (lane & 31)) * kKStride + 16 * s +
                                      8 * (s >= 4 ? 1 - half : half));
    st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], st, 0, 0, 0);
  };

  // Masks the diagonal, raises the reference maximum where needed; returns
  // the exponent offset (-reference, or 0 for a row with nothing unmasked).
  auto softmax_head = [&](int step, f32x16& st) -> float {
    const int key0 = step * kStep + kh * kKB;
    if (key0 + kKB - 1 > min_pos) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool masked = key0 + (i / 4) * 8 + 4 * half + (i % 4) > pos;
        st[i] = masked ? -INFINITY : st[i];
      }
    }
    // The maximum of the raw scores, scaled (the scale is positive).
    float mx = st[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, st[i]);
    mx = xor32_max(mx) * qk_scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kPSlack)) {
      const float mn = fmaxf(m_ref, mx);
      const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m_ref - mn);
      l_part *= alpha;
#pragma unroll
      for (int mt = 0; mt < kPD / 32; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mt][i] *= alpha;
      m_ref = mn;
    }
    return m_ref == -INFINITY ? 0.f : -m_ref;
  };

  // Probability of element i (masked scores are -inf; the scale is > 0).
  auto prob = [&](const f32x16& st, int i, float neg_m) {
    return fast_exp2(__builtin_fmaf(st[i], qk_scale_log2, neg_m));
  };

  // O^T += V^T P^T over two 16-key steps.  The A operand V^T (32 dims x 16
  // keys, keys in the scores' permuted order: k-index 8 half + i is key
  // 16 ks + 4 half + 8 (i/4) + i%4) comes from the key-row V tile with two
  // transposing reads: lane t of 16-lane group q addresses key row
  // 4 half + t/4 (+8 for the second read) and dims 16 (q%2) + 4 (t%4) .. +3.
  const int q16 = lane / 16, t16 = lane % 16;
  const int v_rd = (4 * half + t16 / 4) * kVStride +
                   ((16 * (q16 & 1) + 4 * (t16 % 4)) ^ (((t16 / 4) & 1) ? 8 : 0));
  auto pv = [&](const uint32_t (&pw)[8], const __bf16* vt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, u32x4{pw[4 * ks + 0], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]});
#pragma unroll
      for (int mt = 0; mt < kPD / 32; ++mt) {
        const __bf16* p = vt + (kh * kKB + 16 * ks) * kVStride + 32 * mt + v_rd;
        const u32x2 lo = lds_tr16(p), hi = lds_tr16(p + 8 * kVStride);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[mt], 0, 0, 0);
      }
    }
  };

  // Pipeline over steps j: buffer j%4 holds step j.  Iteration j: barrier
  // (every wavefront is past iteration j-1, so buffer (j+2)%4, last read
  // by step j-2's P·V, is free, and buffer (j+1)%4, written in iteration
  // j-1, is complete); store step j+2 from its register stage and issue
  // that stage's loads for step j+4; then step j+1's score MFMAs
  // interleaved with step j's exponentials, then step j's P·V.  Register
  // stages alternate (sa: even steps); the loop is unrolled by four so that
  // every buffer offset is a constant.  (The scheduling barriers keep the
  // stages' loads in issue order, which the waits for them count on.)
  Stage sa, sb;
  load_stage(block_id(0), 0, sa);
  __builtin_amdgcn_sched_barrier(0);
  load_stage(block_id(1), 1, sb);
  __builtin_amdgcn_sched_barrier(0);
  int bid = block_id(2);
  store_stage(0, sa, 0);
  load_stage(bid, 2, sa);
  bid = block_id(3);
  __builtin_amdgcn_sched_barrier(0);
  store_stage(1, sb, 1);
  load_stage(bid, 3, sb);
  bid = block_id(4);
#pragma unroll
  for (int k = 0; k < kQPieces; ++k) {
    const int f = t + k * kPThreads;
    *(u32x4*)(q_lds + (f / (kPD / 8)) * kQStride + (f % (kPD / 8)) * 16) = qraw[k];
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kPD / 16; ++s) {
    u32x4 v = *(const u32x4*)(q_lds + row * kQStride + (16 * s + 8 * half) * 2);
    if (q_mode == kQNegate) v ^= 0x80008000u;  // exact: -(q·k) = (-q)·k
    if (q_mode == kQZero) v = u32x4{0u, 0u, 0u, 0u};  // every score is 0
    qreg[s] = __builtin_bit_cast(bf16x8, v);
  }
  // Scores of even steps live in st_a, of odd steps in st_b.
  f32x16 st_a, st_b;
#pragma unroll
  for (int i = 0; i < 16; ++i) st_a[i] = 0.f;
#pragma unroll
  for (int s = 0; s < kPD / 16; ++s) score_mfma(st_a, 0, s);

  auto iteration = [&](auto buf, int j, Stage& S, f32x16& st_cur, f32x16& st_next) {
    constexpr int B = decltype(buf)::value;  // j % 4
    __syncthreads();
    store_stage(j + 2, S, (B + 2) % kBufs);
    load_stage(bid, j + 4, S);  // past the last step: harmless re-reads
    bid = block_id(j + 5);
    if (active(j)) {  // later steps are inactive too: nothing is left to do
      const float neg_m = softmax_head(j, st_cur);
      uint32_t pw[8];
#pragma unroll
      for (int i = 0; i < 16; ++i) st_next[i] = 0.f;
#pragma unroll
      for (int s = 0; s < kPD / 16; ++s) {
        score_mfma(st_next, (B + 1) % kBufs, s);  // step j+1 (unused if it is inactive)
        const float p0 = prob(st_cur, 2 * s, neg_m), p1 = prob(st_cur, 2 * s + 1, neg_m);
        l_part += p0 + p1;
        pw[s] = pk_bf16(p0, p1);
      }
      pv(pw, v_lds(B));
    }
  };
  for (int j = 0;; j += kBufs) {
    iteration(Buf<0>{}, j, sa, st_a, st_b);
    if (j + 1 >= nsteps) break;
    iteration(Buf<1>{}, j + 1, sb, st_b, st_a);
    if (j + 2 >= nsteps) break;
    iteration(Buf<2>{}, j + 2, sa, st_a, st_b);
    if (j + 3 >= nsteps) break;
    iteration(Buf<3>{}, j + 3, sb, st_b, st_a);
    if (j + 4 >= nsteps) break;
  }
  __syncthreads();  // the buffers become the merge area
  // Merge the key halves: half kh finishes output dims 64 kh .. 64 kh + 63
  // (accumulator tiles 2 kh and 2 kh + 1) and hands the other half its
  // other two tiles, with its reference and sum.
  float* mo_lds = (float*)lds;                                  // [kh][rg][kPD/4][kWave]
  float* mm_lds = mo_lds + 2 * kRowGroups * (kPD / 4) * kWave;  // [kh][rg][kWave]
  float* ml_lds = mm_lds + 2 * kRowGroups * kWave;              // [kh][rg][kWave]
  const int me = kh * kRowGroups + rg, other = (1 - kh) * kRowGroups + rg;
  mm_lds[me * kWave + lane] = m_ref;
  ml_lds[me * kWave + lane] = l_part;
  f32x16 keep[2];
  auto trade = [&](auto half_index) {
    constexpr int K = decltype(half_index)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        mo_lds[(me * (kPD / 4) + 16 * u + i) * kWave + lane] = oacc[2 * (1 - K) + u][i];
      keep[u] = oacc[2 * K + u];
    }
  };
  if (kh == 0) trade(Buf<0>{});
  else trade(Buf<1>{});
  __syncthreads();
  float m_tot;  // the reference the merged state is relative to (-inf: no key)
  {
    const float m1 = mm_lds[other * kWave + lane], l1 = ml_lds[other * kWave + lane];
    const float M = fmaxf(m_ref, m1);
    const float mu = M == -INFINITY ? 0.f : M;
    const float f0 = fast_exp2(m_ref - mu), f1 = fast_exp2(m1 - mu);
    l_part = l_part * f0 + l1 * f1;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        keep[u][i] = keep[u][i] * f0 + mo_lds[(other * (kPD / 4) + 16 * u + i) * kWave + lane] * f1;
    m_tot = M;
  }
  // The two halves of the wave hold the same rows' other keys.
  const float l_tot = l_part + __shfl_xor(l_part, 32, kWave);

  // The finished tile goes to LDS as rows (row-major, kTileStride bytes per
  // row), then every thread stores whole 16-byte pieces of rows.
  // An output is scaled by v_scale / sum; a prefix split's state by
  // 1 / sum (the merge applies v_scale once, to the merged output).
  uint8_t* tile_lds = lds + kTileOff;
  const float inv = l_tot > 0.f ? (kPrefix ? 1.f : v_scale) / l_tot : 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 64 * kh + 32 * u + q4 * 8 + 4 * half;
      const float x0 = keep[u][4 * q4 + 0], x1 = keep[u][4 * q4 + 1];
      const float x2 = keep[u][4 * q4 + 2], x3 = keep[u][4 * q4 + 3];
      *(u32x2*)(tile_lds + row * kTileStride + d0 * 2) =
          u32x2{pk_bf16(x0 * inv, x1 * inv), pk_bf16(x2 * inv, x3 * inv)};
    }
  if constexpr (kPrefix) {
    if (kh == 0 && half == 0 && row_ok) {
      const int64_t st = ((int64_t)c * n + qi) * num_heads + hq;
      ps.ml[2 * st + 0] = m_tot;
      ps.ml[2 * st + 1] = l_tot;
    }
  }
  __syncthreads();
  constexpr int kRowPieces = kPD * 2 / 16;  // 16-byte pieces per row
  uint16_t* const dst = kPrefix ? ps.o + (int64_t)c * n * num_heads * kPD : (uint16_t*)out;
#pragma unroll
  for (int k = 0; k < kRows * kRowPieces / kPThreads; ++k) {
    const int f = t + k * kPThreads, r = f / kRowPieces, piece = f % kRowPieces;
    const int rq = q_first + r / G;
    if (rq >= n) continue;
    const int64_t grow = (int64_t)(qs + rq) * num_heads + g * G + r % G;
    *(u32x4*)(dst + grow * kPD + 8 * piece) =
        *(const u32x4*)(tile_lds + r * kTileStride + piece * 16);
  }
}

// The prefix mode: a.num_tokens queries (one per sequence) against
// a.prefix.prefix_len keys of table row 0, in a.prefix splits.
template <typename KV, int BS, int G>
static hipError_t launch_prefix(const PrefillArgs& a) {
  const float k_scale = std::is_same<KV, FP8>::value ? a.k_scale : 1.0f;
  const float qk = a.scale * k_scale * kPLog2e;
  const int tiles = (a.num_tokens * G + kRows - 1) / kRows;
  const int splits = (a.prefix.prefix_len + a.prefix.split_len - 1) / a.prefix.split_len;
  if (tiles == 0 || splits == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<KV, BS, G, true>),
                     dim3((unsigned)tiles, (unsigned)a.num_kv_heads, (unsigned)splits),
                     dim3(kPThreads), 0, a.stream, a.out, a.query, a.query_start_loc,
                     a.k_cache, a.v_cache, a.block_tables, a.max_blocks_per_seq, a.seq_lens,
                     a.num_kv_heads, qk == 0.f ? 1.f : fabsf(qk),
                     qk == 0.f ? kQZero : (qk < 0.f ? kQNegate : kQAsIs), 1.0f,
                     PrefixStates{a.prefix.o, a.prefix.ml, a.num_tokens, a.prefix.split_len,
                                  a.prefix.prefix_len});
  return hipGetLastError();
}

template <typename KV, int BS, int G>
static hipError_t launch_prefill(const PrefillArgs& a) {
  if (a.prefix.o) return launch_prefix<KV, BS, G>(a);
  const float k_scale = std::is_same<KV, FP8>::value ? a.k_scale : 1.0f;
  const float v_scale = std::is_same<KV, FP8>::value ? a.v_scale : 1.0f;
  // The kernel takes a positive score scale (see kQNegate, kQZero).
  const float qk = a.scale * k_scale * kPLog2e;
  const int tiles = (a.max_query_len * G + kRows - 1) / kRows;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<KV, BS, G, false>),
                     dim3((unsigned)tiles, (unsigned)a.num_kv_heads, (unsigned)a.num_chunks),
                     dim3(kPThreads), 0, a.stream, a.out, a.query, a.query_start_loc,
                     a.k_cache, a.v_cache, a.block_tables, a.max_blocks_per_seq, a.seq_lens,
                     a.num_kv_heads, qk == 0.f ? 1.f : fabsf(qk),
                     qk == 0.f ? kQZero : (qk < 0.f ? kQNegate : kQAsIs), v_scale,
                     PrefixStates{});
  return hipGetLastError();
}

template <typename KV, int BS>
static hipError_t prefill_group(const PrefillArgs& a) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_prefill<KV, BS, 1>(a);
    case 2: return launch_prefill<KV, BS, 2>(a);
    case 4: return launch_prefill<KV, BS, 4>(a);
    case 8: return launch_prefill<KV, BS, 8>(a);
    default: return kNotInstantiated;
  }
}

template <typename KV>
static hipError_t prefill_block(const PrefillArgs& a) {
  switch (a.block_size) {
    case 16: return prefill_group<KV, 16>(a);
    case 32: return prefill_group<KV, 32>(a);
    case 64: return prefill_group<KV, 64>(a);
    case 128: return prefill_group<KV, 128>(a);
    default: return kNotInstantiated;
  }
}

bool prefill_supported(int32_t q_dtype, int32_t cache_dtype, int head_size, int block_size,
                       int group) {
  return q_dtype == PA_BF16 && (cache_dtype == PA_BF16 || cache_dtype == PA_FP8_E4M3) &&
         head_size == kPD &&
         (block_size == 16 || block_size == 32 || block_size == 64 || block_size == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t prefill(const PrefillArgs& a) {
  if (a.cache_dtype == PA_BF16) return prefill_block<BF16>(a);
  return prefill_block<FP8>(a);
}

}  // namespace pa
