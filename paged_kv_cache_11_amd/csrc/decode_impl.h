// decode_impl.h — the paged decode kernel and the split-K log-sum-exp merge.
//
// What it computes ("vLLM：大语言模型推理与服务库" §4.4 item 3): for every
// sequence s and query head h, walk the physical blocks of s through its
// block table, score q·k for every cached token, take the softmax and weight
// V.  The grid has the partition axis the openeuler.csdn.net essay describes
// ("PagedAttention：把操作系统的分页搬上 GPU": one workgroup per head group,
// sequence and partition of the context), re-cut for gfx950:
//
//   * one workgroup = one (partition, KV head, sequence) with 1, 2 or 4
//     wavefronts that take the partition's blocks round-robin; all
//     G = Hq/Hkv query heads of the group share every K/V byte read;
//   * a (block, KV head) tile is contiguous in the pool, so a wavefront
//     reads it with NLOAD fully coalesced loads (16 bytes per lane, 8 for an
//     fp8 cache, so a lane always holds 8 dims of a bf16/fp8 row) straight
//     into VGPRs, one tile ahead of the one being computed (ping-pong
//     register buffers);
//   * one token row occupies LPR = 4, 8 or 16 lanes, i.e. sits inside a DPP
//     row.  A tile is processed in chunks of SUB loads; with 16-lane rows the
//     G x SUB partial dot products of a lane (16 of them) are
//     reduce-scattered over the row in 4 DPP steps, so every lane ends with
//     one whole score per chunk and the softmax runs once per score;
//     probabilities return to the row with row_newbcast.  With shorter rows
//     the partials are all-reduced instead;
//   * the softmax is online, in fp32, in the log2 domain (v_exp_f32); each
//     token row keeps its own reference maximum per head and rescales its
//     accumulators only when a score exceeds that reference by more than
//     2^8 — exact, because the sum and the accumulators share the reference;
//   * fp8 codes are widened exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8,
//     scale 1; the per-tensor scales are applied to q·k and to the output),
//     so bf16 and fp8 caches share one datapath: q·k by v_dot2_f32_bf16
//     against the packed bf16 query, P·V pairing two tokens per
//     v_dot2_f32_bf16 (P rounded to bf16, accumulation in fp32); an f32
//     cache uses fp32 FMAs;
//   * rows, then wavefronts (through LDS), are merged once per partition;
//     with several partitions a second kernel merges their
//     (max, sum, normalised output) triples with log-sum-exp weights.
#pragma once

#include <utility>

#include "pa_internal.h"

namespace pa {

constexpr int kMaxDecodeWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units a score may exceed the reference by

// Bytes each lane loads per wavefront load: 16 (one dwordx4), except fp8
// caches, whose lanes take 8 bytes so a lane always holds 8 dims of a token
// row (the query and accumulator registers for a GQA group of 8 stay small).
template <typename KV> struct LaneBytes { static constexpr int value = 16; };
template <> struct LaneBytes<FP8> { static constexpr int value = 8; };

template <typename KV, int D, int BS, int G>
struct Geom {
  static constexpr int EB = Elem<KV>::bytes;
  static constexpr int LB = LaneBytes<KV>::value;  // bytes per lane per load
  static constexpr int LW = LB / 4;                // dwords per lane per load
  static constexpr int EPL = LB / EB;              // elements per lane per load
  static constexpr int LPR = D / EPL;              // lanes per token row
  static constexpr int RPL = kWave / LPR;          // token rows per wavefront load
  static constexpr int NLOAD = BS / RPL;           // loads per (block, head) tile
  // Loads handled together: enough for 16 partial scores per lane when a
  // token row fills a DPP row (then reduce-scattered to one score per lane
  // per 16), else the whole tile (all-reduced).
  static constexpr int SUB0 = LPR == 16 ? (16 / G > 2 ? 16 / G : 2) : NLOAD;
  static constexpr int SUB = SUB0 < NLOAD ? SUB0 : NLOAD;
  static constexpr int NCHUNK = NLOAD / SUB;
  static constexpr int N = SUB * G;                // partial scores per lane per chunk
  static constexpr bool kScatter = LPR == 16 && N % 16 == 0;
  static constexpr int NV = kScatter ? N / 16 : N;  // whole scores per lane per chunk
  static constexpr int64_t TILE_BYTES = (int64_t)BS * D * EB;
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "a token row must fit a DPP row");
  static_assert(NLOAD >= 1 && BS % RPL == 0, "a tile must be whole wavefront loads");
  static_assert(NLOAD % SUB == 0, "chunks must tile the loads");
};

template <int... Is, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

constexpr int rev4(int x) { return ((x & 1) << 3) | ((x & 2) << 1) | ((x & 4) >> 1) | ((x & 8) >> 3); }
constexpr int kRowNewBcast = 0x150;  // row_newbcast:k, k = 0..15

template <int K>
__device__ __forceinline__ float bcast16(float x) {
  return u2f((uint32_t)__builtin_amdgcn_mov_dpp((int)f2u(x), kRowNewBcast + K, 0xF, 0xF, false));
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<kQuadXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<kQuadXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kRowHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kRowMirror>(x));
  return x;
}
template <int N>
__device__ __forceinline__ float group_add(float x) {
  if constexpr (N == 1) return x;
  else if constexpr (N == 2) return x + dpp<kQuadXor1>(x);
  else return group_sum<N>(x);
}

// One reduce-scatter step: the lane keeps the half of each pair picked by
// its bit and adds the partner's copy of that half (the partner sends the
// other half it does not keep).
template <int CTRL>
__device__ __forceinline__ float rs_pair(float x0, float x1, bool bit) {
  const float keep = bit ? x1 : x0;
  const float send = bit ? x0 : x1;
  return keep + dpp<CTRL>(send);
}

// Reduce-scatter N partial sums over a 16-lane DPP row: afterwards lane l
// holds r[j] = full sum of v[16 j + rev4(l & 15)].
template <int N>
__device__ __forceinline__ void reduce_scatter16(const float (&v)[N], float (&r)[N / 16], int lane) {
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
  float a[N / 2], b[N / 4], c[N / 8];
#pragma unroll
  for (int j = 0; j < N / 2; ++j) a[j] = rs_pair<kRowMirror>(v[2 * j], v[2 * j + 1], b3);
#pragma unroll
  for (int j = 0; j < N / 4; ++j) b[j] = rs_pair<kRowHalfMirror>(a[2 * j], a[2 * j + 1], b2);
#pragma unroll
  for (int j = 0; j < N / 8; ++j) c[j] = rs_pair<kQuadXor2>(b[2 * j], b[2 * j + 1], b1);
#pragma unroll
  for (int j = 0; j < N / 16; ++j) r[j] = rs_pair<kQuadXor1>(c[2 * j], c[2 * j + 1], b0);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Query registers of one lane: its EPL dims of each of the G heads.  With a
// bf16 or fp8 cache the bf16 query stays packed for v_dot2_f32_bf16 (the
// cache words are widened to bf16 first); with an f32 cache it is fp32.
template <typename KV, typename QT, int G, int EPL>
struct QRegs {
  static constexpr bool kPacked = !std::is_same<KV, F32>::value;
  static_assert(!kPacked || (EPL == 8 && std::is_same<QT, BF16>::value),
                "packed queries are 8 bf16 per lane");
  uint32_t w[kPacked ? G : 1][4];
  float f[kPacked ? 1 : G][kPacked ? 1 : EPL];

  __device__ __forceinline__ void load(const void* query, int64_t row0, int D, int col) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t e0 = (row0 + h) * D + (int64_t)col * EPL;
      if constexpr (kPacked) {
        const u32x4 v = *(const u32x4*)((const uint16_t*)query + e0);
        w[h][0] = v.x; w[h][1] = v.y; w[h][2] = v.z; w[h][3] = v.w;
      } else {
        static_assert(std::is_same<QT, F32>::value && EPL == 4, "f32 cache, f32 queries");
        const u32x4 v = *(const u32x4*)((const float*)query + e0);
        Vec<F32>::to_f32(v, f[h]);
      }
    }
  }

  // Partial q·k over this lane's EPL dims for head h: kw holds the key as 4
  // packed bf16 dwords (packed path) or its 4 fp32 values' bits.
  __device__ __forceinline__ float dot(int h, const uint32_t (&kw)[4]) const {
    if constexpr (kPacked) {
      float a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw[0]), as_bf16x2(w[h][0]), 0.f, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw[1]), as_bf16x2(w[h][1]), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw[2]), as_bf16x2(w[h][2]), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw[3]), as_bf16x2(w[h][3]), a, false);
      return a;
    } else {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) a = __builtin_fmaf(f[h][e], u2f(kw[e]), a);
      return a;
    }
  }
};

// One lane's load of a cache tile as 4 dwords of the form the math uses:
// bf16 words as stored; fp8 codes widened exactly to 8 bf16 (gfx950's scaled
// convert with scale 1); f32 words as stored.
template <typename KV>
__device__ __forceinline__ void widen(const uint32_t* src, uint32_t (&o)[4]) {
  if constexpr (std::is_same<KV, FP8>::value) {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[0], 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[0], 1.0f, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[1], 1.0f, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[1], 1.0f, true));
  } else {
    o[0] = src[0]; o[1] = src[1]; o[2] = src[2]; o[3] = src[3];
  }
}

template <typename OT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (std::is_same<OT, F32>::value) ((float*)out)[idx] = v;
  else ((uint16_t*)out)[idx] = f32_to_bf16_rne(v);
}

// Per-wavefront attention state of one (sequence, KV head) over a run of
// blocks: the lane geometry, the query registers, the online-softmax state
// and the per-block update.
template <typename KV, typename QT, int D, int BS, int G>
struct WaveAttn {
  using GM = Geom<KV, D, BS, G>;
  static constexpr int EPL = GM::EPL, LPR = GM::LPR, RPL = GM::RPL, NLOAD = GM::NLOAD;
  static constexpr int LW = GM::LW, SUB = GM::SUB, NCHUNK = GM::NCHUNK;
  static constexpr int N = GM::N, NV = GM::NV;
  static constexpr bool kScatter = GM::kScatter;

  int lane, col, row;
  float qk_scale_log2;
  QRegs<KV, QT, G, EPL> q;
  // m_ref[h]: the row's reference maximum for head h (uniform over the
  // row).  Scatter layout: every score of a lane belongs to head
  // rev4(lane) % G; lane_ref is that head's reference and l_lane the lane's
  // share of its probability sum.  All-reduce layout: l_row[h], row-uniform.
  float m_ref[G], acc[G][EPL];
  float lane_ref, l_lane;
  float l_row[kScatter ? 1 : G];

  __device__ __forceinline__ void init(int lane_, float qk) {
    lane = lane_;
    col = lane % LPR;
    row = lane / LPR;
    qk_scale_log2 = qk;
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m_ref[h] = -INFINITY;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }
    lane_ref = -INFINITY;
    l_lane = 0.f;
#pragma unroll
    for (int h = 0; h < (kScatter ? 1 : G); ++h) l_row[h] = 0.f;
  }

  // P·V for one chunk: pb[i*G + h] is the probability of the chunk's token
  // row i, head h; vw[i] the widened V words of that row.
  __device__ __forceinline__ void accumulate_pv(const float (&pb)[N], const uint32_t (&vw)[SUB][4]) {
    if constexpr (!std::is_same<KV, F32>::value) {
#pragma unroll
      for (int k = 0; k < SUB / 2; ++k) {
        uint32_t vp[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          vp[2 * d] = __builtin_amdgcn_perm(vw[2 * k + 1][d], vw[2 * k][d], 0x05040100u);      // low halves
          vp[2 * d + 1] = __builtin_amdgcn_perm(vw[2 * k + 1][d], vw[2 * k][d], 0x07060302u);  // high halves
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const bf16x2 pp = as_bf16x2(pack_bf16(pb[(2 * k) * G + h], pb[(2 * k + 1) * G + h]));
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[h][e] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vp[e]), pp, acc[h][e], false);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < SUB; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = __builtin_fmaf(pb[i * G + h], u2f(vw[i][e]), acc[h][e]);
    }
  }

  // One chunk of a (block, KV head) tile: loads c*SUB .. c*SUB+SUB-1.
  template <bool kMasked>
  __device__ __forceinline__ void chunk(const uint32_t (&kt)[NLOAD][LW], const uint32_t (&vt)[NLOAD][LW],
                                        int c, int blk, int L) {
    float v[N];
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      uint32_t kw[4];
      widen<KV>(kt[c * SUB + i], kw);
#pragma unroll
      for (int h = 0; h < G; ++h) v[i * G + h] = q.dot(h, kw);
    }
    auto tok = [&](int i) { return blk * BS + row + (c * SUB + i) * RPL; };
    float pb[N];
    if constexpr (kScatter) {
      float r[NV];
      reduce_scatter16<N>(v, r, lane);
      const int cl = rev4(lane & 15);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        r[j] *= qk_scale_log2;
        if constexpr (kMasked) {
          if (tok((16 * j + cl) / G) >= L) r[j] = -INFINITY;
        }
      }
      bool ex = false;
#pragma unroll
      for (int j = 0; j < NV; ++j) ex |= r[j] > lane_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(ex)) {
        // Raise the row's references: per-head row maxima, broadcast.
        float lm = r[0];
#pragma unroll
        for (int j = 1; j < NV; ++j) lm = fmaxf(lm, r[j]);
        lm = group_max<16 / G>(lm);
        const float own_new = fmaxf(lane_ref, lm);
        l_lane *= own_new == -INFINITY ? 1.f : fast_exp2(lane_ref - own_new);
        lane_ref = own_new;
        static_for<G>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          const float mn = fmaxf(m_ref[h], bcast16<rev4(h)>(lm));
          const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m_ref[h] - mn);
          m_ref[h] = mn;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        });
      }
      float p[NV];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        p[j] = fast_exp2(r[j] - lane_ref);
        if constexpr (kMasked) p[j] = r[j] == -INFINITY ? 0.f : p[j];
        l_lane += p[j];
      }
      static_for<N>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        pb[n] = bcast16<rev4(n % 16)>(p[n / 16]);
      });
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) {
        v[n] = group_sum<LPR>(v[n]) * qk_scale_log2;
        if constexpr (kMasked) {
          if (tok(n / G) >= L) v[n] = -INFINITY;
        }
      }
      bool ex = false;
#pragma unroll
      for (int n = 0; n < N; ++n) ex |= v[n] > m_ref[n % G] + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(ex)) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float rm = v[h];
#pragma unroll
          for (int i = 1; i < SUB; ++i) rm = fmaxf(rm, v[i * G + h]);
          const float mn = fmaxf(m_ref[h], rm);
          const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m_ref[h] - mn);
          m_ref[h] = mn;
          l_row[h] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        }
      }
#pragma unroll
      for (int n = 0; n < N; ++n) {
        float p = fast_exp2(v[n] - m_ref[n % G]);
        if constexpr (kMasked) p = v[n] == -INFINITY ? 0.f : p;
        pb[n] = p;
        l_row[n % G] += p;
      }
    }
    uint32_t vw[SUB][4];
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      widen<KV>(vt[c * SUB + i], vw[i]);
      if constexpr (kMasked) {  // padding slots of the last block may hold anything
        const bool valid = tok(i) < L;
#pragma unroll
        for (int d = 0; d < 4; ++d) vw[i][d] = valid ? vw[i][d] : 0u;
      }
    }
    accumulate_pv(pb, vw);
  }

  // One (block, KV head) tile, chunk by chunk.  kMasked: the sequence's
  // last block, whose slots at or past L are padding.
  template <bool kMasked>
  __device__ __forceinline__ void block(const uint32_t (&kt)[NLOAD][LW], const uint32_t (&vt)[NLOAD][LW],
                                        int blk, int L) {
#pragma unroll
    for (int c = 0; c < NCHUNK; ++c) chunk<kMasked>(kt, vt, c, blk, L);
  }

  // Streams blocks first, first+stride, ... (count of them) of a sequence of
  // L tokens for KV head g through the pipeline: each tile's loads are
  // issued one tile ahead of its computation (ping-pong registers).  The
  // sequence's last block, if partly filled and in the run, comes last.
  // Blocks here are BS-token tiles: a pool block of 2^sub_shift x BS tokens
  // (64 or 128) holds 2^sub_shift consecutive ones (the (block, head) tile
  // of the pool is contiguous), found through table entry index >> sub_shift.
  // NT: K/V lines are read once in this call (see kv_load).
  template <bool NT>
  __device__ __forceinline__ void stream(const void* k_cache, const void* v_cache,
                                         const int32_t* tbl, int g, int num_kv_heads, int first,
                                         int count, int stride, int L, int sub_shift) {
    if (count <= 0) return;
    const int nblk = (L + BS - 1) / BS;
    const bool last_partial = (L % BS) != 0 && first + stride * (count - 1) == nblk - 1;
    const int nfull = count - (last_partial ? 1 : 0);
    const int sub_mask = (1 << sub_shift) - 1;
    const int64_t head_bytes = GM::TILE_BYTES << sub_shift;  // one pool block of one head
    const int64_t block_bytes = (int64_t)num_kv_heads * head_bytes;
    const uint8_t* kbase = (const uint8_t*)k_cache + (int64_t)g * head_bytes + lane * GM::LB;
    const uint8_t* vbase = (const uint8_t*)v_cache + (int64_t)g * head_bytes + lane * GM::LB;
    // Pool block ids of the run, 64 at a time, one per lane.
    int bid_v = 0;
    auto block_id = [&](int j) -> int {
      if ((j & (kWave - 1)) == 0) {
        const int jj = j + lane;
        bid_v = jj < count ? tbl[(first + stride * jj) >> sub_shift] : 0;
        // Wait for the window here, where it is (re)loaded once per 64
        // blocks, so that the read below never waits for the tile loads.
        asm volatile("" : "+v"(bid_v));
      }
      return __builtin_amdgcn_readlane(bid_v, j & (kWave - 1));
    };
    auto blk_of = [&](int j) { return first + stride * j; };
    auto load_tile = [&](int bid, int j, uint32_t (&kt)[NLOAD][LW], uint32_t (&vt)[NLOAD][LW]) {
      const int64_t off = (int64_t)bid * block_bytes + (int64_t)(blk_of(j) & sub_mask) * GM::TILE_BYTES;
      const uint8_t* kp = kbase + off;
      const uint8_t* vp = vbase + off;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        if constexpr (LW == 4) {
          const u32x4 x = kv_load<NT>((const u32x4*)(kp + i * kWave * GM::LB));
          kt[i][0] = x.x; kt[i][1] = x.y; kt[i][2] = x.z; kt[i][3] = x.w;
        } else {
          const u32x2 x = kv_load<NT>((const u32x2*)(kp + i * kWave * GM::LB));
          kt[i][0] = x.x; kt[i][1] = x.y;
        }
      }
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        if constexpr (LW == 4) {
          const u32x4 x = kv_load<NT>((const u32x4*)(vp + i * kWave * GM::LB));
          vt[i][0] = x.x; vt[i][1] = x.y; vt[i][2] = x.z; vt[i][3] = x.w;
        } else {
          const u32x2 x = kv_load<NT>((const u32x2*)(vp + i * kWave * GM::LB));
          vt[i][0] = x.x; vt[i][1] = x.y;
        }
      }
    };
    if (nfull > 0) {
      uint32_t ka[NLOAD][LW], va[NLOAD][LW], kb[NLOAD][LW], vb[NLOAD][LW];
      load_tile(block_id(0), 0, ka, va);
      int j = 0;
      for (; j + 2 < nfull; j += 2) {
        load_tile(block_id(j + 1), j + 1, kb, vb);
        block<false>(ka, va, blk_of(j), L);
        load_tile(block_id(j + 2), j + 2, ka, va);
        block<false>(kb, vb, blk_of(j + 1), L);
      }
      if (nfull - j == 2) {
        load_tile(block_id(j + 1), j + 1, kb, vb);
        block<false>(ka, va, blk_of(j), L);
        block<false>(kb, vb, blk_of(j + 1), L);
      } else {
        block<false>(ka, va, blk_of(j), L);
      }
    }
    if (last_partial) {
      uint32_t kt[NLOAD][LW], vt[NLOAD][LW];
      load_tile(block_id(count - 1), count - 1, kt, vt);
      block<true>(kt, vt, blk_of(count - 1), L);
    }
  }

  // Sums per row and merges the token rows of the wavefront: afterwards
  // every lane holds, for its col, the wavefront's (m_ref, l_h, acc).
  __device__ __forceinline__ void merge_rows(float (&l_h)[G]) {
    if constexpr (kScatter) {
      const float lg = group_add<16 / G>(l_lane);
      static_for<G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        l_h[h] = bcast16<rev4(h)>(lg);
      });
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) l_h[h] = l_row[h];
    }
#pragma unroll
    for (int mask = LPR; mask < kWave; mask <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mo = shfl_xor(m_ref[h], mask);
        const float lo = shfl_xor(l_h[h], mask);
        const float M = fmaxf(m_ref[h], mo);
        const float mu = M == -INFINITY ? 0.f : M;
        const float f = fast_exp2(m_ref[h] - mu), fo = fast_exp2(mo - mu);
        l_h[h] = l_h[h] * f + lo * fo;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * f + shfl_xor(acc[h][e], mask) * fo;
        m_ref[h] = M;
      }
    }
  }
};

template <typename KV, typename QT, int D, int BS, int G>
__global__ __launch_bounds__(kMaxDecodeWaves * kWave) void decode_kernel(
    void* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
    const void* __restrict__ query, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, int max_blocks_per_seq, int num_kv_heads,
    int partition_blocks, int max_parts, float qk_scale_log2, float v_scale, int sub_shift,
    int read_once) {
  using WA = WaveAttn<KV, QT, D, BS, G>;
  constexpr int EPL = WA::EPL, RPL = WA::RPL;
  using OT = QT;

  const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int NW = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int num_heads = num_kv_heads * G;

  const int L = seq_lens[s];
  const int nblk = (L + BS - 1) / BS;
  const int pb = partition_blocks > 0 ? partition_blocks : (nblk > 0 ? nblk : 1);
  const int nparts = nblk > pb ? (nblk + pb - 1) / pb : 1;
  if (part >= nparts) return;
  const int b0 = part * pb;
  const int b1 = min(b0 + pb, nblk);

  WA A;
  A.init(lane, qk_scale_log2);
  A.reset();
  A.q.load(query, (int64_t)s * num_heads + (int64_t)g * G, D, A.col);
  const int span = b1 - b0;
  const int nmine = span > w ? (span - w + NW - 1) / NW : 0;
  if (read_once)
    A.template stream<true>(k_cache, v_cache, block_tables + (int64_t)s * max_blocks_per_seq, g,
                            num_kv_heads, b0 + w, nmine, NW, L, sub_shift);
  else
    A.template stream<false>(k_cache, v_cache, block_tables + (int64_t)s * max_blocks_per_seq, g,
                             num_kv_heads, b0 + w, nmine, NW, L, sub_shift);
  float l_h[G];
  A.merge_rows(l_h);

  const int64_t hq0 = (int64_t)s * num_heads + (int64_t)g * G;
  auto emit = [&](int h, int d, float M, float den, float num) {
    const float o = den > 0.f ? num / den * v_scale : 0.f;
    const int64_t hq = hq0 + h;
    if (nparts == 1) {
      store_out<OT>(out, hq * D + d, o);
    } else {
      part_o[(hq * max_parts + part) * D + d] = o;
      if (d == 0) {
        part_ml[(hq * max_parts + part) * 2 + 0] = M;
        part_ml[(hq * max_parts + part) * 2 + 1] = den;
      }
    }
  };

  if (NW == 1) {
    // Every row now holds the merged state; row r writes heads r, r+RPL, ...
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h % RPL != A.row) continue;
#pragma unroll
      for (int e = 0; e < EPL; ++e) emit(h, A.col * EPL + e, A.m_ref[h], l_h[h], A.acc[h][e]);
    }
    return;
  }

  // Merge the wavefronts through LDS and finish.
  __shared__ float sm_ml[kMaxDecodeWaves][G][2];
  __shared__ float sm_acc[kMaxDecodeWaves][G][D];
  if (A.row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[w][h][A.col * EPL + e] = A.acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { sm_ml[w][h][0] = A.m_ref[h]; sm_ml[w][h][1] = l_h[h]; }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int h = idx / D, d = idx % D;
    float M = sm_ml[0][h][0];
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm_ml[ww][h][0]);
    const float mu = M == -INFINITY ? 0.f : M;
    float den = 0.f, num = 0.f;
    for (int ww = 0; ww < NW; ++ww) {
      const float f = fast_exp2(sm_ml[ww][h][0] - mu);
      den += f * sm_ml[ww][h][1];
      num += f * sm_acc[ww][h][d];
    }
    emit(h, d, M, den, num);
  }
}

// ---------------------------------------------------------------------------
// Balanced split-K.  Per KV head g, the blocks of all sequences form one
// flattened list (sequence after sequence, T blocks in all); it is cut into
// W equal contiguous ranges, one per wavefront ("worker").  A worker walks
// its range sequence by sequence: a sequence it covers entirely is finished
// in place; a sequence cut between workers leaves one partial state per
// worker — at most two per worker, its first and its last piece — which the
// merge kernel combines.  Workers of the KV heads of one block range are
// adjacent, so the heads' tiles of a block (contiguous in the pool) are read
// together.
// ---------------------------------------------------------------------------
constexpr int kBalancedMinTokens = 256;  // fewest tokens a worker is given



__device__ __forceinline__ int nblocks_of(int L, int bs) { return (L + bs - 1) / bs; }

// Sequence lengths are read kScanChunks chunks of 64 (one per lane) at a
// time, all loads of a batch issued before any is used: a worker's start
// then costs one memory round trip per 1024 sequences, not one per 64.
constexpr int kScanChunks = 16;

// Lengths count from token `skip` of each sequence (0: the whole sequence;
// the suffix past a shared prefix otherwise).
__device__ __forceinline__ void load_len_batch(const int32_t* seq_lens, int num_seqs, int c0,
                                               int lane, int bs, int skip,
                                               int (&nb)[kScanChunks], int extra = 0) {
  // Every load is issued unconditionally (past the end it reads the last
  // length again, then ignores it): a load under a condition gets its own
  // wait, which would serialise the batch.
#pragma unroll
  for (int b = 0; b < kScanChunks; ++b) {
    const int s = c0 + b * kWave + lane;
    nb[b] = seq_lens[s < num_seqs ? s : num_seqs - 1];
  }
#pragma unroll
  for (int b = 0; b < kScanChunks; ++b) {
    const int s = c0 + b * kWave + lane;
    nb[b] = s < num_seqs && nb[b] > skip ? nb[b] - skip : 0;
  }
#pragma unroll
  for (int b = 0; b < kScanChunks; ++b) nb[b] = nb[b] > 0 ? nblocks_of(nb[b], bs) + extra : 0;
}

// Inclusive prefix sum over the wavefront's 64 lanes on DPP (row shifts
// within each 16-lane row, then the rows' last lanes broadcast forward):
// a few VALU cycles per step, where a lane shuffle is an LDS round trip.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_scan_incl(v), kWave - 1);
}

// Total blocks of all sequences (wavefront-uniform result).
__device__ __forceinline__ int64_t total_blocks(const int32_t* seq_lens, int num_seqs, int bs,
                                                int skip, int lane, int extra = 0) {
  int t = 0;  // per-lane partial sums stay far below 2^31
  for (int c0 = 0; c0 < num_seqs; c0 += kScanChunks * kWave) {
    int nb[kScanChunks];
    load_len_batch(seq_lens, num_seqs, c0, lane, bs, skip, nb, extra);
#pragma unroll
    for (int b = 0; b < kScanChunks; ++b) t += nb[b];
  }
  return wave_sum(t);
}

// The sequence whose blocks hold flattened position x, and the flattened
// position of its first block (wavefront-uniform).
__device__ __forceinline__ void locate_block(const int32_t* seq_lens, int num_seqs, int bs,
                                             int skip, int64_t x, int lane, int& s_out,
                                             int64_t& base_out, int extra = 0) {
  int64_t base = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += kScanChunks * kWave) {
    int nb[kScanChunks];
    load_len_batch(seq_lens, num_seqs, c0, lane, bs, skip, nb, extra);
#pragma unroll
    for (int b = 0; b < kScanChunks; ++b) {
      if (c0 + b * kWave >= num_seqs) break;
      const int incl = wave_scan_incl(nb[b]);
      const int chunk = __builtin_amdgcn_readlane(incl, kWave - 1);
      if (base + chunk > x) {
        const uint64_t found = __builtin_amdgcn_ballot_w64(base + incl > x);
        const int k = __builtin_ctzll(found);
        s_out = c0 + b * kWave + k;
        base_out = base + __builtin_amdgcn_readlane(incl - nb[b], k);
        return;
      }
      base += chunk;
    }
  }
  s_out = num_seqs;
  base_out = base;
}

// The same two questions from one load of every length, where they fit one
// batch (num_seqs <= kScanChunks * 64): raw[b] holds seq_lens[64 b + lane]
// (0 past num_seqs), from which the total and the located sequence follow
// with no second pass over memory.
__device__ __forceinline__ void load_all_lens(const int32_t* seq_lens, int num_seqs, int lane,
                                              int (&raw)[kScanChunks]) {
#pragma unroll
  for (int b = 0; b < kScanChunks; ++b) raw[b] = seq_lens[min(b * kWave + lane, num_seqs - 1)];
#pragma unroll
  for (int b = 0; b < kScanChunks; ++b) raw[b] = b * kWave + lane < num_seqs ? raw[b] : 0;
}

__device__ __forceinline__ int units_of(int len, int bs, int skip, int extra) {
  return len > skip ? nblocks_of(len - skip, bs) + extra : 0;
}

__device__ __forceinline__ int64_t total_blocks_of(const int (&raw)[kScanChunks], int bs, int skip,
                                                   int extra = 0) {
  int t = 0;
#pragma unroll
  for (int b = 0; b < kScanChunks; ++b) t += units_of(raw[b], bs, skip, extra);
  return wave_sum(t);
}

__device__ __forceinline__ void locate_block_of(const int (&raw)[kScanChunks], int num_seqs, int bs,
                                                int skip, int64_t x, int& s_out,
                                                int64_t& base_out, int extra = 0) {
  int64_t base = 0;
#pragma unroll
  for (int b = 0; b < kScanChunks; ++b) {
    if (b * kWave >= num_seqs) break;
    const int nb = units_of(raw[b], bs, skip, extra);
    const int incl = wave_scan_incl(nb);
    const int chunk = __builtin_amdgcn_readlane(incl, kWave - 1);
    if (base + chunk > x) {
      const uint64_t found = __builtin_amdgcn_ballot_w64(base + incl > x);
      const int k = __builtin_ctzll(found);
      s_out = b * kWave + k;
      base_out = base + __builtin_amdgcn_readlane(incl - nb, k);
      return;
    }
    base += chunk;
  }
  s_out = num_seqs;
  base_out = base;
}

// raw[b] for a wavefront-uniform b.
__device__ __forceinline__ int lens_chunk(const int (&raw)[kScanChunks], int b) {
  int v = 0;
#pragma unroll
  for (int i = 0; i < kScanChunks; ++i) v = i == b ? raw[i] : v;
  return v;
}

__device__ __forceinline__ int64_t worker_start(int64_t T, int v, int W) { return T * v / W; }

// The worker whose range holds flattened position x.
__device__ __forceinline__ int worker_of(int64_t T, int64_t x, int W) {
  return (int)(((x + 1) * W + T - 1) / T - 1);
}

// Workers actually used for T blocks of bs tokens: at most W, and none with
// fewer than kBalancedMinTokens tokens (rounded to whole blocks).
__device__ __forceinline__ int effective_workers(int64_t T, int W, int bs) {
  const int min_blocks = kBalancedMinTokens / bs > 1 ? kBalancedMinTokens / bs : 1;
  const int64_t want = (T + min_blocks - 1) / min_blocks;
  return (int)(want < W ? (want > 0 ? want : 1) : W);
}

// Online log-sum-exp merge, for one output element, of np partial states:
// state p has maximum m_p, sum l_p and accumulator a_p (normalised by l_p
// when kNormalised).  Returns sum_p 2^(m_p - M) a'_p / sum_p 2^(m_p - M) l_p
// with M = max_p m_p and a'_p the unnormalised accumulator.  The loads of
// sixteen states are issued together.
template <bool kNormalised, typename StateFn>
__device__ __forceinline__ float merge_element(const float* acc, const float* ml, int np, int D,
                                               int h, int d, StateFn state) {
  constexpr int kBatch = 16;
  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int p0 = 0; p0 < np; p0 += kBatch) {
    float m[kBatch], l[kBatch], a[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int p = p0 + q < np ? p0 + q : np - 1;
      const int64_t st = state(p, h);
      m[q] = ml[2 * st];
      l[q] = ml[2 * st + 1];
      a[q] = acc[st * D + d];
    }
    // One rescale per batch: raise M to the batch maximum first.
    float bm = -INFINITY;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) bm = p0 + q < np ? fmaxf(bm, m[q]) : bm;
    if (bm > M) {
      const float f = M == -INFINITY ? 0.f : fast_exp2(M - bm);
      num *= f;
      den *= f;
      M = bm;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const float e = (p0 + q >= np || M == -INFINITY) ? 0.f : fast_exp2(m[q] - M);
      num = __builtin_fmaf(e * (kNormalised ? l[q] : 1.f), a[q], num);
      den = __builtin_fmaf(e, l[q], den);
    }
  }
  return den > 0.f ? num / den : 0.f;
}

template <typename KV, typename QT, int D, int BS, int G>
__global__ __launch_bounds__(kMaxDecodeWaves * kWave) void decode_balanced_kernel(
    void* __restrict__ out, float* __restrict__ part_acc, float* __restrict__ part_ml,
    int32_t* __restrict__ merges, int32_t* __restrict__ cuts, const void* __restrict__ query,
    const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens, int num_seqs,
    int max_blocks_per_seq, int num_kv_heads, int workers_per_head, float qk_scale_log2,
    float v_scale, int sub_shift, int read_once_hint, SuffixStates sx) {
  using WA = WaveAttn<KV, QT, D, BS, G>;
  constexpr int EPL = WA::EPL, RPL = WA::RPL;
  using OT = QT;
  const int lane = threadIdx.x & (kWave - 1);
  const int worker = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int g = worker % num_kv_heads, vw = worker / num_kv_heads;
  if (vw >= workers_per_head) return;
  const int num_heads = num_kv_heads * G;

  const int64_t T = total_blocks(seq_lens, num_seqs, BS, sx.skip, lane);
  const int W = effective_workers(T, workers_per_head, BS);
  // The caller declared that no block is read twice: evict-first loads.
  const bool read_once = read_once_hint != 0;
  int32_t* merge = merges + 2 * (int64_t)worker;
  if (lane == 0) merge[0] = -1;  // no merge task unless the last run sets one
  if (vw >= W) return;
  const int64_t start = worker_start(T, vw, W), end = worker_start(T, vw + 1, W);
  if (start >= end) return;
  int s;
  int64_t base;
  locate_block(seq_lens, num_seqs, BS, sx.skip, start, lane, s, base);
  // With a skip, the table row starts at the first block past it.
  const int tbl_skip = sx.skip / (BS << sub_shift);

  WA A;
  A.init(lane, qk_scale_log2);
  int64_t pos = start;
  while (pos < end && s < num_seqs) {
    const int L = max(seq_lens[s] - sx.skip, 0);
    const int nblk = nblocks_of(L, BS);
    const int64_t seg_end = base + nblk;
    if (nblk > 0) {
      const int b_lo = (int)(pos - base);
      const int b_hi = (int)((end < seg_end ? end : seg_end) - base);
      A.reset();
      A.q.load(query, (int64_t)s * num_heads + (int64_t)g * G, D, A.col);
      const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq + tbl_skip;
      if (read_once)
        A.template stream<true>(k_cache, v_cache, row, g, num_kv_heads, b_lo, b_hi - b_lo, 1, L,
                                sub_shift);
      else
        A.template stream<false>(k_cache, v_cache, row, g, num_kv_heads, b_lo, b_hi - b_lo, 1, L,
                                 sub_shift);
      float l_h[G];
      A.merge_rows(l_h);
      const bool whole = b_lo == 0 && b_hi == nblk;
      const int slot = pos == start ? 0 : 1;
      const int64_t hq0 = (int64_t)s * num_heads + (int64_t)g * G;
      if (b_lo == 0 && lane == 0) {
        // The worker holding the sequence's first unit records how it is
        // cut (first worker, 2 * pieces + first slot) per sequence, and, if
        // it is cut, as this worker's merge task.
        const int code = (whole ? 1 : worker_of(T, seg_end - 1, W) - vw + 1) * 2 + slot;
        cuts[2 * ((int64_t)s * num_kv_heads + g) + 0] = vw;
        cuts[2 * ((int64_t)s * num_kv_heads + g) + 1] = code;
        if (!whole) {
          merge[0] = s;
          merge[1] = code;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (h % RPL != A.row) continue;
        if (whole && !sx.acc) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            const float o = l_h[h] > 0.f ? A.acc[h][e] / l_h[h] * v_scale : 0.f;
            store_out<OT>(out, (hq0 + h) * D + A.col * EPL + e, o);
          }
        } else {
          // A piece of a cut sequence, or (suffix states kept) a whole one.
          const int64_t pslot = whole ? hq0 + h : ((int64_t)worker * 2 + slot) * G + h;
          float* dacc = whole ? sx.acc : part_acc;
          float* dml = whole ? sx.ml : part_ml;
#pragma unroll
          for (int e = 0; e < EPL; ++e) dacc[pslot * D + A.col * EPL + e] = A.acc[h][e];
          if (A.col == 0) {
            dml[pslot * 2 + 0] = A.m_ref[h];
            dml[pslot * 2 + 1] = l_h[h];
          }
        }
      }
      pos = base + b_hi;
    }
    if (pos >= seg_end) {
      base = seg_end;
      ++s;
    }
  }
}

// Finishes what the balanced kernels left.  The worker holding a
// sequence's first unit recorded how the sequence is cut: per sequence and
// KV head {first worker, 2 * pieces + slot}, and for a cut sequence the
// same as that worker's merge task {s, 2 * pieces + slot} (else -1).  A
// cut sequence is merged from its pieces' (m, l, acc): the first worker's
// (that slot) and slot 0 of each following worker.  A whole sequence was
// finished by its worker.  Two grids do the same merges, one element per
// thread: per (query head, KV head, sequence) when there are few
// sequences, per (query head, worker, KV head) when there are many — what
// a reduce costs is mostly the dispatch of its workgroups.

template <typename OT, int D, int G>
__device__ __forceinline__ void merge_cut(void* out, const float* part_acc, const float* part_ml,
                                          int s, int va, int code, int h, int g, int d,
                                          int num_kv_heads, float v_scale) {
  const int np = code >> 1, slot0 = code & 1;
  auto state = [&](int p, int hh) -> int64_t {
    return ((int64_t)((va + p) * num_kv_heads + g) * 2 + (p == 0 ? slot0 : 0)) * G + hh;
  };
  const float o = merge_element<false>(part_acc, part_ml, np, D, h, d, state);
  store_out<OT>(out, ((int64_t)s * num_kv_heads * G + g * G + h) * D + d, o * v_scale);
}

// Per (query head h, KV head g, sequence s); empty sequences get zeros.
template <typename OT, int D, int G>
__global__ __launch_bounds__(D) void balanced_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ part_acc,
    const float* __restrict__ part_ml, const int32_t* __restrict__ cuts,
    const int32_t* __restrict__ seq_lens, int num_kv_heads, float v_scale) {
  const int h = blockIdx.x, g = blockIdx.y, s = blockIdx.z, d = threadIdx.x;
  const int L = seq_lens[s];
  const int va = cuts[2 * ((int64_t)s * num_kv_heads + g) + 0];
  const int code = cuts[2 * ((int64_t)s * num_kv_heads + g) + 1];
  if (L == 0) {
    store_out<OT>(out, ((int64_t)s * num_kv_heads * G + g * G + h) * D + d, 0.f);
    return;
  }
  if ((code >> 1) <= 1) return;
  merge_cut<OT, D, G>(out, part_acc, part_ml, s, va, code, h, g, d, num_kv_heads, v_scale);
}

// Per (query head h, worker vw, KV head g): the worker's merge task, and
// zeros for the empty sequences among vw * D .. vw * D + D - 1 (+ the
// grid's multiples), one sequence per thread.
template <typename OT, int D, int G>
__global__ __launch_bounds__(D) void balanced_reduce_tasks_kernel(
    void* __restrict__ out, const float* __restrict__ part_acc,
    const float* __restrict__ part_ml, const int32_t* __restrict__ merges,
    const int32_t* __restrict__ seq_lens, int num_seqs, int num_kv_heads, float v_scale) {
  const int h = blockIdx.x, vw = blockIdx.y, g = blockIdx.z, d = threadIdx.x;
  const int32_t* task = merges + 2 * ((int64_t)vw * num_kv_heads + g);
  const int s = task[0], code = task[1];
  for (int e = vw * D + d; e < num_seqs; e += gridDim.y * D)
    if (seq_lens[e] == 0)
      for (int i = 0; i < D; ++i)
        store_out<OT>(out, ((int64_t)e * num_kv_heads * G + g * G + h) * D + i, 0.f);
  if (s < 0) return;
  merge_cut<OT, D, G>(out, part_acc, part_ml, s, vw, code, h, g, d, num_kv_heads, v_scale);
}

// The same merges with one wavefront per (sequence, KV head, group of H =
// min(G, 512 / D) heads), for D G >= 256: lane l merges D H / 64 consecutive
// outputs of head l / (64 / H) of the group from 16-byte state loads, the
// states of sixteen pieces (G = 8) or eight loaded together (one reference
// raise per batch), and writes them; empty sequences get zeros, whole ones were
// finished by their worker.  Far fewer workgroups than the kernels above,
// which take G D-thread workgroups per sequence and KV head.
constexpr int kReduceWaves = 4;

template <int D, int G>
struct ReduceShape {
  static constexpr int H = G * D > 512 ? 512 / D : G;  // heads per wavefront
  static constexpr int kGroups = G / H;                // wavefronts per (sequence, KV head)
};

template <typename OT, int D, int G>
__global__ __launch_bounds__(kReduceWaves * kWave) void balanced_reduce_wave_kernel(
    void* __restrict__ out, const float* __restrict__ part_acc,
    const float* __restrict__ part_ml, const int32_t* __restrict__ cuts,
    const int32_t* __restrict__ seq_lens, int num_seqs, int num_kv_heads, float v_scale) {
  constexpr int H = ReduceShape<D, G>::H, kGroups = ReduceShape<D, G>::kGroups;
  constexpr int kLanesPerHead = kWave / H, kDims = D / kLanesPerHead, kVecs = kDims / 4;
  constexpr int kBatch = G >= 8 ? 16 : 8;
  static_assert(kDims % 4 == 0, "whole 4-element groups per lane");
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = (int64_t)blockIdx.x * kReduceWaves +
                       __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  if (item >= (int64_t)num_seqs * num_kv_heads * kGroups) return;
  const int64_t sg = item / kGroups;  // (sequence, KV head)
  const int s = (int)(sg / num_kv_heads), g = (int)(sg % num_kv_heads);
  const int h = (int)(item % kGroups) * H + lane / kLanesPerHead;  // head within the group of G
  const int d0 = (lane % kLanesPerHead) * kDims;
  const int L = seq_lens[s];
  const int va = cuts[2 * sg + 0], code = cuts[2 * sg + 1];
  const int np = code >> 1, slot0 = code & 1;
  if (L > 0 && np <= 1) return;  // a whole sequence: finished by its worker
  float num[kVecs][4], den = 0.f, M = -INFINITY;
#pragma unroll
  for (int v = 0; v < kVecs; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) num[v][i] = 0.f;
  for (int p0 = 0; L > 0 && p0 < np; p0 += kBatch) {
    float m[kBatch], l[kBatch];
    f32x4 a[kBatch][kVecs];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int p = p0 + q < np ? p0 + q : np - 1;
      const int64_t st =
          ((int64_t)((va + p) * num_kv_heads + g) * 2 + (p == 0 ? slot0 : 0)) * G + h;
      m[q] = part_ml[2 * st];
      l[q] = part_ml[2 * st + 1];
#pragma unroll
      for (int v = 0; v < kVecs; ++v) a[q][v] = *(const f32x4*)(part_acc + st * D + d0 + 4 * v);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) bm = p0 + q < np ? fmaxf(bm, m[q]) : bm;
    if (bm > M) {
      const float f = M == -INFINITY ? 0.f : fast_exp2(M - bm);
#pragma unroll
      for (int v = 0; v < kVecs; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) num[v][i] *= f;
      den *= f;
      M = bm;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const float e = (p0 + q >= np || M == -INFINITY) ? 0.f : fast_exp2(m[q] - M);
#pragma unroll
      for (int v = 0; v < kVecs; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) num[v][i] = __builtin_fmaf(e, a[q][v][i], num[v][i]);
      den = __builtin_fmaf(e, l[q], den);
    }
  }
  // As merge_cut: num / den (0 when den is 0, as for an empty sequence)
  // times v_scale, rounded once.
  const int64_t o = ((int64_t)s * num_kv_heads * G + g * G + h) * D + d0;
#pragma unroll
  for (int v = 0; v < kVecs; ++v) {
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (den > 0.f ? num[v][i] / den : 0.f) * v_scale;
    if constexpr (std::is_same<OT, F32>::value) {
      *(f32x4*)((float*)out + o + 4 * v) = f32x4{x[0], x[1], x[2], x[3]};
    } else {
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16);
      *(u32x2*)((uint16_t*)out + o + 4 * v) = u32x2{w0, w1};
    }
  }
}

// The last step of a shared-prefix decode: the log-sum-exp merge of each
// sequence's suffix (its pieces when the balanced split cut it, else the
// whole-sequence state the suffix mode kept) with the prefix's splits.
// Every state has its own reference maximum (log2 domain) and exponent sum;
// the suffix's are unnormalised fp32 accumulators, the prefix splits'
// outputs normalised by their sums, in bf16.  A state with no keys has
// m = -inf and is skipped.
// Workgroups of kMergeThreads, grid (sequence, element block of
// 4 kMergeThreads outputs); a thread owns 4 consecutive output elements of
// one head (16-byte loads).  The prefix
// states, the cut records and the whole-sequence states do not depend on
// each other, so all their loads are issued before any is used; only the
// pieces of a cut sequence wait for its cut record.
constexpr int kMergeThreads = 256;

template <typename OT, int D, int G>
__global__ __launch_bounds__(kMergeThreads) void prefix_merge_kernel(
    void* __restrict__ out, const float* __restrict__ part_acc,
    const float* __restrict__ part_ml, const int32_t* __restrict__ cuts,
    const int32_t* __restrict__ seq_lens, int num_seqs, int num_kv_heads, float v_scale,
    SuffixStates sx, const uint16_t* __restrict__ prefix_o, const float* __restrict__ prefix_ml,
    int prefix_splits) {
  constexpr int kMaxSplits = kMaxPrefixSplits;
  const int s = blockIdx.x;
  const int num_heads = num_kv_heads * G;
  const bool has_suffix = seq_lens[s] > sx.skip;
  for (int e0 = (blockIdx.y * kMergeThreads + threadIdx.x) * 4; e0 < num_heads * D;
       e0 += gridDim.y * kMergeThreads * 4) {
    const int h = e0 / D, d = e0 % D;  // query head (of all num_heads) and first dim
    const int g = h / G, hg = h % G;
    const int64_t hq = (int64_t)s * num_heads + h;
    float M = -INFINITY, den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    // A state with its own sum l: an unnormalised accumulator a enters with
    // weight 2^(m - M), a normalised output (norm) with 2^(m - M) l.
    auto add = [&](float m, float l, f32x4 a, bool norm) {
      if (m == -INFINITY) return;
      if (m > M) {
        const float f = M == -INFINITY ? 0.f : fast_exp2(M - m);
        num *= f;
        den *= f;
        M = m;
      }
      const float e = fast_exp2(m - M);
      num += (norm ? e * l : e) * a;
      den = __builtin_fmaf(e, l, den);
    };
    // Every load that does not depend on another is issued up front (the
    // suffix words are read even for an empty suffix, whose slots hold
    // stale values that are then ignored), so the merge waits for at most
    // two rounds of memory latency: these, and the pieces of a cut suffix.
    const int va = cuts[2 * ((int64_t)s * num_kv_heads + g) + 0];
    const int code = cuts[2 * ((int64_t)s * num_kv_heads + g) + 1];
    const float wm = sx.ml[2 * hq];  // the whole-sequence state (used if not cut)
    const float wl = sx.ml[2 * hq + 1];
    const f32x4 wa = *(const f32x4*)(sx.acc + hq * D + d);
    float pm[kMaxSplits], pl[kMaxSplits];
    f32x4 pa[kMaxSplits];
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c) {
      if (c < prefix_splits) {
        const int64_t st = (int64_t)c * num_seqs * num_heads + hq;
        pm[c] = prefix_ml[2 * st];
        pl[c] = prefix_ml[2 * st + 1];
        pa[c] = bf16x4_to_f32x4(*(const u32x2*)(prefix_o + st * D + d));
      }
    }
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c)
      if (c < prefix_splits) add(pm[c], pl[c], pa[c], true);
    if (has_suffix) {
      const int np = code >> 1, slot0 = code & 1;
      if (np <= 1) {
        add(wm, wl, wa, false);
      } else {
        for (int p = 0; p < np; ++p) {
          const int64_t st =
              ((int64_t)((va + p) * num_kv_heads + g) * 2 + (p == 0 ? slot0 : 0)) * G + hg;
          add(part_ml[2 * st], part_ml[2 * st + 1], *(const f32x4*)(part_acc + st * D + d), false);
        }
      }
    }
    const float inv = den > 0.f ? v_scale / den : 0.f;
    if constexpr (std::is_same<OT, F32>::value) {
      *(f32x4*)((float*)out + hq * D + d) = num * inv;
    } else {
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(num[0] * inv) |
                          ((uint32_t)f32_to_bf16_rne(num[1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(num[2] * inv) |
                          ((uint32_t)f32_to_bf16_rne(num[3] * inv) << 16);
      *(u32x2*)((uint16_t*)out + hq * D + d) = u32x2{w0, w1};
    }
  }
}

// prefix_merge_kernel with one wavefront per (sequence, KV head), for
// D G >= 256 (the layout of balanced_reduce_wave_kernel): the cut record,
// the prefix splits' states and the suffix's states (its whole-sequence
// state, or the pieces of a cut suffix, which wait for the cut record only)
// are requested four at a time, the prefix's and the suffix's first four
// together, before any is used.
// kNorm: the states are outputs normalised by their own sum, in bf16 (the
// prefix splits); else unnormalised fp32 accumulators (the suffix pieces).
template <int D, int G, bool kNorm>
struct MergeBatch {
  static constexpr int kLanesPerHead = kWave / G, kDims = D / kLanesPerHead, kVecs = kDims / 4;
  static constexpr int kN = 4;
  using Acc = typename std::conditional<kNorm, uint16_t, float>::type;
  float m[kN], l[kN];
  f32x4 a[kN][kVecs];
  // States idx(0 .. n-1) from q0 on (at most kN; the rest repeat the last).
  template <typename IndexFn>
  __device__ __forceinline__ void load(const float* ml, const Acc* acc, int q0, int n, int d0,
                                       IndexFn idx) {
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int64_t st = idx(q0 + q < n ? q0 + q : n - 1);
      m[q] = ml[2 * st];
      l[q] = ml[2 * st + 1];
#pragma unroll
      for (int v = 0; v < kVecs; ++v) {
        if constexpr (kNorm)
          a[q][v] = bf16x4_to_f32x4(*(const u32x2*)(acc + st * D + d0 + 4 * v));
        else
          a[q][v] = *(const f32x4*)(acc + st * D + d0 + 4 * v);
      }
    }
  }
  // Adds states q0 .. min(n, q0 + kN) - 1 (states with m = -inf hold no
  // keys and are skipped) to the running (M, den, num).
  __device__ __forceinline__ void absorb(int q0, int n, float& M, float& den,
                                         float (&num)[kVecs][4]) const {
    float bm = -INFINITY;
#pragma unroll
    for (int q = 0; q < kN; ++q) bm = q0 + q < n ? fmaxf(bm, m[q]) : bm;
    if (bm > M) {
      const float f = M == -INFINITY ? 0.f : fast_exp2(M - bm);
#pragma unroll
      for (int v = 0; v < kVecs; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) num[v][i] *= f;
      den *= f;
      M = bm;
    }
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const float e = (q0 + q >= n || m[q] == -INFINITY) ? 0.f : fast_exp2(m[q] - M);
      const float w = kNorm ? e * l[q] : e;
#pragma unroll
      for (int v = 0; v < kVecs; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) num[v][i] = __builtin_fmaf(w, a[q][v][i], num[v][i]);
      den = __builtin_fmaf(e, l[q], den);
    }
  }
};

template <typename OT, int D, int G>
__global__ __launch_bounds__(kReduceWaves * kWave) void prefix_merge_wave_kernel(
    void* __restrict__ out, const float* __restrict__ part_acc,
    const float* __restrict__ part_ml, const int32_t* __restrict__ cuts,
    const int32_t* __restrict__ seq_lens, int num_seqs, int num_kv_heads, float v_scale,
    SuffixStates sx, const uint16_t* __restrict__ prefix_o, const float* __restrict__ prefix_ml,
    int prefix_splits) {
  using MB = MergeBatch<D, G, false>;
  using PB = MergeBatch<D, G, true>;
  constexpr int kVecs = MB::kVecs;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = (int64_t)blockIdx.x * kReduceWaves +
                       __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  if (item >= (int64_t)num_seqs * num_kv_heads) return;
  const int s = (int)(item / num_kv_heads), g = (int)(item % num_kv_heads);
  const int h = lane / MB::kLanesPerHead, d0 = (lane % MB::kLanesPerHead) * MB::kDims;
  const int num_heads = num_kv_heads * G;
  const int64_t hq = (int64_t)s * num_heads + g * G + h;
  const bool has_suffix = seq_lens[s] > sx.skip;
  const int va = cuts[2 * item + 0], code = cuts[2 * item + 1];
  const int np = code >> 1, slot0 = code & 1;
  // The suffix's states: the whole-sequence state (np <= 1) or the pieces.
  const int ns = has_suffix ? (np <= 1 ? 1 : np) : 0;
  auto prefix_idx = [&](int c) -> int64_t { return (int64_t)c * num_seqs * num_heads + hq; };
  auto piece_idx = [&](int p) -> int64_t {
    return ((int64_t)((va + p) * num_kv_heads + g) * 2 + (p == 0 ? slot0 : 0)) * G + h;
  };
  const bool whole = np <= 1;
  const float* s_ml = whole ? sx.ml : part_ml;
  const float* s_acc = whole ? sx.acc : part_acc;
  auto suffix_idx = [&](int p) -> int64_t { return whole ? hq : piece_idx(p); };
  float M = -INFINITY, den = 0.f, num[kVecs][4];
#pragma unroll
  for (int v = 0; v < kVecs; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) num[v][i] = 0.f;
  PB pb;
  MB sb;
  if (prefix_splits > 0) pb.load(prefix_ml, prefix_o, 0, prefix_splits, d0, prefix_idx);
  if (ns > 0) sb.load(s_ml, s_acc, 0, ns, d0, suffix_idx);
  if (prefix_splits > 0) pb.absorb(0, prefix_splits, M, den, num);
  for (int c0 = MB::kN; c0 < prefix_splits; c0 += MB::kN) {
    pb.load(prefix_ml, prefix_o, c0, prefix_splits, d0, prefix_idx);
    pb.absorb(c0, prefix_splits, M, den, num);
  }
  if (ns > 0) sb.absorb(0, ns, M, den, num);
  for (int p0 = MB::kN; p0 < ns; p0 += MB::kN) {
    sb.load(s_ml, s_acc, p0, ns, d0, suffix_idx);
    sb.absorb(p0, ns, M, den, num);
  }
  const float inv = den > 0.f ? v_scale / den : 0.f;
  const int64_t o = hq * D + d0;
#pragma unroll
  for (int v = 0; v < kVecs; ++v) {
    const float x0 = num[v][0] * inv, x1 = num[v][1] * inv;
    const float x2 = num[v][2] * inv, x3 = num[v][3] * inv;
    if constexpr (std::is_same<OT, F32>::value) {
      *(f32x4*)((float*)out + o + 4 * v) = f32x4{x0, x1, x2, x3};
    } else {
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(x0) | ((uint32_t)f32_to_bf16_rne(x1) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(x2) | ((uint32_t)f32_to_bf16_rne(x3) << 16);
      *(u32x2*)((uint16_t*)out + o + 4 * v) = u32x2{w0, w1};
    }
  }
}

// Log-sum-exp merge of the fixed partitions of one (query head, KV head,
// sequence), one output element per thread: partition p of query head h
// left (m_p, l_p, o_p) with o_p normalised;
// out = sum_p 2^(m_p - M) l_p o_p / sum_p 2^(m_p - M) l_p.
template <typename OT, int D, int G>
__global__ __launch_bounds__(D) void lse_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const int32_t* __restrict__ seq_lens, int num_kv_heads,
    int block_size, int partition_blocks, int max_parts) {
  const int h = blockIdx.x, g = blockIdx.y, s = blockIdx.z, d = threadIdx.x;
  const int L = seq_lens[s];
  const int nblk = (L + block_size - 1) / block_size;
  const int nparts = nblk > partition_blocks ? (nblk + partition_blocks - 1) / partition_blocks : 1;
  if (nparts <= 1) return;
  const int num_heads = num_kv_heads * G;
  const int64_t hq0 = (int64_t)s * num_heads + (int64_t)g * G;
  // Partition p of head h is state (hq0 + h) * max_parts + p; the decode
  // kernel already applied the value scale and normalised each output.
  auto state = [&](int p, int hh) -> int64_t { return (hq0 + hh) * max_parts + p; };
  store_out<OT>(out, (hq0 + h) * D + d, merge_element<true>(part_o, part_ml, nparts, D, h, d, state));
}

// The same merge by one workgroup of kLseWaves wavefronts per (sequence,
// KV head, group of ReduceShape heads), for D G >= 256: wavefront w merges
// partitions w, w + kLseWaves, ... sixteen at a time (16-byte state loads,
// D H / 64 consecutive outputs of one head per lane, H = ReduceShape::H),
// the partial merges meet in LDS and wavefront 0 writes the outputs.  A
// sequence of 64 partitions then takes one round of state loads per
// wavefront, where lse_reduce_kernel takes four.  (Sixteen wavefronts of
// four partitions each measured the same: the kernel's fixed cost, not its
// loads, sets its time.)
constexpr int kLseWaves = 4;

template <typename OT, int D, int G>
__global__ __launch_bounds__(kLseWaves * kWave) void lse_reduce_wg_kernel(
    void* __restrict__ out, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const int32_t* __restrict__ seq_lens, int num_kv_heads,
    int block_size, int partition_blocks, int max_parts) {
  constexpr int H = ReduceShape<D, G>::H, kGroups = ReduceShape<D, G>::kGroups;
  constexpr int kLanesPerHead = kWave / H, kDims = D / kLanesPerHead, kVecs = kDims / 4;
  constexpr int kBatch = 16;
  static_assert(kDims % 4 == 0, "whole 4-element groups per lane");
  __shared__ float red[kLseWaves][2 + kDims][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t sg = blockIdx.x / kGroups;  // (sequence, KV head)
  const int s = (int)(sg / num_kv_heads), g = (int)(sg % num_kv_heads);
  const int h = (int)(blockIdx.x % kGroups) * H + lane / kLanesPerHead;  // head within G
  const int d0 = (lane % kLanesPerHead) * kDims;
  const int L = seq_lens[s];
  const int nblk = (L + block_size - 1) / block_size;
  const int nparts = nblk > partition_blocks ? (nblk + partition_blocks - 1) / partition_blocks : 1;
  if (nparts <= 1) return;  // the decode kernel wrote the output
  const int64_t hq = (int64_t)s * num_kv_heads * G + (int64_t)g * G + h;
  float M = -INFINITY, den = 0.f, num[kVecs][4];
#pragma unroll
  for (int v = 0; v < kVecs; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) num[v][i] = 0.f;
  // This wavefront's partitions w, w + kLseWaves, ...: n_mine of them.
  const int n_mine = nparts > w ? (nparts - w + kLseWaves - 1) / kLseWaves : 0;
  for (int q0 = 0; q0 < n_mine; q0 += kBatch) {
    float m[kBatch], l[kBatch];
    f32x4 a[kBatch][kVecs];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int p = w + kLseWaves * (q0 + q < n_mine ? q0 + q : n_mine - 1);
      const int64_t st = hq * max_parts + p;
      m[q] = part_ml[2 * st];
      l[q] = part_ml[2 * st + 1];
#pragma unroll
      for (int v = 0; v < kVecs; ++v) a[q][v] = *(const f32x4*)(part_o + st * D + d0 + 4 * v);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) bm = q0 + q < n_mine ? fmaxf(bm, m[q]) : bm;
    if (bm > M) {
      const float f = M == -INFINITY ? 0.f : fast_exp2(M - bm);
#pragma unroll
      for (int v = 0; v < kVecs; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) num[v][i] *= f;
      den *= f;
      M = bm;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      // Normalised states: each adds e l o to the numerator, e l to the sum.
      const float el = (q0 + q >= n_mine || M == -INFINITY) ? 0.f : fast_exp2(m[q] - M) * l[q];
#pragma unroll
      for (int v = 0; v < kVecs; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) num[v][i] = __builtin_fmaf(el, a[q][v][i], num[v][i]);
      den += el;
    }
  }
  red[w][0][lane] = M;
  red[w][1][lane] = den;
#pragma unroll
  for (int v = 0; v < kVecs; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][2 + 4 * v + i][lane] = num[v][i];
  __syncthreads();
  if (w != 0) return;
  float Mt = -INFINITY;
  for (int x = 0; x < kLseWaves; ++x) Mt = fmaxf(Mt, red[x][0][lane]);
  float dt = 0.f, nt[kDims];
#pragma unroll
  for (int i = 0; i < kDims; ++i) nt[i] = 0.f;
#pragma unroll 2
  for (int x = 0; x < kLseWaves; ++x) {
    const float mx = red[x][0][lane];
    const float f = mx == -INFINITY ? 0.f : fast_exp2(mx - Mt);
    dt = __builtin_fmaf(f, red[x][1][lane], dt);
#pragma unroll
    for (int i = 0; i < kDims; ++i) nt[i] = __builtin_fmaf(f, red[x][2 + i][lane], nt[i]);
  }
  const int64_t o = hq * D + d0;
#pragma unroll
  for (int v = 0; v < kVecs; ++v) {
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = dt > 0.f ? nt[4 * v + i] / dt : 0.f;
    if constexpr (std::is_same<OT, F32>::value) {
      *(f32x4*)((float*)out + o + 4 * v) = f32x4{x[0], x[1], x[2], x[3]};
    } else {
      const uint32_t w0 = (uint32_t)f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16);
      *(u32x2*)((uint16_t*)out + o + 4 * v) = u32x2{w0, w1};
    }
  }
}

// Wavefronts per workgroup: enough blocks per wavefront to keep its
// one-tile-ahead pipeline busy, at most four.
}  // namespace pa

#include "decode_mfma.h"

namespace pa {

// Whether a (cache, query, head size, group) combination has the
// matrix-core engine.
template <typename KV, typename QT, int D, int G>
constexpr bool kHasMfma = D == kMD && (G == 4 || G == 8) && !std::is_same<KV, F32>::value &&
                          std::is_same<QT, BF16>::value;

inline int decode_waves(int partition_blocks, int max_seq_len, int block_size) {
  const int blocks = partition_blocks > 0 ? partition_blocks
                                          : (max_seq_len + block_size - 1) / block_size;
  if (blocks >= 64) return 4;
  if (blocks >= 24) return 2;
  return 1;
}

// PBS: the pool's block size.  The vector engine works on tiles of at most
// 32 tokens (BS), a pool block of 64 or 128 being 2 or 4 consecutive tiles;
// the matrix-core engine takes the pool block size directly.
template <typename KV, typename QT, int D, int PBS, int G>
hipError_t launch_decode(const DecodeArgs& a) {
  constexpr int BS = PBS < 32 ? PBS : 32;
  constexpr int kSubShift = PBS == 128 ? 2 : (PBS == 64 ? 1 : 0);
  static_assert((BS << kSubShift) == PBS, "pool blocks are whole tiles");
  const float k_scale = std::is_same<KV, FP8>::value ? a.k_scale : 1.0f;
  const float v_scale = std::is_same<KV, FP8>::value ? a.v_scale : 1.0f;
  const float qk = a.scale * k_scale * kLog2e;
  if (a.balanced_workers > 0) {
    const int per_head = a.balanced_workers / a.num_kv_heads;
    const int workers = per_head * a.num_kv_heads;
    const int wg = (workers + kMaxDecodeWaves - 1) / kMaxDecodeWaves;
    bool mfma = false;
    if constexpr (kHasMfma<KV, QT, D, G>) mfma = a.engine == kEngineMfma;
    static_assert(!kHasMfma<KV, QT, D, G> || D * G >= 4 * kWave,
                  "the matrix-core engine writes no merge tasks: its reduce is the wavefront one");
    if constexpr (kHasMfma<KV, QT, D, G>) {
      if (mfma)
        launch_main(a, decode_balanced_mfma_kernel<KV, QT, PBS, G>, dim3((unsigned)wg),
                           dim3(kMaxDecodeWaves * kWave), a.out, a.part_o, a.part_ml,
                           a.cuts, a.query, a.k_cache, a.v_cache, a.block_tables,
                           a.seq_lens,
                           a.num_seqs, a.max_blocks_per_seq, a.num_kv_heads, per_head, qk, v_scale,
                           a.read_once, a.suffix, a.append);
    }
    if (!mfma)
      launch_main(a, decode_balanced_kernel<KV, QT, D, BS, G>, dim3((unsigned)wg),
                         dim3(kMaxDecodeWaves * kWave), a.out, a.part_o, a.part_ml,
                         a.merges, a.cuts, a.query, a.k_cache, a.v_cache, a.block_tables,
                         a.seq_lens,
                         a.num_seqs, a.max_blocks_per_seq, a.num_kv_heads, per_head, qk, v_scale,
                         kSubShift, a.read_once, a.suffix);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.prefix_o) {
      if constexpr (D * G >= 4 * kWave)
        hipLaunchKernelGGL((prefix_merge_wave_kernel<QT, D, G>),
                         dim3((unsigned)(((int64_t)a.num_seqs * a.num_kv_heads + kReduceWaves - 1) /
                                         kReduceWaves)),
                         dim3(kReduceWaves * kWave), 0, a.stream, a.out, a.part_o, a.part_ml,
                         a.cuts, a.seq_lens, a.num_seqs, a.num_kv_heads, v_scale, a.suffix,
                         a.prefix_o, a.prefix_ml, a.prefix_splits);
      else
        hipLaunchKernelGGL((prefix_merge_kernel<QT, D, G>),
                         dim3((unsigned)a.num_seqs,
                              (unsigned)((a.num_heads * D + 4 * kMergeThreads - 1) /
                                         (4 * kMergeThreads))),
                         dim3(kMergeThreads),
                         0, a.stream, a.out, a.part_o, a.part_ml, a.cuts, a.seq_lens, a.num_seqs,
                         a.num_kv_heads, v_scale, a.suffix, a.prefix_o, a.prefix_ml,
                         a.prefix_splits);
    } else if constexpr (D * G >= 4 * kWave)
      hipLaunchKernelGGL((balanced_reduce_wave_kernel<QT, D, G>),
                         dim3((unsigned)(((int64_t)a.num_seqs * a.num_kv_heads *
                                              ReduceShape<D, G>::kGroups +
                                          kReduceWaves - 1) /
                                         kReduceWaves)),
                         dim3(kReduceWaves * kWave), 0, a.stream, a.out, a.part_o, a.part_ml,
                         a.cuts, a.seq_lens, a.num_seqs, a.num_kv_heads, v_scale);
    else if (a.num_seqs <= per_head)
      hipLaunchKernelGGL((balanced_reduce_kernel<QT, D, G>),
                         dim3((unsigned)G, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs), dim3(D),
                         0, a.stream, a.out, a.part_o, a.part_ml, a.cuts, a.seq_lens,
                         a.num_kv_heads, v_scale);
    else
      hipLaunchKernelGGL((balanced_reduce_tasks_kernel<QT, D, G>),
                         dim3((unsigned)G, (unsigned)per_head, (unsigned)a.num_kv_heads), dim3(D),
                         0, a.stream, a.out, a.part_o, a.part_ml, a.merges, a.seq_lens,
                         a.num_seqs, a.num_kv_heads, v_scale);
    return hipGetLastError();
  }
  const int tiles_per_part = a.partition_blocks << kSubShift;  // 0: whole sequence
  // Fixed partitions on the matrix cores where that engine is built and not
  // pinned away (one wavefront per partition; a whole sequence in one
  // partition stays on the vector engine, whose wavefronts share it).
  bool mfma_parts = false;
  if constexpr (kHasMfma<KV, QT, D, G>) {
    mfma_parts = a.engine == kEngineMfma && a.partition_blocks > 0;
    if (mfma_parts) {
      const int units = a.partition_blocks * PBS / MfmaAttn<KV, PBS, G>::UBS;
      launch_main(a, decode_partitioned_mfma_kernel<KV, QT, PBS, G>,
                  dim3((unsigned)((a.max_parts + kMaxDecodeWaves - 1) / kMaxDecodeWaves),
                       (unsigned)a.num_kv_heads, (unsigned)a.num_seqs),
                  dim3(kMaxDecodeWaves * kWave), a.out, a.part_o, a.part_ml, a.query, a.k_cache,
                  a.v_cache, a.block_tables, a.seq_lens, a.max_blocks_per_seq, a.num_kv_heads,
                  units, a.max_parts, qk, v_scale, a.read_once);
    }
  }
  if (!mfma_parts) {
    const int nw = a.num_waves > 0 ? a.num_waves : decode_waves(tiles_per_part, a.max_seq_len, BS);
    launch_main(a, decode_kernel<KV, QT, D, BS, G>,
                dim3((unsigned)a.max_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs),
                dim3(nw * kWave), a.out, a.part_o, a.part_ml, a.query, a.k_cache, a.v_cache,
                a.block_tables, a.seq_lens, a.max_blocks_per_seq, a.num_kv_heads, tiles_per_part,
                a.max_parts, qk, v_scale, kSubShift, a.read_once);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  if constexpr (D * G >= 4 * kWave)
    hipLaunchKernelGGL((lse_reduce_wg_kernel<QT, D, G>),
                       dim3((unsigned)((int64_t)a.num_seqs * a.num_kv_heads *
                                       ReduceShape<D, G>::kGroups)),
                       dim3(kLseWaves * kWave), 0, a.stream, a.out, a.part_o, a.part_ml,
                       a.seq_lens, a.num_kv_heads, a.block_size, a.partition_blocks, a.max_parts);
  else
    hipLaunchKernelGGL((lse_reduce_kernel<QT, D, G>),
                       dim3((unsigned)G, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs), dim3(D),
                       0, a.stream, a.out, a.part_o, a.part_ml, a.seq_lens, a.num_kv_heads,
                       a.block_size, a.partition_blocks, a.max_parts);
  return hipGetLastError();
}

template <typename KV, typename QT, int D, int BS>
hipError_t dispatch_group(const DecodeArgs& a) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_decode<KV, QT, D, BS, 1>(a);
    case 2: return launch_decode<KV, QT, D, BS, 2>(a);
    case 4: return launch_decode<KV, QT, D, BS, 4>(a);
    case 8: return launch_decode<KV, QT, D, BS, 8>(a);
    default: return kNotInstantiated;
  }
}

template <typename KV, typename QT, int D>
hipError_t dispatch_block(const DecodeArgs& a) {
  switch (a.block_size) {
    case 16: return dispatch_group<KV, QT, D, 16>(a);
    case 32: return dispatch_group<KV, QT, D, 32>(a);
    case 64: return dispatch_group<KV, QT, D, 64>(a);
    case 128: return dispatch_group<KV, QT, D, 128>(a);
    default: return kNotInstantiated;
  }
}

}  // namespace pa
