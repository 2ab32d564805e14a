// decode_impl.h — the paged decode kernel and the split-K log-sum-exp merge.
//
// What it computes ("vLLM：大语言模型推理与服务库" §4.4 item 3): for every
// sequence s and query head h, walk the physical blocks of s through its
// block table, score q·k for every cached token, take the softmax and weight
// V.  Grid axes follow the partitioned grid the openeuler.csdn.net essay
// describes ("PagedAttention：把操作系统的分页搬上 GPU": one workgroup per
// head group, sequence and partition of the context), re-cut for gfx950:
//
//   * one workgroup = one (partition, KV head, sequence); its 4 wavefronts
//     take the partition's blocks round-robin, so all G = Hq/Hkv query heads
//     of the group share every K/V byte read from HBM;
//   * a (block, KV head) tile is contiguous in the pool, so a wavefront reads
//     it with NLOAD fully coalesced 1 KiB loads (16 bytes per lane) straight
//     into VGPRs; one token row occupies LPR = 4/8/16 lanes, i.e. sits inside
//     a DPP row, and q·k reduces with 2-4 DPP adds;
//   * the next block's loads are issued before the current block is
//     computed (register double buffering);
//   * softmax is online in fp32 in the log2 domain (exp2 on v_exp_f32); each
//     DPP row of a wavefront keeps its own running max / sum over the tokens
//     it saw, so the per-block update needs no cross-row traffic; rows, then
//     wavefronts (through LDS), are merged once per partition;
//   * with several partitions per sequence each workgroup writes its
//     (max, sum, normalised output) and a second kernel merges them.
#pragma once

#include "pa_internal.h"

namespace pa {

constexpr int kDecodeWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;

template <typename KV, int D, int BS>
struct TileShape {
  static constexpr int EB = Elem<KV>::bytes;
  static constexpr int EPL = 16 / EB;        // elements per lane per load
  static constexpr int LPR = D / EPL;        // lanes per token row
  static constexpr int RPL = kWave / LPR;    // token rows per wavefront load
  static constexpr int NLOAD = BS / RPL;     // loads per (block, head) tile
  static constexpr int64_t TILE_VECS = (int64_t)BS * D * EB / 16;
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "a token row must fit a DPP row");
  static_assert(NLOAD >= 1 && BS % RPL == 0, "a tile must be whole wavefront loads");
};

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Query registers of one lane: its EPL dims of each of the G heads.
// bf16 cache: kept packed for v_dot2_f32_bf16; otherwise widened to fp32.
template <typename KV, typename QT, int G, int EPL>
struct QRegs {
  static constexpr bool kPacked = std::is_same<KV, BF16>::value && std::is_same<QT, BF16>::value;
  uint32_t w[kPacked ? G : 1][4];
  float f[kPacked ? 1 : G][kPacked ? 1 : EPL];

  __device__ __forceinline__ void load(const void* query, int64_t row0, int D, int col) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t e0 = (row0 + h) * D + (int64_t)col * EPL;
      if constexpr (kPacked) {
        const u32x4 v = *(const u32x4*)((const uint16_t*)query + e0);
        w[h][0] = v.x; w[h][1] = v.y; w[h][2] = v.z; w[h][3] = v.w;
      } else if constexpr (std::is_same<QT, F32>::value) {
        static_assert(EPL == 4, "f32 queries pair with an f32 cache");
        const u32x4 v = *(const u32x4*)((const float*)query + e0);
        Vec<F32>::to_f32(v, f[h]);
      } else {  // bf16 query, widened
#pragma unroll
        for (int j = 0; j < EPL / 8; ++j) {
          const u32x4 v = *(const u32x4*)((const uint16_t*)query + e0 + 8 * j);
          Vec<BF16>::to_f32(v, f[h] + 8 * j);
        }
      }
    }
  }

  // Partial q·k over this lane's EPL dims for head h; kf holds the widened
  // key (unused on the packed path).
  __device__ __forceinline__ float dot(int h, const u32x4& k, const float* kf) const {
    if constexpr (kPacked) {
      float a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.x), as_bf16x2(w[h][0]), 0.f, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.y), as_bf16x2(w[h][1]), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.z), as_bf16x2(w[h][2]), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.w), as_bf16x2(w[h][3]), a, false);
      return a;
    } else {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a = __builtin_fmaf(f[h][e], kf[e], a);
      return a;
    }
  }
};

template <typename OT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (std::is_same<OT, F32>::value) ((float*)out)[idx] = v;
  else ((uint16_t*)out)[idx] = f32_to_bf16_rne(v);
}

template <typename KV, typename QT, int D, int BS, int G>
__global__ __launch_bounds__(kDecodeWaves * kWave) void decode_kernel(
    void* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
    const void* __restrict__ query, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, int max_blocks_per_seq, int num_kv_heads,
    int partition_blocks, int max_parts, float qk_scale_log2, float v_scale) {
  using TS = TileShape<KV, D, BS>;
  constexpr int EPL = TS::EPL, LPR = TS::LPR, RPL = TS::RPL, NLOAD = TS::NLOAD;
  constexpr int NW = kDecodeWaves;
  using OT = QT;

  const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int col = lane % LPR, row = lane / LPR;
  const int num_heads = num_kv_heads * G;

  const int L = seq_lens[s];
  const int nblk = (L + BS - 1) / BS;
  const int pb = partition_blocks > 0 ? partition_blocks : (nblk > 0 ? nblk : 1);
  const int nparts = nblk > pb ? (nblk + pb - 1) / pb : 1;
  if (part >= nparts) return;
  const int b0 = part * pb;
  const int b1 = min(b0 + pb, nblk);

  QRegs<KV, QT, G, EPL> q;
  q.load(query, (int64_t)s * num_heads + (int64_t)g * G, D, col);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int32_t* tbl = block_tables + (int64_t)s * max_blocks_per_seq;
  const int span = b1 - b0;
  const int nmine = span > w ? (span - w + NW - 1) / NW : 0;
  const int64_t block_vecs = (int64_t)num_kv_heads * TS::TILE_VECS;
  const u32x4* kbase = (const u32x4*)k_cache + (int64_t)g * TS::TILE_VECS + lane;
  const u32x4* vbase = (const u32x4*)v_cache + (int64_t)g * TS::TILE_VECS + lane;

  // Block ids of this wavefront's blocks, 64 at a time, one per lane.
  int bid_v = 0;
  auto block_id = [&](int j) -> int {
    if ((j & (kWave - 1)) == 0) {
      const int jj = j + lane;
      bid_v = jj < nmine ? tbl[b0 + w + NW * jj] : 0;
    }
    return __builtin_amdgcn_readlane(bid_v, j & (kWave - 1));
  };
  auto load_tile = [&](int bid, u32x4 (&kt)[NLOAD], u32x4 (&vt)[NLOAD]) {
    const u32x4* kp = kbase + (int64_t)bid * block_vecs;
    const u32x4* vp = vbase + (int64_t)bid * block_vecs;
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) kt[i] = kp[i * kWave];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) vt[i] = vp[i * kWave];
  };
  auto process = [&](const u32x4 (&kt)[NLOAD], const u32x4 (&vt)[NLOAD], int blk) {
    float sc[NLOAD][G];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      float kf[std::is_same<KV, BF16>::value ? 1 : EPL];
      if constexpr (!std::is_same<KV, BF16>::value) Vec<KV>::to_f32(kt[i], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) sc[i][h] = q.dot(h, kt[i], kf);
    }
#pragma unroll
    for (int i = 0; i < NLOAD; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) sc[i][h] = group_sum<LPR>(sc[i][h]) * qk_scale_log2;

    float vf[NLOAD][EPL];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) Vec<KV>::to_f32(vt[i], vf[i]);

    if ((blk + 1) * BS > L) {  // the sequence's last, partly filled block
      const int tok0 = blk * BS + row;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        const bool valid = tok0 + i * RPL < L;
#pragma unroll
        for (int h = 0; h < G; ++h) sc[i][h] = valid ? sc[i][h] : -INFINITY;
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[i][e] = valid ? vf[i][e] : 0.f;
      }
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int i = 1; i < NLOAD; ++i) bm = fmaxf(bm, sc[i][h]);
      const float mn = fmaxf(m[h], bm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - mu);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        const float p = fast_exp2(sc[i][h] - mu);
        ps += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = __builtin_fmaf(p, vf[i][e], acc[h][e]);
      }
      l[h] = l[h] * alpha + ps;
      m[h] = mn;
    }
  };

  if (nmine > 0) {
    u32x4 kc[NLOAD], vc[NLOAD];
    load_tile(block_id(0), kc, vc);
    for (int j = 0; j + 1 < nmine; ++j) {
      u32x4 kn[NLOAD], vn[NLOAD];
      load_tile(block_id(j + 1), kn, vn);
      process(kc, vc, b0 + w + NW * j);
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) { kc[i] = kn[i]; vc[i] = vn[i]; }
    }
    process(kc, vc, b0 + w + NW * (nmine - 1));
  }

  // Merge the DPP rows of this wavefront (lanes with equal col).
#pragma unroll
  for (int mask = LPR; mask < kWave; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = shfl_xor(m[h], mask);
      const float lo = shfl_xor(l[h], mask);
      const float M = fmaxf(m[h], mo);
      const float mu = M == -INFINITY ? 0.f : M;
      const float f = fast_exp2(m[h] - mu), fo = fast_exp2(mo - mu);
      l[h] = l[h] * f + lo * fo;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * f + shfl_xor(acc[h][e], mask) * fo;
      m[h] = M;
    }
  }

  // Merge the wavefronts through LDS and finish.
  __shared__ float sm_ml[NW][G][2];
  __shared__ float sm_acc[NW][G][D];
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[w][h][col * EPL + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { sm_ml[w][h][0] = m[h]; sm_ml[w][h][1] = l[h]; }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
    const int h = idx / D, d = idx % D;
    float M = sm_ml[0][h][0];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm_ml[ww][h][0]);
    const float mu = M == -INFINITY ? 0.f : M;
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = fast_exp2(sm_ml[ww][h][0] - mu);
      den += f * sm_ml[ww][h][1];
      num += f * sm_acc[ww][h][d];
    }
    const float o = den > 0.f ? num / den * v_scale : 0.f;
    const int64_t hq = (int64_t)s * num_heads + (int64_t)g * G + h;
    if (nparts == 1) {
      store_out<OT>(out, hq * D + d, o);
    } else {
      part_o[(hq * max_parts + part) * D + d] = o;
      if (d == 0) {
        part_ml[(hq * max_parts + part) * 2 + 0] = M;
        part_ml[(hq * max_parts + part) * 2 + 1] = den;
      }
    }
  }
}

// Log-sum-exp merge of the partitions of one (sequence, query head):
// M = max_p m_p, w_p = 2^(m_p - M) * l_p, out = sum_p w_p o_p / sum_p w_p.
template <typename OT, int D>
__global__ __launch_bounds__(kWave) void lse_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const int32_t* __restrict__ seq_lens, int num_heads,
    int block_size, int partition_blocks, int max_parts) {
  const int hq_in_seq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int L = seq_lens[s];
  const int nblk = (L + block_size - 1) / block_size;
  const int nparts = nblk > partition_blocks ? (nblk + partition_blocks - 1) / partition_blocks : 1;
  if (nparts <= 1) return;
  const int64_t hq = (int64_t)s * num_heads + hq_in_seq;
  const float* ml = part_ml + hq * max_parts * 2;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  const float mu = M == -INFINITY ? 0.f : M;
  constexpr int DPL = D / kWave;
  float num[DPL], den = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) num[e] = 0.f;
  const float* po = part_o + hq * max_parts * D + lane * DPL;
  for (int p = 0; p < nparts; ++p) {
    const float wgt = fast_exp2(ml[2 * p] - mu) * ml[2 * p + 1];
    den += wgt;
#pragma unroll
    for (int e = 0; e < DPL; ++e) num[e] = __builtin_fmaf(wgt, po[(int64_t)p * D + e], num[e]);
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e)
    store_out<OT>(out, hq * D + lane * DPL + e, den > 0.f ? num[e] / den : 0.f);
}

template <typename KV, typename QT, int D, int BS, int G>
hipError_t launch_decode(const DecodeArgs& a) {
  const float k_scale = std::is_same<KV, FP8>::value ? a.k_scale : 1.0f;
  const float v_scale = std::is_same<KV, FP8>::value ? a.v_scale : 1.0f;
  const float qk = a.scale * k_scale * kLog2e;
  hipLaunchKernelGGL((decode_kernel<KV, QT, D, BS, G>),
                     dim3((unsigned)a.max_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs),
                     dim3(kDecodeWaves * kWave), 0, a.stream, a.out, a.part_o, a.part_ml, a.query,
                     a.k_cache, a.v_cache, a.block_tables, a.seq_lens, a.max_blocks_per_seq,
                     a.num_kv_heads, a.partition_blocks, a.max_parts, qk, v_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  hipLaunchKernelGGL((lse_reduce_kernel<QT, D>), dim3((unsigned)a.num_heads, (unsigned)a.num_seqs),
                     dim3(kWave), 0, a.stream, a.out, a.part_o, a.part_ml, a.seq_lens, a.num_heads,
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
    default: return hipErrorInvalidValue;
  }
}

template <typename KV, typename QT, int D>
hipError_t dispatch_block(const DecodeArgs& a) {
  switch (a.block_size) {
    case 16: return dispatch_group<KV, QT, D, 16>(a);
    case 32: return dispatch_group<KV, QT, D, 32>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
