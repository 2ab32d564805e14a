// decode_mfma.h — the paged decode of a GQA group on the matrix cores.
//
// Same computation as the wavefront engine in decode_impl.h ("vLLM：大语言
// 模型推理与服务库" §4.4 item 3: gather each sequence's K/V through its block
// table, softmax of the scaled scores, weighted sum of V), for head size 128
// and groups of G = 4 or 8 query heads.  Where the group is large (an fp8
// cache with G = 8 does 16 multiply-adds per cached byte), the vector ALU
// path runs out of issue slots long before HBM runs out of bandwidth, so
// here both contractions go to v_mfma_f32_16x16x32_bf16 with the G query
// heads as the 16-wide N side (G real columns, the rest zero):
//
//   * S^T = K · Q^T per 32-key tile: A = K (16 keys x 32 dims per MFMA)
//     straight from the pool into registers (16 bytes per lane, a key row
//     read by 4 lanes as 64 contiguous bytes; fp8 widened exactly to bf16),
//     B = Q^T (the dims permuted the same way, loaded once).  C leaves each
//     lane 4 keys x 1 head per 16-key group;
//   * online softmax in fp32, log2 domain, with the same lazy reference as
//     the vector path: one reference per head, raised (and the
//     accumulators rescaled) only when a score exceeds it by 2^8, so the
//     common step needs no cross-lane reduction;
//   * O^T += V^T · P^T: P^T is already in the B layout (the 8 keys of a
//     lane are its two groups' 4).  V goes through a per-wavefront LDS tile
//     row-major, as read from the pool (fp8 widened to bf16), with fully
//     coalesced loads and conflict-free 16-byte writes; gfx950's transposing
//     LDS read (ds_read_b64_tr_b16) then hands each lane 4 keys of one dim,
//     the A layout, with no repacking.
//
// The tile loop runs one tile ahead in registers (ping-pong), as the vector
// path does.  Only runs of consecutive blocks of one sequence (the balanced
// split) use this engine.
#pragma once

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kMD = 128;                // head size

__device__ __forceinline__ f32x4 mfma16(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, u32x4{a[0], a[1], a[2], a[3]}),
      __builtin_bit_cast(bf16x8_t, u32x4{b[0], b[1], b[2], b[3]}), c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: A[m = l%16][k = 4(l/16) + j], B[k][n = l%16],
// C[4(l/16) + i][l%16] (the 16x16x32 layout with 4 k per lane).
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16k16(const uint32_t (&a)[2], const uint32_t (&b)[2], f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, u32x2{a[0], a[1]}),
                                                  __builtin_bit_cast(s16x4_t, u32x2{b[0], b[1]}), c,
                                                  0, 0, 0);
}

// Keys per tile: 32 (two 16-key groups, P·V with k = 32) where a tile's raw
// words fit the registers twice over, else 16 (bf16: one group, P·V with
// k = 16).
template <typename KV> struct MfmaTileKeys { static constexpr int value = 32; };
template <> struct MfmaTileKeys<BF16> { static constexpr int value = 16; };

// Row stride of the LDS V tile (bf16): a 256-byte key row plus 32 bytes, so
// the 4 rows a 16-lane group reads with one transposing load, and the 8
// rows of a 32-lane pass, fall on distinct banks.
constexpr int kVRow = kMD + 16;

// ds_read_b64_tr_b16: in each 16-lane group, lane t supplies the address of
// 4 consecutive 16-bit elements F[t][0..3]; lane j receives
// {F[4k + j/4][j%4] : k = 0..3} (layout probed on gfx950).
typedef short s16x4_t2 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const __bf16* p) {
  const s16x4_t2 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t2*)(p));
  return __builtin_bit_cast(u32x2, v);
}

template <typename KV, int BS, int G>
struct MfmaAttn {
  static constexpr int EB = Elem<KV>::bytes;
  static constexpr int KEYS = MfmaTileKeys<KV>::value;     // keys per tile
  static constexpr int KG = KEYS / 16;                      // 16-key groups per tile
  static constexpr int NBT = KEYS > BS ? KEYS / BS : 1;     // blocks a tile touches
  // Unit of the balanced split: runs start and end on multiples of UBS
  // tokens (a pool block, or a 32-token part of a larger one), so that runs
  // are balanced to 32 tokens whatever the block size.
  static constexpr int UBS = BS < 32 ? BS : 32;
  static constexpr int KL = 16 * kMD * EB / (kWave * 16);   // K 16-byte loads per key group
  static constexpr int CPR = kMD * EB / 16;                 // 16-byte chunks of a V row
  static constexpr int VRL = kWave / CPR;                   // V rows per wavefront load
  static constexpr int VL = KEYS / VRL;                     // V loads per tile
  static_assert(G == 4 || G == 8, "the matrix-core path takes groups of 4 or 8");
  static_assert(KEYS % BS == 0 || BS % KEYS == 0, "tiles and blocks nest");

  // One tile's raw cache words: K for its key groups; V rows vr + VRL*i,
  // 16-byte chunk vc of each.
  struct Tile {
    u32x4 k[KG][KL];
    u32x4 v[VL];
  };

  int lane, n, g4;        // head column n = lane % 16, lane group g4 = lane / 16
  int vr, vc;             // V staging: rows vr + VRL*i, 16-byte chunk vc
  float qk_scale_log2;
  uint32_t q[4][4];       // Q^T operand per k-step (packed bf16)
  f32x4 acc[kMD / 16];    // O^T: dims 16mb + 4g4 + i, head n
  float m_ref, l_lane;
  __bf16* vt;             // this wavefront's V^T tile in LDS
  const __bf16* newk;     // fused append: the new token's K and V as the tile uses them (LDS)
  const __bf16* newv;

  static constexpr int kLdsElems = KEYS * kVRow;

  __device__ __forceinline__ void init(int lane_, float qk, __bf16* vt_, const __bf16* newk_ = nullptr,
                                       const __bf16* newv_ = nullptr) {
    lane = lane_;
    newk = newk_;
    newv = newv_;
    n = lane % 16;
    g4 = lane / 16;
    vr = lane / CPR;
    vc = lane % CPR;
    qk_scale_log2 = qk;
    vt = vt_;
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int mb = 0; mb < kMD / 16; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref = -INFINITY;
    l_lane = 0.f;
  }

  // Dims of k-step s (8 consecutive) as read from K by lane group g4.
  __device__ __forceinline__ int kstep_dim0(int s) const {
    if constexpr (EB == 1) return 16 * g4 + 64 * (s / 2) + 8 * (s % 2);
    else return 8 * g4 + 32 * s;
  }

  // Query rows row0 .. row0+G-1 (bf16) as the B operand; columns >= G zero.
  __device__ __forceinline__ void load_q(const void* query, int64_t row0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n < G) v = *(const u32x4*)((const uint16_t*)query + (row0 + n) * kMD + kstep_dim0(s));
      q[s][0] = v.x; q[s][1] = v.y; q[s][2] = v.z; q[s][3] = v.w;
    }
  }

  // Loads the tile whose first key is k0 (a sequence position; a multiple
  // of 16, and of KEYS when blocks hold at least 32 tokens); bid(j) gives
  // the physical id of the sequence's block j.  NT: the lines are read once
  // in this call, so they are loaded non-temporally (evict first), which
  // keeps the stream from churning the caches and lowers its latency under
  // load (about 10% on the bf16 and fp8 decode workloads).
  template <bool NT, typename BidFn>
  __device__ __forceinline__ void load_tile(const uint8_t* kh, const uint8_t* vh, int64_t block_bytes,
                                            int k0, BidFn bid, Tile& T) const {
    int b[NBT];
#pragma unroll
    for (int u = 0; u < NBT; ++u) b[u] = bid(k0 / BS + u);
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int key = k0 + 16 * kg;  // a 16-key group lies in one block
      const uint8_t* kb = kh + (int64_t)b[key / BS - k0 / BS] * block_bytes +
                          ((key % BS) + n) * kMD * EB + 16 * g4;
#pragma unroll
      for (int i = 0; i < KL; ++i) T.k[kg][i] = kv_load<NT>((const u32x4*)(kb + 64 * i));
    }
    // V: wavefront load i reads rows VRL*i .. +VRL of the tile, whole rows.
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int key = k0 + vr + VRL * i;  // tile row vr + VRL*i
      const int u = key / BS - k0 / BS;
      const int bb = NBT == 1 ? b[0] : b[u < NBT ? u : NBT - 1];
      T.v[i] = kv_load<NT>(
          (const u32x4*)(vh + (int64_t)bb * block_bytes + (key % BS) * kMD * EB + 16 * vc));
    }
  }

  // K operand of key group kg, k-step s, as 4 dwords of packed bf16.
  __device__ __forceinline__ void k_operand(const Tile& T, int kg, int s, uint32_t (&a)[4]) const {
    if constexpr (EB == 1) {
      const u32x4& w = T.k[kg][s / 2];
      const uint32_t lo = (s % 2) ? w.z : w.x, hi = (s % 2) ? w.w : w.y;
      a[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
      a[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
      a[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
      a[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    } else {
      const u32x4& w = T.k[kg][s];
      a[0] = w.x; a[1] = w.y; a[2] = w.z; a[3] = w.w;
    }
  }

  // Writes the tile's V rows into LDS as bf16 (fp8 widened exactly), rows
  // at or past lim zeroed (the padding slots of a block may hold anything,
  // and 0 * NaN is NaN).
  __device__ __forceinline__ void stage_v(const Tile& T, int lim) const {
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int r = vr + VRL * i;
      const bool ok = lim >= KEYS || r < lim;
      __bf16* row = vt + r * kVRow;
      if constexpr (EB == 1) {
        const uint32_t src[4] = {T.v[i].x, T.v[i].y, T.v[i].z, T.v[i].w};
        uint32_t w[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          w[2 * c] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[c], 1.0f, false));
          w[2 * c + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[c], 1.0f, true));
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) w[x] = ok ? w[x] : 0u;
        // 16 dims = 32 bytes per lane; odd rows write their halves in the
        // other order so that a 16-lane pass covers distinct banks.
        const int h0 = r & 1;
        u32x4* dst = (u32x4*)(row + 16 * vc);
        dst[h0] = h0 ? u32x4{w[4], w[5], w[6], w[7]} : u32x4{w[0], w[1], w[2], w[3]};
        dst[1 - h0] = h0 ? u32x4{w[0], w[1], w[2], w[3]} : u32x4{w[4], w[5], w[6], w[7]};
      } else {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *(u32x4*)(row + 8 * vc) = ok ? T.v[i] : z;
      }
    }
  }

  // One tile: lim valid keys (tile-relative, a prefix).  app >= 0: tile
  // row app is the appended token, whose K and V come from newk / newv
  // instead of T and the pool.
  __device__ __forceinline__ void tile(const Tile& T, int lim, int app = -1) {
    // S^T per 16-key group: independent chains of 4 MFMAs.
    f32x4 c[KG];
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) c[kg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {
        uint32_t a[4];
        k_operand(T, kg, s, a);
        if (app >= 0 && kg == app / 16) {
          const u32x4 w = *(const u32x4*)(newk + kstep_dim0(s));
          const bool mine = n == app % 16;
          a[0] = mine ? w.x : a[0];
          a[1] = mine ? w.y : a[1];
          a[2] = mine ? w.z : a[2];
          a[3] = mine ? w.w : a[3];
        }
        c[kg] = mfma16(a, q[s], c[kg]);
      }
    stage_v(T, lim);
    if (app >= 0 && lane < 16) {
      // Row app of the V tile (bf16 dims in order, as stage_v leaves every
      // row), written again from the new token: 8 dims (16 bytes) per lane.
      *(u32x4*)(vt + app * kVRow + 8 * lane) = *(const u32x4*)(newv + 8 * lane);
    }

    float x[KG][4];
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[kg][i] = c[kg][i] * qk_scale_log2;
    if (lim < KEYS) {
#pragma unroll
      for (int kg = 0; kg < KG; ++kg)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[kg][i] = 16 * kg + 4 * g4 + i < lim ? x[kg][i] : -INFINITY;
    }
    float lm = x[0][0];
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int i = 0; i < 4; ++i) lm = fmaxf(lm, x[kg][i]);
    if (__builtin_amdgcn_ballot_w64(lm > m_ref + kRescaleSlack)) {
      // Raise the head's reference to the maximum over its 4 lanes.
      float gm = fmaxf(lm, __shfl_xor(lm, 16, kWave));
      gm = fmaxf(gm, __shfl_xor(gm, 32, kWave));
      const float mn = fmaxf(m_ref, gm);
      const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m_ref - mn);
      l_lane *= alpha;
#pragma unroll
      for (int mb = 0; mb < kMD / 16; ++mb) acc[mb] *= alpha;
      m_ref = mn;
    }
    const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
    float p[KG][4];
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[kg][i] = fast_exp2(x[kg][i] + neg_m);
        l_lane += p[kg][i];
      }
    // O^T += V^T P^T.  k = 32: keys 4g4.. and 16 + 4g4..; k = 16: keys 4g4..
    if constexpr (KG == 2) {
      const uint32_t pw[4] = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                              pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
      // Lane (n, g4) addresses row 4g4 + n/4, dims 16mb + 4(n%4): the
      // transposing read returns keys 4g4..4g4+3 of dim 16mb + n.
      const __bf16* base = vt + (4 * g4 + n / 4) * kVRow + 4 * (n % 4);
#pragma unroll
      for (int mb = 0; mb < kMD / 16; ++mb) {
        const u32x2 lo = lds_read_tr16(base + 16 * mb);
        const u32x2 hi = lds_read_tr16(base + 16 * kVRow + 16 * mb);
        const uint32_t a[4] = {lo.x, lo.y, hi.x, hi.y};
        acc[mb] = mfma16(a, pw, acc[mb]);
      }
    } else {
      const uint32_t pw[2] = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3])};
      const __bf16* base = vt + (4 * g4 + n / 4) * kVRow + 4 * (n % 4);
#pragma unroll
      for (int mb = 0; mb < kMD / 16; ++mb) {
        const u32x2 lo = lds_read_tr16(base + 16 * mb);
        const uint32_t a[2] = {lo.x, lo.y};
        acc[mb] = mfma16k16(a, pw, acc[mb]);
      }
    }
  }

  // Units first .. first+count-1 (UBS tokens each) of a sequence of L
  // tokens, KV head g.
  // app >= 0: the run ends at the sequence's end and its last key is the
  // appended token (row app of the last tile).
  // win_ok: win_v already holds the run's first block-id window (blocks
  // 0..63; the run starts at the sequence's first unit).  nxt_v: a window
  // load for the next run, in flight; once the run's first two tiles are
  // requested the stream waits for it and parks it in this lane's slot of
  // nxt_lds, where the next run finds it (kept out of the registers that
  // outlive the run, so that nothing loaded is waited for between runs).
  template <bool NT>
  __device__ __forceinline__ void stream(const void* k_cache, const void* v_cache, const int32_t* tbl,
                                         int g, int num_kv_heads, int first, int count, int L,
                                         int app, int nxt_v, int* nxt_lds, int win_v, bool win_ok) {
    if (count <= 0) {
      nxt_lds[lane] = nxt_v;
      return;
    }
    const int64_t tile_bytes = (int64_t)BS * kMD * EB;
    const int64_t block_bytes = (int64_t)num_kv_heads * tile_bytes;
    const uint8_t* kh = (const uint8_t*)k_cache + (int64_t)g * tile_bytes;
    const uint8_t* vh = (const uint8_t*)v_cache + (int64_t)g * tile_bytes;
    // Keys of the run: key0 .. min(L, key0 + count*UBS); its blocks
    // blk0 .. blk_last.
    const int key0 = first * UBS;
    const int run_end = (first + count) * UBS < L ? (first + count) * UBS : L;
    const int blk0 = key0 / BS, blk_last = ((first + count) * UBS - 1) / BS;
    const int ntiles = (count * UBS + KEYS - 1) / KEYS;
    // Block ids of the run, 64 at a time, one per lane (the requests come
    // in non-decreasing order); past the run the last block is repeated
    // (its keys are masked).
    int bid_v = win_v, cached = win_ok ? 0 : -1;
    auto bid = [&](int blk) -> int {
      const int j = (blk < blk_last ? blk : blk_last) - blk0;
      const int chunk = j / kWave;
      if (chunk != cached) {
        const int jj = blk0 + chunk * kWave + lane;
        bid_v = tbl[jj < blk_last ? jj : blk_last];
        cached = chunk;
        // Wait for the window here, where it is reloaded (once per 64
        // blocks), so that the read below never waits for the tile loads.
        asm volatile("" : "+v"(bid_v));
      }
      return __builtin_amdgcn_readlane(bid_v, j % kWave);
    };
    auto limit = [&](int t) {
      const int lim = run_end - (key0 + t * KEYS);
      return lim < KEYS ? lim : KEYS;
    };
    auto k0_of = [&](int t) { return key0 + t * KEYS; };
    // Two tiles per pass, each loaded one tile ahead; the last one or two
    // tiles are taken after the loop, so every load is used and none is in
    // flight when the run ends.
    Tile ta, tb;
    load_tile<NT>(kh, vh, block_bytes, k0_of(0), bid, ta);
    int t = 0;
    for (; t + 3 <= ntiles; t += 2) {
      load_tile<NT>(kh, vh, block_bytes, k0_of(t + 1), bid, tb);
      nxt_lds[lane] = nxt_v;  // (no wait after the first pass)
      tile(ta, limit(t));
      load_tile<NT>(kh, vh, block_bytes, k0_of(t + 2), bid, ta);
      tile(tb, limit(t + 1));
    }
    if (t + 2 == ntiles) {
      load_tile<NT>(kh, vh, block_bytes, k0_of(t + 1), bid, tb);
      nxt_lds[lane] = nxt_v;
      tile(ta, limit(t));
      tile(tb, limit(t + 1), app);
    } else {
      nxt_lds[lane] = nxt_v;
      tile(ta, limit(t), app);
    }
  }

  // Sum of the head's probabilities over its 4 lanes.
  __device__ __forceinline__ float l_total() const {
    float l = l_lane + __shfl_xor(l_lane, 16, kWave);
    return l + __shfl_xor(l, 32, kWave);
  }
};

// The balanced split of decode_balanced_kernel, on the matrix-core engine.
template <typename KV, typename QT, int BS, int G>
__global__ __launch_bounds__(kMaxDecodeWaves * kWave, 2) void decode_balanced_mfma_kernel(
    void* __restrict__ out, float* __restrict__ part_acc, float* __restrict__ part_ml,
    int32_t* __restrict__ cuts, const void* __restrict__ query,
    const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens, int num_seqs,
    int max_blocks_per_seq, int num_kv_heads, int workers_per_head, float qk_scale_log2,
    float v_scale, int read_once_hint, SuffixStates sx, AppendTokens ap) {
  static_assert(std::is_same<QT, BF16>::value, "bf16 queries");
  using MA = MfmaAttn<KV, BS, G>;
  constexpr int D = kMD;
  constexpr int EB = Elem<KV>::bytes;
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[kMaxDecodeWaves][MA::kLdsElems];
  __shared__ __attribute__((aligned(16))) __bf16 new_lds[kMaxDecodeWaves][2][D];
  __shared__ int win_lds[kMaxDecodeWaves][kWave];  // the next run's block-id window
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int worker = blockIdx.x * (blockDim.x / kWave) + wv;
  const int g = worker % num_kv_heads, vw = worker / num_kv_heads;
  if (vw >= workers_per_head) return;
  const int num_heads = num_kv_heads * G;

  // The split's units: each sequence with keys counts its units of UBS
  // tokens plus kRunCost more that hold no keys (at its end), the cost of a
  // run's start, so that a worker whose range starts more runs is given
  // fewer keys.
  constexpr int kRunCost = 1;
  // Every length in one load where they fit one batch (the total, the
  // worker's first sequence and its window of lengths all come from it).
  const bool one_load = num_seqs <= kScanChunks * kWave;
  int raw[kScanChunks];
  if (one_load) load_all_lens(seq_lens, num_seqs, lane, raw);
  const int64_t T = one_load ? total_blocks_of(raw, MA::UBS, sx.skip, kRunCost)
                             : total_blocks(seq_lens, num_seqs, MA::UBS, sx.skip, lane, kRunCost);
  const int W = effective_workers(T, workers_per_head, MA::UBS);
  // The caller declared that no block is read twice: evict-first loads.
  const bool read_once = read_once_hint != 0;
  if (vw >= W) return;
  const int64_t start = worker_start(T, vw, W), end = worker_start(T, vw + 1, W);
  if (start >= end) return;
  int s;
  int64_t base;
  if (one_load) locate_block_of(raw, num_seqs, MA::UBS, sx.skip, start, s, base, kRunCost);
  else locate_block(seq_lens, num_seqs, MA::UBS, sx.skip, start, lane, s, base, kRunCost);
  const int tbl_skip = sx.skip / BS;  // table entries of the skipped tokens

  MA A;
  A.init(lane, qk_scale_log2, vt_lds[wv], new_lds[wv][0], new_lds[wv][1]);

  // Fused append: the run that reaches a sequence's end writes that
  // sequence's new token (position L-1) for this KV head into its pool slot
  // and keeps it in LDS as the tiles see it (an fp8 pool: quantised exactly
  // as the cache write does, then widened back), so its last tile uses it
  // instead of the slot's old contents.  Lanes 0..15 take 8 dims each.
  auto append_token = [&](int q, int L, const int32_t* row) {
    const int pos = L - 1;
    const int64_t bid = row[pos / BS];
    const int64_t slot_elem = ((bid * num_kv_heads + g) * BS + pos % BS) * (int64_t)D;
    if (lane < 16) {
      const int64_t src = ((int64_t)q * num_kv_heads + g) * D + 8 * lane;
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        const u32x4 w = *(const u32x4*)((const uint16_t*)(kv ? ap.v : ap.k) + src);
        uint8_t* pool = (uint8_t*)(kv ? v_cache : k_cache) + (slot_elem + 8 * lane) * EB;
        u32x4 tw = w;  // the 8 dims as the tiles see them (bf16)
        if constexpr (EB == 1) {
          const float sc = kv ? ap.v_scale : ap.k_scale;
          const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
          uint32_t b[2] = {0u, 0u};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = u2f((wd[j / 2] >> (16 * (j % 2))) << 16);
            b[j / 4] |= f32_to_e4m3fn(x / sc) << (8 * (j % 4));
          }
          *(u32x2*)pool = u32x2{b[0], b[1]};
          uint32_t lo0, hi0, lo1, hi1;
          lo0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[0], 1.0f, false));
          hi0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[0], 1.0f, true));
          lo1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[1], 1.0f, false));
          hi1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[1], 1.0f, true));
          tw = u32x4{lo0, hi0, lo1, hi1};
        } else {
          *(u32x4*)pool = w;
        }
        *(u32x4*)(new_lds[wv][kv] + 8 * lane) = tw;
      }
    }
  };
  // Lengths of sequences len_base .. len_base + 63, one per lane (past the
  // end: 0, or the last sequence's repeated), so that a run's start does not
  // wait for a load of its length.
  int len_base, len_v;
  if (one_load) {
    len_base = s & ~(kWave - 1);
    len_v = lens_chunk(raw, s / kWave);
  } else {
    len_base = s;
    len_v = seq_lens[min(s + lane, num_seqs - 1)];
    asm volatile("" : "+v"(len_v));
  }
  auto len_at = [&](int q) -> int {  // q >= len_base, wavefront-uniform
    if (q - len_base >= kWave) {
      len_base = q;
      len_v = seq_lens[min(q + lane, num_seqs - 1)];
      asm volatile("" : "+v"(len_v));
    }
    return __builtin_amdgcn_readlane(len_v, q - len_base);
  };
  // The block-id window (blocks 0..63) of the sequence win_s, loaded while
  // the previous run streamed and parked in win_lds; the next run uses it if
  // it is that sequence.
  int win_s = -1;
  int64_t pos = start;
  while (pos < end && s < num_seqs) {
    const int L = max(len_at(s) - sx.skip, 0);
    const int nblk = nblocks_of(L, MA::UBS);  // units of the split with keys
    const int64_t seg_end = base + (nblk > 0 ? nblk + kRunCost : 0);
    const int64_t vend = end < seg_end ? end : seg_end;  // this worker's end in the sequence
    if (nblk > 0 && pos - base < nblk) {
      const int b_lo = (int)(pos - base);
      const int b_hi = (int)(vend - base < nblk ? vend - base : nblk);
      const int64_t hq0 = (int64_t)s * num_heads + (int64_t)g * G;
      A.reset();
      A.load_q(query, hq0);
      const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq + tbl_skip;
      // The appended token's row in the run's last tile, if this run ends
      // the sequence.
      int app = -1;
      if (ap.k && b_hi == nblk) {
        append_token(s, L, row);
        app = (L - 1) - (b_lo * MA::UBS + ((b_hi - b_lo) * MA::UBS + MA::KEYS - 1) / MA::KEYS * MA::KEYS -
                         MA::KEYS);
      }
      // The next run's sequence: the next one with keys among the lengths at
      // hand (else none is prefetched).  Its window is requested now, one
      // load whatever the case (a harmless table read when there is none).
      int sn = -1, ln = 0;
      {
        const int rel = s + 1 - len_base;
        if (rel < kWave) {
          const uint64_t more = __builtin_amdgcn_ballot_w64(len_base + lane < num_seqs &&
                                                            len_v > sx.skip) &
                                (~0ull << rel);
          if (more) {
            sn = len_base + __builtin_ctzll(more);
            ln = __builtin_amdgcn_readlane(len_v, sn - len_base) - sx.skip;
          }
        }
      }
      const int last_n = ln > 0 ? (ln - 1) / BS : 0;
      int nxt_v = block_tables[(int64_t)(sn >= 0 ? sn : s) * max_blocks_per_seq + tbl_skip +
                               (lane < last_n ? lane : last_n)];
      const bool win_ok = win_s == s && b_lo == 0;
      const int win_v = win_ok ? win_lds[wv][lane] : 0;
      if (read_once)
        A.template stream<true>(k_cache, v_cache, row, g, num_kv_heads, b_lo, b_hi - b_lo, L, app,
                                nxt_v, win_lds[wv], win_v, win_ok);
      else
        A.template stream<false>(k_cache, v_cache, row, g, num_kv_heads, b_lo, b_hi - b_lo, L, app,
                                 nxt_v, win_lds[wv], win_v, win_ok);
      win_s = sn;
      const float l_tot = A.l_total();
      const bool whole = b_lo == 0 && b_hi == nblk;
      const int slot = pos == start ? 0 : 1;
      if (b_lo == 0 && lane == 0) {
        // The sequence's cut record, which the reduce and merge kernels read
        // (every shape of this engine takes the wavefront reduce, which needs
        // no per-worker merge tasks).
        const int code = (whole ? 1 : worker_of(T, base + nblk - 1, W) - vw + 1) * 2 + slot;
        cuts[2 * ((int64_t)s * num_kv_heads + g) + 0] = vw;
        cuts[2 * ((int64_t)s * num_kv_heads + g) + 1] = code;
      }
      if (A.n < G) {
        const int h = A.n;
        if (whole && !sx.acc) {
          const float inv = l_tot > 0.f ? v_scale / l_tot : 0.f;
#pragma unroll
          for (int mb = 0; mb < D / 16; ++mb) {
            const int d0 = 16 * mb + 4 * A.g4;
            const uint32_t w0 = pack_bf16(A.acc[mb][0] * inv, A.acc[mb][1] * inv);
            const uint32_t w1 = pack_bf16(A.acc[mb][2] * inv, A.acc[mb][3] * inv);
            *(u32x2*)((uint16_t*)out + (hq0 + h) * D + d0) = u32x2{w0, w1};
          }
        } else {
          // A piece of a cut sequence, or (suffix states kept) a whole one.
          const int64_t pslot = whole ? hq0 + h : ((int64_t)worker * 2 + slot) * G + h;
          float* dacc = whole ? sx.acc : part_acc;
          float* dml = whole ? sx.ml : part_ml;
#pragma unroll
          for (int mb = 0; mb < D / 16; ++mb)
            *(f32x4*)(dacc + pslot * D + 16 * mb + 4 * A.g4) = A.acc[mb];
          if (A.g4 == 0) {
            dml[pslot * 2 + 0] = A.m_ref;
            dml[pslot * 2 + 1] = l_tot;
          }
        }
      }
    }
    if (nblk > 0) pos = vend;
    if (pos >= seg_end) {
      base = seg_end;
      ++s;
    }
  }
}

// Fixed partitions on the matrix-core engine (the split-K decode with a
// separate log-sum-exp reduce): workgroup (x, g, s) takes partitions
// 4x .. 4x+3 of sequence s for KV head g, one per wavefront, each a run of
// partition_units units of the sequence streamed as the balanced split
// streams a run.  Its outputs are decode_kernel's: the output itself when
// the sequence has one partition, else per partition the output normalised
// by its own sum, times v_scale, and its (reference, sum) for
// lse_reduce_kernel.
template <typename KV, typename QT, int BS, int G>
__global__ __launch_bounds__(kMaxDecodeWaves * kWave, 2) void decode_partitioned_mfma_kernel(
    void* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
    const void* __restrict__ query, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, int max_blocks_per_seq, int num_kv_heads,
    int partition_units, int max_parts, float qk_scale_log2, float v_scale, int read_once_hint) {
  static_assert(std::is_same<QT, BF16>::value, "bf16 queries");
  using MA = MfmaAttn<KV, BS, G>;
  constexpr int D = kMD;
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[kMaxDecodeWaves][MA::kLdsElems];
  __shared__ int win_lds[kMaxDecodeWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int part = blockIdx.x * (blockDim.x / kWave) + wv, g = blockIdx.y, s = blockIdx.z;
  const int num_heads = num_kv_heads * G;
  const int L = seq_lens[s];
  const int nunits = nblocks_of(L, MA::UBS);
  const int nparts = nunits > partition_units ? (nunits + partition_units - 1) / partition_units : 1;
  if (part >= nparts) return;
  const int u0 = part * partition_units;
  const int u1 = u0 + partition_units < nunits ? u0 + partition_units : nunits;
  const int64_t hq0 = (int64_t)s * num_heads + (int64_t)g * G;
  MA A;
  A.init(lane, qk_scale_log2, vt_lds[wv]);
  A.reset();
  A.load_q(query, hq0);
  const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
  const int nxt_v = row[0];  // no run follows: a harmless table read, parked and unused
  if (read_once_hint)
    A.template stream<true>(k_cache, v_cache, row, g, num_kv_heads, u0, u1 - u0, L, -1, nxt_v,
                            win_lds[wv], 0, false);
  else
    A.template stream<false>(k_cache, v_cache, row, g, num_kv_heads, u0, u1 - u0, L, -1, nxt_v,
                             win_lds[wv], 0, false);
  const float l_tot = A.l_total();
  if (A.n < G) {
    const int64_t hq = hq0 + A.n;
    const float inv = l_tot > 0.f ? v_scale / l_tot : 0.f;
    if (nparts == 1) {
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb) {
        const int d0 = 16 * mb + 4 * A.g4;
        const uint32_t w0 = pack_bf16(A.acc[mb][0] * inv, A.acc[mb][1] * inv);
        const uint32_t w1 = pack_bf16(A.acc[mb][2] * inv, A.acc[mb][3] * inv);
        *(u32x2*)((uint16_t*)out + hq * D + d0) = u32x2{w0, w1};
      }
    } else {
      const int64_t st = hq * max_parts + part;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb)
        *(f32x4*)(part_o + st * D + 16 * mb + 4 * A.g4) = A.acc[mb] * inv;
      if (A.g4 == 0) {
        part_ml[st * 2 + 0] = A.m_ref;
        part_ml[st * 2 + 1] = l_tot;
      }
    }
  }
}

}  // namespace pa
