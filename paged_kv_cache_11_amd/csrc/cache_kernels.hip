// cache_kernels.hip — the slot-mapped cache write and the block copy.
//
// Cache write: "vLLM：大语言模型推理与服务库" §4.3 item 2 — each new token's
// K/V goes into its sequence's current block; the block (and so the slot)
// was chosen by the caller's allocator.  Block copy: the copy-on-write step
// of the fork/append/free primitives in "vLLM 高性能大语言模型推理引擎深度
// 技术评估与分布式架构展望" and "vLLM 深度解析" §3.1.  Block swap: the same
// whole-block move between the HBM pool and a pool in pinned host memory,
// the SWAP mode of preemption (the first of those pages, its section on
// preemption; "vLLM 深度解析" §3.2, preemption strategies).
//
// All move 16-byte chunks: in the cache write every thread moves one chunk
// of the destination, so each wavefront writes 1 KiB of contiguous pool (one
// token row of a head is head_size contiguous elements); a block move
// streams one block of all heads, which is contiguous.
#include "pa_internal.h"

namespace pa {

// One thread per 16-byte destination chunk; chunk c of row (t, h).
template <typename SRC, typename DST>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const int64_t* __restrict__ slot_mapping, int64_t total_chunks, int64_t pool_slots,
    int chunks_per_row, int num_kv_heads, int block_size, int head_size,
    float k_scale, float v_scale) {
  constexpr int SB = Elem<SRC>::bytes, DB = Elem<DST>::bytes;
  constexpr int EPC = 16 / DB;  // elements per destination chunk
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total_chunks) return;
  const int c = (int)(i % chunks_per_row);
  const int64_t row = i / chunks_per_row;        // t * Hkv + h
  const int h = (int)(row % num_kv_heads);
  const int64_t t = row / num_kv_heads;
  const int64_t slot = slot_mapping[t];
  const int64_t src_elem = row * (int64_t)head_size + (int64_t)c * EPC;
  // The source chunks do not depend on the slot: load them before testing
  // it, so the two loads overlap.
  constexpr int NSRC = EPC * SB / 16;  // 16-byte source vectors per chunk
  u32x4 ks[NSRC], vs[NSRC];
#pragma unroll
  for (int j = 0; j < NSRC; ++j) {
    ks[j] = ((const u32x4*)(key + src_elem * SB))[j];
    vs[j] = ((const u32x4*)(value + src_elem * SB))[j];
  }
  // A negative slot is a padding token; one past the pool is a caller's
  // error that must not write outside it.  Both are skipped.
  if (slot < 0 || slot >= pool_slots) return;
  const int64_t blk = slot / block_size;
  const int off = (int)(slot % block_size);
  const int64_t dst_elem =
      ((blk * num_kv_heads + h) * block_size + off) * (int64_t)head_size + (int64_t)c * EPC;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const u32x4* src = kv ? vs : ks;
    uint8_t* dst = (kv ? v_cache : k_cache) + dst_elem * DB;
    if constexpr (std::is_same<SRC, DST>::value) {
      *(u32x4*)dst = src[0];
    } else {
      static_assert(std::is_same<DST, FP8>::value, "only fp8 caches quantise");
      const float sc = kv ? v_scale : k_scale;
      float x[EPC];
#pragma unroll
      for (int j = 0; j < NSRC; ++j) Vec<SRC>::to_f32(src[j], x + j * Vec<SRC>::n);
      uint32_t out[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t b = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) b |= f32_to_e4m3fn(x[4 * j + k] / sc) << (8 * k);
        out[j] = b;
      }
      *(u32x4*)dst = u32x4{out[0], out[1], out[2], out[3]};
    }
  }
}

template <typename SRC, typename DST>
static hipError_t launch_cache_write(const CacheWriteArgs& a) {
  const int chunks_per_row = a.head_size * Elem<DST>::bytes / 16;
  const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * chunks_per_row;
  const int64_t nblocks = (total + 255) / 256;
  hipLaunchKernelGGL((cache_write_kernel<SRC, DST>), dim3((unsigned)nblocks), dim3(256), 0,
                     a.stream, (const uint8_t*)a.key, (const uint8_t*)a.value,
                     (uint8_t*)a.k_cache, (uint8_t*)a.v_cache, a.slot_mapping, total,
                     (int64_t)a.num_blocks * a.block_size, chunks_per_row, a.num_kv_heads, a.block_size, a.head_size, a.k_scale,
                     a.v_scale);
  return hipGetLastError();
}

hipError_t cache_write(const CacheWriteArgs& a) {
  if (a.src_dtype == a.cache_dtype) {
    switch (a.cache_dtype) {
      case PA_F32: return launch_cache_write<F32, F32>(a);
      case PA_BF16: return launch_cache_write<BF16, BF16>(a);
      default: return launch_cache_write<FP8, FP8>(a);
    }
  }
  if (a.src_dtype == PA_F32) return launch_cache_write<F32, FP8>(a);
  return launch_cache_write<BF16, FP8>(a);
}

// grid: x = chunk group of one block, y = pair, z = 0 (K) / 1 (V).
// Whole-block moves: work item (pair, pool) is one block of all heads of K
// or V, block_chunks 16-byte chunks, split over wgs_per_block workgroups.
// Each thread issues kMoveUnroll loads before its stores, so a wavefront
// keeps 4 KiB in flight: what reads of pinned host memory across the host
// link need to cover their latency.  Pairs naming a block outside either
// pool are skipped.
constexpr int kMoveUnroll = 4;
constexpr int kMoveThreads = 256;

__global__ __launch_bounds__(kMoveThreads) void move_blocks_kernel(
    const uint8_t* __restrict__ src_k, const uint8_t* __restrict__ src_v,
    uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v,
    const int64_t* __restrict__ block_mapping, int64_t src_blocks, int64_t dst_blocks,
    int64_t block_chunks, int wgs_per_block) {
  const int64_t item = blockIdx.x / wgs_per_block;
  const int part = (int)(blockIdx.x % wgs_per_block);
  const int64_t pair = item >> 1;
  const bool is_v = item & 1;
  const int64_t src = block_mapping[2 * pair], dst = block_mapping[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const u32x4* s = (const u32x4*)(is_v ? src_v : src_k) + src * block_chunks;
  u32x4* d = (u32x4*)(is_v ? dst_v : dst_k) + dst * block_chunks;
  constexpr int64_t kPerPass = (int64_t)kMoveThreads * kMoveUnroll;
  for (int64_t base = part * kPerPass; base < block_chunks; base += wgs_per_block * kPerPass) {
    u32x4 r[kMoveUnroll];
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
      const int64_t c = base + u * kMoveThreads + threadIdx.x;
      if (c < block_chunks) r[u] = s[c];
    }
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
      const int64_t c = base + u * kMoveThreads + threadIdx.x;
      if (c < block_chunks) d[c] = r[u];
    }
  }
}

hipError_t move_blocks(const MoveBlocksArgs& a) {
  const int64_t block_bytes =
      (int64_t)a.num_kv_heads * a.block_size * a.head_size * dtype_bytes(a.cache_dtype);
  const int64_t block_chunks = block_bytes / 16;
  const int64_t per_pass = (int64_t)kMoveThreads * kMoveUnroll;
  int64_t wgs = (block_chunks + per_pass - 1) / per_pass;
  if (wgs > 16) wgs = 16;
  const int64_t grid = (int64_t)a.num_pairs * 2 * wgs;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(move_blocks_kernel, dim3((unsigned)grid), dim3(kMoveThreads), 0, a.stream,
                     (const uint8_t*)a.src_k, (const uint8_t*)a.src_v, (uint8_t*)a.dst_k,
                     (uint8_t*)a.dst_v, a.block_mapping, (int64_t)a.src_blocks,
                     (int64_t)a.dst_blocks, block_chunks, (int)wgs);
  return hipGetLastError();
}

}  // namespace pa
