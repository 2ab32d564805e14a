// pa_internal.h — host-side argument bundles and launcher declarations
// shared between the C ABI (pa_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/pa.h"
#include "pa_device.h"

namespace pa {

inline int dtype_bytes(int32_t dt) { return dt == PA_F32 ? 4 : dt == PA_BF16 ? 2 : 1; }

// Upper bound on the wavefronts of the balanced split; the workspace of a
// balanced decode holds two partial states per wavefront.
constexpr int kMaxBalancedWorkers = 4096;

// What a launcher returns for a shape it has no kernel for (the C ABI maps
// it, and only it, to PA_ERR_UNSUPPORTED).
constexpr hipError_t kNotInstantiated = hipErrorNotSupported;

struct CacheWriteArgs {
  const void* key;
  const void* value;
  int32_t src_dtype;
  int32_t num_tokens;
  void* k_cache;
  void* v_cache;
  int32_t cache_dtype;
  int32_t num_blocks, block_size, num_kv_heads, head_size;
  const int64_t* slot_mapping;
  float k_scale, v_scale;
  hipStream_t stream;
};

// Whole-block moves between two pools of the same geometry (the same pool
// for the copy-on-write copy; the HBM pool and a pinned host pool for swap).
struct MoveBlocksArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  int32_t cache_dtype;
  int32_t src_blocks, dst_blocks, block_size, num_kv_heads, head_size;
  const int64_t* block_mapping;
  int32_t num_pairs;
  hipStream_t stream;
};

// Suffix mode of the balanced kernels (the part of a shared-prefix decode
// past the prefix): every sequence is walked from token `skip` (a multiple
// of the pool block size; its table row from entry skip / block size), and
// when `acc` is set, a sequence a worker holds whole leaves its
// unnormalised state in acc[s * num_heads + h][D], ml[...][2] instead of
// its output (cut sequences leave their pieces as usual), for a merge with
// the prefix's states.
// Fused append (pa_decode_append): each sequence's newest token (position
// seq_len - 1) arrives as bf16 K and V rows [num_seqs][num_kv_heads][head
// size]; the decode kernel writes them into the pool slot the table gives
// (quantised with k_scale / v_scale for an fp8 pool, as the cache write
// does) and attends to them in place of the slot's old contents.  Null k:
// a plain decode.
struct AppendTokens {
  const void* k;
  const void* v;
  float k_scale, v_scale;
};

struct SuffixStates {
  int skip;
  float* acc;
  float* ml;
};

struct DecodeArgs {
  void* out;
  const void* query;
  int32_t q_dtype;
  int32_t num_seqs, num_heads, head_size;
  const void* k_cache;
  const void* v_cache;
  int32_t cache_dtype;
  int32_t num_blocks, block_size, num_kv_heads;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  float scale, k_scale, v_scale;
  int32_t partition_blocks;  // blocks per partition; 0 = whole sequence
  int32_t max_parts;         // grid extent over partitions
  float* part_o;             // [num_seqs][num_heads][max_parts][head_size]
  float* part_ml;            // [num_seqs][num_heads][max_parts][2]
  int32_t* merges;           // balanced split: per wavefront {sequence or -1, 2*pieces+slot}
  int32_t* cuts;             // balanced split: per (sequence, KV head) {first worker, 2*pieces+slot}
  int32_t num_waves;         // wavefronts per workgroup; 0 = chosen from the partition size
  int32_t balanced_workers;  // > 0: balanced split over this many wavefronts (multiple of Hkv)
  int32_t engine;            // balanced split: kEngineValu or kEngineMfma (where compiled)
  int32_t read_once;         // 1: no block is read twice in the call (evict-first loads)
  // Shared-prefix decode: the balanced split runs in suffix mode, and a
  // merge kernel joins each sequence's suffix state with prefix_splits
  // prefix states into the output: each split's output normalised by its
  // own sum, bf16 ([(split * num_seqs + s) * num_heads + h][head_size]),
  // and its (reference, sum), fp32 ([...][2]).
  SuffixStates suffix;
  AppendTokens append;
  const uint16_t* prefix_o;
  const float* prefix_ml;
  int32_t prefix_splits;
  // Measurement (pa_profile_next_decode): events recorded right before and
  // after the main decode kernel, or null.
  hipEvent_t prof_start, prof_stop;
  hipStream_t stream;
};

// Launches the main decode kernel of a call, between the call's profiling
// events when it has them (hipExtLaunchKernelGGL records them on the
// stream immediately around this one dispatch).
template <typename... KArgs, typename... Args>
inline void launch_main(const DecodeArgs& a, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                        Args... args) {
  if (a.prof_start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, a.stream, a.prof_start, a.prof_stop, 0,
                          args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, a.stream, args...);
}

// Engines of the balanced decode: the wavefront (vector ALU) engine, or the
// matrix-core engine for head size 128 with groups of 4 or 8.
constexpr int32_t kEngineValu = 0, kEngineMfma = 1;

struct PrefillArgs {
  void* out;
  const void* query;
  int32_t q_dtype;
  int32_t num_tokens, num_heads, head_size;
  const int32_t* query_start_loc;
  int32_t num_chunks, max_query_len;
  const void* k_cache;
  const void* v_cache;
  int32_t cache_dtype;
  int32_t num_blocks, block_size, num_kv_heads;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* seq_lens;
  float scale, k_scale, v_scale;
  // Prefix mode (o != nullptr): num_tokens decode queries against the
  // first prefix_len keys of block_tables row 0, non-causal, in splits of
  // split_len keys; the splits' states go to o / ml (see prefill_kernels).
  struct {
    uint16_t* o;
    float* ml;
    int32_t split_len, prefix_len;
  } prefix;
  hipStream_t stream;
};

hipError_t cache_write(const CacheWriteArgs& a);
hipError_t move_blocks(const MoveBlocksArgs& a);

// Decode launchers, one per (query, cache) dtype pair; each dispatches on
// head_size, block_size and group size.  Return kNotInstantiated for a
// shape that was not instantiated.
hipError_t decode_f32(const DecodeArgs& a);
hipError_t decode_bf16(const DecodeArgs& a);
hipError_t decode_fp8(const DecodeArgs& a);
bool decode_supported(int32_t q_dtype, int32_t cache_dtype, int head_size, int block_size,
                      int group);

hipError_t prefill(const PrefillArgs& a);

// Most splits the keys of a shared prefix are cut into (the merge kernel
// holds one state per split in registers).
constexpr int kMaxPrefixSplits = 16;

// Devices the library keeps per-device state for (ids 0 .. kMaxDevices-1).
constexpr int kMaxDevices = 64;

// Host validation, workspace carving and launch of a decode call (the body
// of pa_decode; `who` names the entry point in error messages).
int32_t decode_call(void* out, const void* query, int32_t q_dtype, int32_t num_seqs,
                    int32_t num_heads, int32_t head_size, const void* k_cache,
                    const void* v_cache, int32_t cache_dtype, int32_t num_blocks,
                    int32_t block_size, int32_t num_kv_heads, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                    float scale, float k_scale, float v_scale, int32_t partition_size,
                    int32_t flags, void* workspace, size_t workspace_bytes, void* stream,
                    const char* who, const struct DecodeExtras* extra = nullptr);

// What a shared-prefix decode adds to the balanced split (see DecodeArgs).
struct DecodeExtras {
  SuffixStates suffix;
  AppendTokens append;
  const uint16_t* prefix_o;
  const float* prefix_ml;
  int32_t prefix_splits;
  // Called after every host check passed, before the decode kernels are
  // enqueued (the shared-prefix product goes first on the stream).
  int32_t (*before_launch)(const void* ctx);
  const void* ctx;
};
bool prefill_supported(int32_t q_dtype, int32_t cache_dtype, int head_size, int block_size,
                       int group);

}  // namespace pa
