// pa_api.hip — the C ABI of the library (declared in include/pa.h):
// host-side validation, workspace carving and launch dispatch.  No call
// allocates memory or synchronises; every error is detected on the host
// before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <string>

#include <string.h>

#include "pa_error.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

// Events for the next decode call's main kernel (pa_profile_next_decode).
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return PA_OK;
}

bool valid_dtype(int32_t d) { return d == PA_F32 || d == PA_BF16 || d == PA_FP8_E4M3; }

int32_t check_pool(const void* k_cache, const void* v_cache, int32_t cache_dtype,
                   int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_size) {
  if (!k_cache || !v_cache) return fail(PA_ERR_INVALID, "k_cache / v_cache is NULL");
  if (!valid_dtype(cache_dtype)) return fail(PA_ERR_INVALID, "unknown cache dtype %d", cache_dtype);
  if (num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_size <= 0)
    return fail(PA_ERR_INVALID,
                "pool sizes must be positive (num_blocks %d, block_size %d, num_kv_heads %d, "
                "head_size %d)", num_blocks, block_size, num_kv_heads, head_size);
  if (((uintptr_t)k_cache | (uintptr_t)v_cache) % 16 != 0)
    return fail(PA_ERR_INVALID, "k_cache / v_cache must be 16-byte aligned");
  if ((head_size * pa::dtype_bytes(cache_dtype)) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "a head row must be a multiple of 16 bytes (head_size %d)",
                head_size);
  return PA_OK;
}

int32_t hip_result(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  if (e == pa::kNotInstantiated)
    return fail(PA_ERR_UNSUPPORTED, "%s: shape not instantiated", what);
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A pointer argument must be aligned to `align` bytes (NULL passes; the
// callers check for it where it matters).
int32_t check_align(const void* p, size_t align, const char* name) {
  if ((uintptr_t)p % align != 0)
    return fail(PA_ERR_INVALID, "%s must be %zu-byte aligned", name, align);
  return PA_OK;
}

// Grid y and z extents are at most 65535 workgroups.
constexpr int64_t kMaxGridYZ = 65535;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Partitions of the longest sequence (1 when not split).
int64_t decode_max_parts(int32_t max_seq_len, int32_t partition_size) {
  if (partition_size <= 0 || max_seq_len <= partition_size) return 1;
  return ceil_div(max_seq_len, partition_size);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// PA_DECODE_WAVES=1|2|4 pins the wavefronts per decode workgroup (a tuning
// knob, read once); otherwise the library picks from the partition size.
int32_t decode_waves_override() {
  static const int32_t v = [] {
    const char* e = getenv("PA_DECODE_WAVES");
    const int x = e ? atoi(e) : 0;
    return (x == 1 || x == 2 || x == 4) ? x : 0;
  }();
  return v;
}

bool has_mfma_engine(int32_t q_dtype, int32_t cache_dtype, int32_t head_size, int32_t group) {
  return head_size == 128 && (group == 4 || group == 8) && q_dtype == PA_BF16 &&
         cache_dtype != PA_F32;
}

// The balanced decode's engine from the call's flags: a pinned engine if
// asked for; the vector engine when the tables share blocks (its 1 KiB row
// loads take fewer cache-line requests than the matrix-core operand loads
// when lines come from L2 and MALL rather than HBM); else the matrix cores
// where that engine is built.  Returns -1 for a pinned engine that is not
// built for the shape.
int32_t decode_engine(int32_t flags, int32_t q_dtype, int32_t cache_dtype, int32_t head_size,
                      int32_t group) {
  const bool has_mfma = has_mfma_engine(q_dtype, cache_dtype, head_size, group);
  if (flags & PA_DECODE_ENGINE_VALU) return pa::kEngineValu;
  if (flags & PA_DECODE_ENGINE_MFMA) return has_mfma ? pa::kEngineMfma : -1;
  if ((flags & PA_DECODE_SHARED) || !has_mfma) return pa::kEngineValu;
  return pa::kEngineMfma;
}

// Compute units of the current device, queried once per device.
using pa::kMaxDevices;
std::atomic<int32_t> g_device_cus[kMaxDevices];

int32_t device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int32_t c = g_device_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < kMaxDevices) g_device_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Wavefronts of the balanced split per compute unit of the current device,
// capped by the workspace layout: PA_BALANCED_WAVES_PER_CU pins it (a
// tuning knob, read once); by default 4 (one workgroup per CU) for the
// matrix-core engine, whose wavefronts keep two tiles in flight with little
// arithmetic between them, and 8 (two per SIMD, so that one's loads hide
// the other's score and softmax arithmetic) for the vector engine.  Whole
// workgroups per CU matter: a fraction leaves some CUs with one more
// workgroup than others for the whole kernel.
int32_t balanced_workers_for_device(int32_t engine) {
  static const int pinned = [] {
    const char* e = getenv("PA_BALANCED_WAVES_PER_CU");
    const int x = e ? atoi(e) : 0;
    return (x >= 1 && x <= 32) ? x : 0;
  }();
  const int per_cu = pinned ? pinned : (engine == pa::kEngineMfma ? 4 : 8);
  const int cus = device_cus();
  if (cus <= 0) return 0;
  const int64_t w = (int64_t)cus * per_cu;
  return (int32_t)(w < pa::kMaxBalancedWorkers ? w : pa::kMaxBalancedWorkers);
}

// The address a kernel uses for p: device memory as is, pinned host memory
// through its device mapping.  Anything else (pageable host memory, an
// unknown address) is refused, since a kernel touching it would fault.
int32_t device_view(const void* p, const char* name, const void** out) {
  hipPointerAttribute_t at;
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return fail(PA_ERR_INVALID, "%s is neither device memory nor pinned host memory", name);
  }
  if (at.type == hipMemoryTypeDevice) {
    *out = p;
    return PA_OK;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer && at.hostPointer) {
    *out = (const uint8_t*)at.devicePointer + ((const uint8_t*)p - (const uint8_t*)at.hostPointer);
    return PA_OK;
  }
  return fail(PA_ERR_INVALID, "%s is neither device memory nor pinned host memory", name);
}


}  // namespace

int32_t pa::record_error(int32_t code, const char* msg) {
  if (code == PA_OK) g_last_error.clear();
  else g_last_error = msg;
  return code;
}

// Validation and launch of a decode call, shared by pa_decode (caller's
// workspace) and pa_decode_no_alloc (the library's static scratch).
int32_t pa::decode_call(void* out, const void* query, int32_t q_dtype, int32_t num_seqs,
                           int32_t num_heads, int32_t head_size, const void* k_cache,
                           const void* v_cache, int32_t cache_dtype, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           int32_t max_seq_len, float scale, float k_scale, float v_scale,
                           int32_t partition_size, int32_t flags, void* workspace,
                           size_t workspace_bytes, void* stream, const char* who,
                           const pa::DecodeExtras* extra) {
  if (int32_t r = check_pool(k_cache, v_cache, cache_dtype, num_blocks, block_size, num_kv_heads,
                             head_size))
    return r;
  if (num_seqs < 0) return fail(PA_ERR_INVALID, "num_seqs %d < 0", num_seqs);
  if (num_heads <= 0 || num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "num_heads %d must be a positive multiple of num_kv_heads %d",
                num_heads, num_kv_heads);
  if (!valid_dtype(q_dtype)) return fail(PA_ERR_INVALID, "unknown query dtype %d", q_dtype);
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID, "max_blocks_per_seq must be > 0");
  if (max_seq_len < 0 || (int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID, "max_seq_len %d does not fit %d blocks of %d tokens", max_seq_len,
                max_blocks_per_seq, block_size);
  const bool balanced = partition_size == PA_PARTITION_BALANCED;
  if (!balanced && (partition_size < 0 || partition_size % block_size != 0))
    return fail(PA_ERR_INVALID,
                "partition_size %d must be PA_PARTITION_BALANCED, 0 or a multiple of block_size %d",
                partition_size, block_size);
  if (!(scale == scale) || !(k_scale == k_scale) || !(v_scale == v_scale))
    return fail(PA_ERR_INVALID, "scales must not be NaN");
  const int32_t known = PA_DECODE_READ_ONCE | PA_DECODE_SHARED | PA_DECODE_ENGINE_VALU |
                        PA_DECODE_ENGINE_MFMA;
  if ((flags & ~known) != 0) return fail(PA_ERR_INVALID, "unknown decode flags %#x", flags);
  if ((flags & PA_DECODE_READ_ONCE) && (flags & PA_DECODE_SHARED))
    return fail(PA_ERR_INVALID, "PA_DECODE_READ_ONCE and PA_DECODE_SHARED exclude each other");
  if ((flags & PA_DECODE_ENGINE_VALU) && (flags & PA_DECODE_ENGINE_MFMA))
    return fail(PA_ERR_INVALID, "two engines pinned");
  const int group = num_heads / num_kv_heads;
  if (!pa::decode_supported(q_dtype, cache_dtype, head_size, block_size, group))
    return fail(PA_ERR_UNSUPPORTED,
                "decode not built for q dtype %d, cache dtype %d, head_size %d, block_size %d, "
                "group %d", q_dtype, cache_dtype, head_size, block_size, group);
  const bool append = extra && extra->append.k;
  // The fused append runs on the matrix-core engine only.
  const int32_t engine =
      append ? ((flags & PA_DECODE_ENGINE_VALU) ? -1
                                                : decode_engine(PA_DECODE_ENGINE_MFMA, q_dtype,
                                                                cache_dtype, head_size, group))
             : decode_engine(flags, q_dtype, cache_dtype, head_size, group);
  if (engine < 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: the matrix-core decode engine is not built for this "
                "shape%s", who, append ? " (the fused append needs it)" : "");
  if (num_seqs == 0) return ok();
  if (!out || !query || !block_tables || !seq_lens)
    return fail(PA_ERR_INVALID, "out / query / block_tables / seq_lens is NULL");
  if (int32_t r = check_align(out, 16, "out")) return r;
  if (int32_t r = check_align(query, 16, "query")) return r;
  if (int32_t r = check_align(block_tables, 4, "block_tables")) return r;
  if (int32_t r = check_align(seq_lens, 4, "seq_lens")) return r;
  if (append) {
    if (!extra->append.v) return fail(PA_ERR_INVALID, "%s: v_new is NULL", who);
    if (int32_t r = check_align(extra->append.k, 16, "k_new")) return r;
    if (int32_t r = check_align(extra->append.v, 16, "v_new")) return r;
    if (cache_dtype == PA_FP8_E4M3 && (!(k_scale > 0.f) || !(v_scale > 0.f)))
      return fail(PA_ERR_INVALID, "%s: fp8 scales must be > 0", who);
  }
  const int64_t mp = balanced ? 1 : decode_max_parts(max_seq_len, partition_size);
  if (!balanced && (num_seqs > kMaxGridYZ || num_kv_heads > kMaxGridYZ))
    return fail(PA_ERR_INVALID,
                "%d sequences / %d KV heads exceed the %lld a partitioned decode grid takes "
                "(the balanced split takes any number of sequences)",
                num_seqs, num_kv_heads, (long long)kMaxGridYZ);
  if (mp > kMaxGridYZ) return fail(PA_ERR_INVALID, "too many partitions (%lld)", (long long)mp);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  int32_t workers = 0;
  int32_t* a_merges = nullptr;
  int32_t* a_cuts = nullptr;
  if (mp > 1 || balanced) {
    const size_t need = pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_size,
                                                 max_seq_len, partition_size);
    if (!workspace || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (int32_t r = check_align(workspace, 16, "workspace")) return r;
    const size_t n = balanced ? (size_t)pa::kMaxBalancedWorkers * 2 * (num_heads / num_kv_heads)
                              : (size_t)num_seqs * num_heads * mp;
    part_o = (float*)workspace;
    part_ml = (float*)((char*)workspace + align256(n * head_size * sizeof(float)));
    if (balanced) {
      a_merges = (int32_t*)((char*)part_ml + align256(n * 2 * sizeof(float)));
      a_cuts = (int32_t*)((char*)a_merges +
                          align256((size_t)pa::kMaxBalancedWorkers * 2 * sizeof(int32_t)));
      const int32_t w = balanced_workers_for_device(engine);
      if (w <= 0) return fail(PA_ERR_HIP, "cannot query the device's compute units");
      workers = (w / num_kv_heads) * num_kv_heads;
      if (workers < num_kv_heads) workers = num_kv_heads;
    }
  }
  pa::DecodeArgs a{};
  a.out = out; a.query = query; a.q_dtype = q_dtype;
  a.num_seqs = num_seqs; a.num_heads = num_heads; a.head_size = head_size;
  a.k_cache = k_cache; a.v_cache = v_cache; a.cache_dtype = cache_dtype;
  a.num_blocks = num_blocks; a.block_size = block_size; a.num_kv_heads = num_kv_heads;
  a.block_tables = block_tables; a.max_blocks_per_seq = max_blocks_per_seq;
  a.seq_lens = seq_lens; a.max_seq_len = max_seq_len;
  a.scale = scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.partition_blocks = mp > 1 ? partition_size / block_size : 0;
  a.max_parts = (int32_t)mp;
  a.part_o = part_o; a.part_ml = part_ml;
  a.num_waves = decode_waves_override();
  a.balanced_workers = workers;
  a.merges = a_merges;
  a.cuts = a_cuts;
  a.engine = engine;
  a.read_once = (flags & PA_DECODE_READ_ONCE) ? 1 : 0;
  a.prof_start = g_prof_start;
  a.prof_stop = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
  if (extra) {
    if (!balanced) return fail(PA_ERR_INVALID, "%s: runs in the balanced split", who);
    if (append) {
      a.append = extra->append;
      a.append.k_scale = k_scale;
      a.append.v_scale = v_scale;
    }
    a.suffix = extra->suffix;
    a.prefix_o = extra->prefix_o;
    a.prefix_ml = extra->prefix_ml;
    a.prefix_splits = extra->prefix_splits;
    if (extra->before_launch) {
      if (int32_t r = extra->before_launch(extra->ctx)) return r;
    }
  }
  a.stream = (hipStream_t)stream;
  hipError_t e;
  if (cache_dtype == PA_F32) e = pa::decode_f32(a);
  else if (cache_dtype == PA_BF16) e = pa::decode_bf16(a);
  else e = pa::decode_fp8(a);
  return hip_result(e, who);
}

extern "C" {

int32_t pa_version(void) { return 100; }

const char* pa_strerror(int32_t code) {
  switch (code) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID: return "PA_ERR_INVALID: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: combination not built";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime error";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: not enough free blocks";
    default: return "unknown pa error code";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

size_t pa_pool_bytes(int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                     int32_t head_size, int32_t cache_dtype) {
  if (num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_size <= 0 ||
      !valid_dtype(cache_dtype))
    return 0;
  return (size_t)num_blocks * num_kv_heads * block_size * head_size * pa::dtype_bytes(cache_dtype);
}

int32_t pa_cache_write(const void* key, const void* value, int32_t src_dtype, int32_t num_tokens,
                       void* k_cache, void* v_cache, int32_t cache_dtype, int32_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                       const int64_t* slot_mapping, float k_scale, float v_scale,
                       void* stream) {
  if (int32_t r = check_pool(k_cache, v_cache, cache_dtype, num_blocks, block_size, num_kv_heads,
                             head_size))
    return r;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "num_tokens %d < 0", num_tokens);
  if (!valid_dtype(src_dtype)) return fail(PA_ERR_INVALID, "unknown src dtype %d", src_dtype);
  if (src_dtype != cache_dtype && !(cache_dtype == PA_FP8_E4M3 && src_dtype != PA_FP8_E4M3))
    return fail(PA_ERR_UNSUPPORTED, "no cache write from dtype %d into dtype %d", src_dtype,
                cache_dtype);
  if (cache_dtype == PA_FP8_E4M3 && src_dtype != PA_FP8_E4M3 &&
      !(k_scale > 0.f && v_scale > 0.f && k_scale < INFINITY && v_scale < INFINITY))
    return fail(PA_ERR_INVALID, "fp8 scales must be finite and positive");
  if (num_tokens == 0) return ok();
  if (!key || !value || !slot_mapping)
    return fail(PA_ERR_INVALID, "key / value / slot_mapping is NULL");
  if (int32_t r = check_align(key, 16, "key")) return r;
  if (int32_t r = check_align(value, 16, "value")) return r;
  if (int32_t r = check_align(slot_mapping, 8, "slot_mapping")) return r;
  if ((head_size * pa::dtype_bytes(src_dtype)) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "a source head row must be a multiple of 16 bytes");
  pa::CacheWriteArgs a{key, value, src_dtype, num_tokens, k_cache, v_cache, cache_dtype,
                       num_blocks, block_size, num_kv_heads, head_size, slot_mapping, k_scale,
                       v_scale, (hipStream_t)stream};
  return hip_result(pa::cache_write(a), "pa_cache_write");
}

int32_t pa_copy_blocks(void* k_cache, void* v_cache, int32_t cache_dtype, int32_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                       const int64_t* block_mapping, int32_t num_pairs, void* stream) {
  if (int32_t r = check_pool(k_cache, v_cache, cache_dtype, num_blocks, block_size, num_kv_heads,
                             head_size))
    return r;
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return ok();
  if (!block_mapping) return fail(PA_ERR_INVALID, "block_mapping is NULL");
  if (int32_t r = check_align(block_mapping, 8, "block_mapping")) return r;
  pa::MoveBlocksArgs a{k_cache,    v_cache,      k_cache,      v_cache,
                       cache_dtype, num_blocks,  num_blocks,   block_size,
                       num_kv_heads, head_size,  block_mapping, num_pairs,
                       (hipStream_t)stream};
  return hip_result(pa::move_blocks(a), "pa_copy_blocks");
}

int32_t pa_swap_blocks(const void* src_k, const void* src_v, int32_t src_num_blocks, void* dst_k,
                       void* dst_v, int32_t dst_num_blocks, int32_t cache_dtype, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_size, const int64_t* block_mapping,
                       int32_t num_pairs, void* stream) {
  if (int32_t r = check_pool(src_k, src_v, cache_dtype, src_num_blocks, block_size, num_kv_heads,
                             head_size))
    return r;
  if (int32_t r = check_pool(dst_k, dst_v, cache_dtype, dst_num_blocks, block_size, num_kv_heads,
                             head_size))
    return r;
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "num_pairs %d < 0", num_pairs);
  const void *sk, *sv, *dk, *dv, *map = nullptr;
  if (int32_t r = device_view(src_k, "src_k", &sk)) return r;
  if (int32_t r = device_view(src_v, "src_v", &sv)) return r;
  if (int32_t r = device_view(dst_k, "dst_k", &dk)) return r;
  if (int32_t r = device_view(dst_v, "dst_v", &dv)) return r;
  if (num_pairs == 0) return ok();
  if (!block_mapping) return fail(PA_ERR_INVALID, "block_mapping is NULL");
  if (int32_t r = check_align(block_mapping, 8, "block_mapping")) return r;
  if (int32_t r = device_view(block_mapping, "block_mapping", &map)) return r;
  pa::MoveBlocksArgs a{sk, sv, (void*)dk, (void*)dv, cache_dtype, src_num_blocks, dst_num_blocks,
                       block_size, num_kv_heads, head_size, (const int64_t*)map, num_pairs,
                       (hipStream_t)stream};
  return hip_result(pa::move_blocks(a), "pa_swap_blocks");
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_size, int32_t max_seq_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      num_heads % num_kv_heads != 0)
    return 0;
  if (partition_size == PA_PARTITION_BALANCED) {
    const size_t n = (size_t)pa::kMaxBalancedWorkers * 2 * (num_heads / num_kv_heads);
    return align256(n * head_size * sizeof(float)) + align256(n * 2 * sizeof(float)) +
           align256((size_t)pa::kMaxBalancedWorkers * 2 * sizeof(int32_t)) +
           align256((size_t)num_seqs * num_kv_heads * 2 * sizeof(int32_t));
  }
  const int64_t mp = decode_max_parts(max_seq_len, partition_size);
  if (mp <= 1) return 0;
  const size_t n = (size_t)num_seqs * num_heads * mp;
  return align256(n * head_size * sizeof(float)) + align256(n * 2 * sizeof(float));
}

int32_t pa_profile_next_decode(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PA_ERR_INVALID, "pa_profile_next_decode: give both events or neither");
  g_prof_start = (hipEvent_t)start_event;
  g_prof_stop = (hipEvent_t)stop_event;
  return ok();
}

int32_t pa_decode(void* out, const void* query, int32_t q_dtype, int32_t num_seqs,
                  int32_t num_heads, int32_t head_size, const void* k_cache, const void* v_cache,
                  int32_t cache_dtype, int32_t num_blocks, int32_t block_size,
                  int32_t num_kv_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* seq_lens, int32_t max_seq_len, float scale, float k_scale,
                  float v_scale, int32_t partition_size, int32_t flags, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return pa::decode_call(out, query, q_dtype, num_seqs, num_heads, head_size, k_cache, v_cache,
                     cache_dtype, num_blocks, block_size, num_kv_heads, block_tables,
                     max_blocks_per_seq, seq_lens, max_seq_len, scale, k_scale, v_scale,
                     partition_size, flags, workspace, workspace_bytes, stream, "pa_decode");
}

int32_t pa_decode_append(void* out, const void* query, int32_t q_dtype, int32_t num_seqs,
                         int32_t num_heads, int32_t head_size, const void* k_new,
                         const void* v_new, const void* k_cache, const void* v_cache,
                         int32_t cache_dtype, int32_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                         int32_t max_seq_len, float scale, float k_scale, float v_scale,
                         int32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && !k_new) return fail(PA_ERR_INVALID, "pa_decode_append: k_new is NULL");
  pa::DecodeExtras x{};
  x.append.k = num_seqs > 0 ? k_new : nullptr;
  x.append.v = v_new;
  return pa::decode_call(out, query, q_dtype, num_seqs, num_heads, head_size, k_cache, v_cache,
                         cache_dtype, num_blocks, block_size, num_kv_heads, block_tables,
                         max_blocks_per_seq, seq_lens, max_seq_len, scale, k_scale, v_scale,
                         PA_PARTITION_BALANCED, flags, workspace, workspace_bytes, stream,
                         "pa_decode_append", num_seqs > 0 ? &x : nullptr);
}

// Splits of a shared prefix: enough (query tile, KV head, split) workgroups
// to give every compute unit one, each split a multiple of 128 keys (whole
// blocks and whole 64-key steps), at most kMaxPrefixSplits.
using pa::kMaxPrefixSplits;
constexpr int32_t kPrefixSplitQuantum = 128;

static int32_t prefix_split_len(int32_t prefix_len, int32_t num_seqs, int32_t group,
                                int32_t num_kv_heads, int32_t cus) {
  // PA_PREFIX_SPLITS pins the number of splits (a tuning knob, read once).
  static const int pinned = [] {
    const char* e = getenv("PA_PREFIX_SPLITS");
    const int x = e ? atoi(e) : 0;
    return (x >= 1 && x <= kMaxPrefixSplits) ? x : 0;
  }();
  const int64_t tiles = ceil_div((int64_t)num_seqs * group, 128) * num_kv_heads;
  const int64_t quanta = ceil_div(prefix_len, kPrefixSplitQuantum);
  int64_t want = tiles > 0 ? ceil_div(cus > 0 ? cus : 256, tiles) : 1;
  if (pinned) want = pinned;
  if (want > kMaxPrefixSplits) want = kMaxPrefixSplits;
  if (want > quanta) want = quanta;
  if (want < 1) want = 1;
  return (int32_t)(ceil_div(quanta, want) * kPrefixSplitQuantum);
}

size_t pa_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_size,
                                              int32_t prefix_len) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      num_heads % num_kv_heads != 0 || prefix_len < 0)
    return 0;
  const size_t bal = pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_size, 0,
                                              PA_PARTITION_BALANCED);
  const size_t rows = (size_t)num_seqs * num_heads;
  int64_t splits = ceil_div(prefix_len, kPrefixSplitQuantum);
  if (splits > kMaxPrefixSplits) splits = kMaxPrefixSplits;
  return bal + align256(rows * head_size * 4) + align256(rows * 2 * 4) +
         align256((size_t)splits * rows * head_size * 2) + align256((size_t)splits * rows * 2 * 4);
}

int32_t pa_decode_shared_prefix(void* out, const void* query, int32_t q_dtype, int32_t num_seqs,
                                int32_t num_heads, int32_t head_size, const void* k_cache,
                                const void* v_cache, int32_t cache_dtype, int32_t num_blocks,
                                int32_t block_size, int32_t num_kv_heads,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t max_seq_len, int32_t prefix_len,
                                float scale, float k_scale, float v_scale, int32_t flags,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t r = check_pool(k_cache, v_cache, cache_dtype, num_blocks, block_size, num_kv_heads,
                             head_size))
    return r;
  if (num_seqs < 0) return fail(PA_ERR_INVALID, "num_seqs %d < 0", num_seqs);
  if (num_heads <= 0 || num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "num_heads %d must be a positive multiple of num_kv_heads %d",
                num_heads, num_kv_heads);
  if (prefix_len < 0 || prefix_len % block_size != 0 || prefix_len > max_seq_len)
    return fail(PA_ERR_INVALID,
                "prefix_len %d must be a multiple of block_size %d in [0, max_seq_len %d]",
                prefix_len, block_size, max_seq_len);
  if (num_kv_heads > kMaxGridYZ)
    return fail(PA_ERR_INVALID, "%d KV heads exceed the grid's %lld", num_kv_heads,
                (long long)kMaxGridYZ);
  const int group = num_heads / num_kv_heads;
  if (prefix_len > 0 && !pa::prefill_supported(q_dtype, cache_dtype, head_size, block_size, group))
    return fail(PA_ERR_UNSUPPORTED,
                "the shared-prefix product is not built for q dtype %d, cache dtype %d, "
                "head_size %d, block_size %d, group %d",
                q_dtype, cache_dtype, head_size, block_size, group);
  if (num_seqs == 0) return ok();
  const size_t need = pa_decode_shared_prefix_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                             head_size, prefix_len);
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (int32_t r = check_align(workspace, 16, "workspace")) return r;
  if (!query || !block_tables) return fail(PA_ERR_INVALID, "query / block_tables is NULL");
  if (int32_t r = check_align(query, 16, "query")) return r;
  if (int32_t r = check_align(block_tables, 4, "block_tables")) return r;
  // Carve: the balanced split's workspace, the suffix states, the prefix states.
  const size_t bal = pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_size, 0,
                                              PA_PARTITION_BALANCED);
  const size_t rows = (size_t)num_seqs * num_heads;
  char* p = (char*)workspace + bal;
  pa::DecodeExtras ex{};
  ex.suffix.skip = prefix_len;
  ex.suffix.acc = (float*)p;
  p += align256(rows * head_size * 4);
  ex.suffix.ml = (float*)p;
  p += align256(rows * 2 * 4);
  uint16_t* pre_o = (uint16_t*)p;
  int32_t splits = 0;
  int32_t split_len = 0;
  if (prefix_len > 0) {
    split_len = prefix_split_len(prefix_len, num_seqs, group, num_kv_heads, device_cus());
    splits = (int32_t)ceil_div(prefix_len, split_len);
  }
  p += align256((size_t)splits * rows * head_size * 2);
  float* pre_ml = (float*)p;
  ex.prefix_o = pre_o;
  ex.prefix_ml = pre_ml;
  ex.prefix_splits = splits;
  // The prefix: every sequence's query against the shared blocks of row 0,
  // enqueued by decode_call once all its checks have passed.
  pa::PrefillArgs a{};
  if (splits > 0) {
    a.query = query; a.q_dtype = q_dtype;
    a.num_tokens = num_seqs; a.num_heads = num_heads; a.head_size = head_size;
    a.k_cache = k_cache; a.v_cache = v_cache; a.cache_dtype = cache_dtype;
    a.num_blocks = num_blocks; a.block_size = block_size; a.num_kv_heads = num_kv_heads;
    a.block_tables = block_tables; a.max_blocks_per_seq = max_blocks_per_seq;
    a.scale = scale; a.k_scale = k_scale; a.v_scale = v_scale;
    a.prefix.o = pre_o;
    a.prefix.ml = pre_ml;
    a.prefix.split_len = split_len;
    a.prefix.prefix_len = prefix_len;
    a.stream = (hipStream_t)stream;
    ex.before_launch = [](const void* ctx) -> int32_t {
      return hip_result(pa::prefill(*(const pa::PrefillArgs*)ctx), "pa_decode_shared_prefix");
    };
    ex.ctx = &a;
  }
  // The suffixes through the balanced split, then the merge.
  return pa::decode_call(out, query, q_dtype, num_seqs, num_heads, head_size, k_cache, v_cache,
                         cache_dtype, num_blocks, block_size, num_kv_heads, block_tables,
                         max_blocks_per_seq, seq_lens, max_seq_len, scale, k_scale, v_scale,
                         PA_PARTITION_BALANCED, flags, workspace, bal, stream,
                         "pa_decode_shared_prefix", &ex);
}

int32_t pa_prefill_chunk(void* out, const void* query, int32_t q_dtype, int32_t num_tokens,
                         int32_t num_heads, int32_t head_size, const int32_t* query_start_loc,
                         int32_t num_chunks, int32_t max_query_len, const void* k_cache,
                         const void* v_cache, int32_t cache_dtype, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, float scale,
                         float k_scale, float v_scale, void* stream) {
  if (int32_t r = check_pool(k_cache, v_cache, cache_dtype, num_blocks, block_size, num_kv_heads,
                             head_size))
    return r;
  if (num_tokens < 0 || num_chunks < 0 || max_query_len < 0)
    return fail(PA_ERR_INVALID, "negative size");
  if (num_heads <= 0 || num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "num_heads %d must be a positive multiple of num_kv_heads %d",
                num_heads, num_kv_heads);
  if (!valid_dtype(q_dtype)) return fail(PA_ERR_INVALID, "unknown query dtype %d", q_dtype);
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID, "max_blocks_per_seq must be > 0");
  if (!(scale == scale) || !(k_scale == k_scale) || !(v_scale == v_scale))
    return fail(PA_ERR_INVALID, "scales must not be NaN");
  const int group = num_heads / num_kv_heads;
  if (!pa::prefill_supported(q_dtype, cache_dtype, head_size, block_size, group))
    return fail(PA_ERR_UNSUPPORTED,
                "prefill not built for q dtype %d, cache dtype %d, head_size %d, block_size %d, "
                "group %d", q_dtype, cache_dtype, head_size, block_size, group);
  if (num_tokens == 0 || num_chunks == 0) return ok();
  if (!out || !query || !query_start_loc || !block_tables || !seq_lens)
    return fail(PA_ERR_INVALID, "a device array argument is NULL");
  if (int32_t r = check_align(out, 16, "out")) return r;
  if (int32_t r = check_align(query, 16, "query")) return r;
  if (int32_t r = check_align(query_start_loc, 4, "query_start_loc")) return r;
  if (int32_t r = check_align(block_tables, 4, "block_tables")) return r;
  if (int32_t r = check_align(seq_lens, 4, "seq_lens")) return r;
  if (num_chunks > kMaxGridYZ || num_kv_heads > kMaxGridYZ)
    return fail(PA_ERR_INVALID, "%d chunks / %d KV heads exceed the grid's %lld", num_chunks,
                num_kv_heads, (long long)kMaxGridYZ);
  pa::PrefillArgs a{};
  a.out = out; a.query = query; a.q_dtype = q_dtype;
  a.num_tokens = num_tokens; a.num_heads = num_heads; a.head_size = head_size;
  a.query_start_loc = query_start_loc; a.num_chunks = num_chunks; a.max_query_len = max_query_len;
  a.k_cache = k_cache; a.v_cache = v_cache; a.cache_dtype = cache_dtype;
  a.num_blocks = num_blocks; a.block_size = block_size; a.num_kv_heads = num_kv_heads;
  a.block_tables = block_tables; a.max_blocks_per_seq = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.scale = scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.stream = (hipStream_t)stream;
  return hip_result(pa::prefill(a), "pa_prefill_chunk");
}

}  // extern "C"

namespace pa {

bool decode_supported(int32_t q_dtype, int32_t cache_dtype, int head_size, int block_size,
                      int group) {
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
  const bool bs_ok = block_size == 16 || block_size == 32 || block_size == 64 || block_size == 128;
  if (!g_ok || !bs_ok) return false;
  if (q_dtype == PA_F32 && cache_dtype == PA_F32) return head_size == 64;
  if (q_dtype == PA_BF16 && (cache_dtype == PA_BF16 || cache_dtype == PA_FP8_E4M3))
    return head_size == 64 || head_size == 128;
  return false;
}

}  // namespace pa
