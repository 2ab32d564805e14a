// decode_no_alloc.hip — pa_decode without a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The split-K partial states, merge tasks and cut records that pa_decode
// keeps in the caller's workspace live here in a file-scope device array of
// PA_DECODE_NO_ALLOC_SCRATCH_BYTES.  Every GPU the library runs on holds its
// own copy of the array until the process ends, and every call on that GPU
// shares it: calls that overlap on one GPU (different streams, or another
// thread) race on it and must be serialised by the caller.  Nothing in it
// needs clearing between calls: the decode kernels write every partial
// state, merge task and cut record the reduce kernels read.
#include "pa_error.h"
#include "pa_internal.h"

#include <atomic>
#include <mutex>

#include <stdio.h>

namespace {

// In host code `scratch` names a host-side stand-in, not the device memory:
// its device address comes from hipGetSymbolAddress, once per device, and
// only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[PA_DECODE_NO_ALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[pa::kMaxDevices];

int32_t fail_msg(int32_t code, const char* msg) { return pa::record_error(code, msg); }

// The current device's address of `scratch`, looked up on the first call on
// that device (with that device current) and kept per device.
int32_t device_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= pa::kMaxDevices)
    return fail_msg(PA_ERR_HIP, "pa_decode_no_alloc: cannot identify the current device");
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        char buf[256];
        snprintf(buf, sizeof buf, "pa_decode_no_alloc: hipGetSymbolAddress failed on device %d: %s",
                 dev, hipGetErrorString(e));
        return fail_msg(PA_ERR_HIP, buf);
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PA_OK;
}

}  // namespace

extern "C" int32_t pa_decode_no_alloc(
    void* out, const void* query, int32_t q_dtype, int32_t num_seqs, int32_t num_heads,
    int32_t head_size, const void* k_cache, const void* v_cache, int32_t cache_dtype,
    int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, float scale,
    float k_scale, float v_scale, int32_t partition_size, int32_t flags, void* stream) {
  const size_t need = pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_size,
                                               max_seq_len, partition_size);
  if (need > (size_t)PA_DECODE_NO_ALLOC_SCRATCH_BYTES) {
    char buf[256];
    snprintf(buf, sizeof buf,
             "pa_decode_no_alloc: this split needs %zu bytes of scratch, more than the %zu the "
             "library holds per device (use pa_decode with a workspace)",
             need, (size_t)PA_DECODE_NO_ALLOC_SCRATCH_BYTES);
    return fail_msg(PA_ERR_WORKSPACE, buf);
  }
  void* ws = nullptr;
  if (need > 0) {
    if (int32_t r = device_scratch(&ws)) return r;
  }
  return pa::decode_call(out, query, q_dtype, num_seqs, num_heads, head_size, k_cache, v_cache,
                         cache_dtype, num_blocks, block_size, num_kv_heads, block_tables,
                         max_blocks_per_seq, seq_lens, max_seq_len, scale, k_scale, v_scale,
                         partition_size, flags, ws, need, stream, "pa_decode_no_alloc");
}
