/* pa_device_client.c: the device calls of the library's C ABI from plain C.
 *
 * No Python and no torch: device memory comes from hipMalloc, the calls run
 * on the default stream, and inputs are drawn from a 32-bit linear
 * congruential generator (x <- 1664525 x + 1013904223, value
 * (x >> 8) * 2^-23 - 1, exact in fp32) that the test repeats on the host.
 * Scenario, fp32 pools (8 query / 2 KV heads, head size 64, block 16):
 *   1. a block manager places three sequences of 1, 37 and 100 tokens;
 *      pa_cache_write writes their K/V; pa_decode with 32-token partitions
 *      (split-K and the log-sum-exp reduce) answers one query each;
 *   2. sequence 2 is forked into 3 and both get one more token: the
 *      manager's copy-on-write pair goes through pa_copy_blocks, the two
 *      new tokens through pa_cache_write, and pa_decode in one partition
 *      answers the two sequences.
 * Every result is printed as "name v1 v2 ..." for the test to compare with
 * the oracle.  Exit status 0 unless a call fails. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "pa.h"

#define HQ 8
#define HKV 2
#define D 64
#define BS 16
#define NB 24
#define MAXB 8

static uint32_t lcg = 12345u;

static float next_value(void) {
  lcg = lcg * 1664525u + 1013904223u;
  return (float)(lcg >> 8) * (1.0f / 8388608.0f) - 1.0f;
}

static void fill(float* x, size_t n) {
  size_t i;
  for (i = 0; i < n; ++i) x[i] = next_value();
}

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static int pa_ok(int32_t rc, const char* what) {
  if (rc != PA_OK) {
    fprintf(stderr, "%s: %s (%s)\n", what, pa_strerror(rc), pa_last_error());
    return 0;
  }
  return 1;
}

static void print_i64(const char* name, const int64_t* v, int n) {
  int i;
  printf("%s", name);
  for (i = 0; i < n; ++i) printf(" %lld", (long long)v[i]);
  printf("\n");
}

static void print_f32(const char* name, const float* v, int n) {
  int i;
  printf("%s", name);
  for (i = 0; i < n; ++i) printf(" %.9g", v[i]);
  printf("\n");
}

/* Copies n bytes to a new device buffer. */
static void* to_device(const void* host, size_t n) {
  void* d = NULL;
  if (!hip_ok(hipMalloc(&d, n), "hipMalloc")) return NULL;
  if (!hip_ok(hipMemcpy(d, host, n, hipMemcpyHostToDevice), "hipMemcpy")) return NULL;
  return d;
}

int main(void) {
  const int32_t lens0[3] = {1, 37, 100};
  const int64_t ids[3] = {0, 1, 2}, ids2[2] = {2, 3};
  int64_t slots[138], slots2[2], cow[4];
  int32_t tables[3 * MAXB], lens[3], ncow = 0, i, total = 0;
  float *k0, *v0, *q1, *out1, kn[2 * HKV * D], vn[2 * HKV * D], q2[2 * HQ * D], out2[2 * HQ * D];
  void *kpool = NULL, *vpool = NULL, *dk, *dv, *dslots, *dq, *dout, *dtables, *dlens, *ws = NULL;
  size_t pool_bytes = pa_pool_bytes(NB, HKV, BS, D, PA_F32), ws_bytes;
  pa_block_manager* bm = pa_bm_create(NB, BS);
  if (!bm) return 1;

  /* 1. three sequences, one decode with split-K. */
  for (i = 0; i < 3; ++i) {
    if (!pa_ok(pa_bm_add(bm, ids[i], lens0[i], slots + total), "pa_bm_add")) return 1;
    total += lens0[i];
  }
  print_i64("slots", slots, total);
  k0 = (float*)malloc(sizeof(float) * total * HKV * D);
  v0 = (float*)malloc(sizeof(float) * total * HKV * D);
  q1 = (float*)malloc(sizeof(float) * 3 * HQ * D);
  out1 = (float*)malloc(sizeof(float) * 3 * HQ * D);
  if (!k0 || !v0 || !q1 || !out1) return 1;
  fill(k0, (size_t)total * HKV * D);
  fill(v0, (size_t)total * HKV * D);
  fill(q1, 3 * HQ * D);

  if (!hip_ok(hipMalloc(&kpool, pool_bytes), "hipMalloc") ||
      !hip_ok(hipMalloc(&vpool, pool_bytes), "hipMalloc"))
    return 1;
  dk = to_device(k0, sizeof(float) * total * HKV * D);
  dv = to_device(v0, sizeof(float) * total * HKV * D);
  dslots = to_device(slots, sizeof(int64_t) * total);
  if (!dk || !dv || !dslots) return 1;
  if (!pa_ok(pa_cache_write(dk, dv, PA_F32, total, kpool, vpool, PA_F32, NB, BS, HKV, D, dslots,
                            1.0f, 1.0f, NULL), "pa_cache_write"))
    return 1;

  if (!pa_ok(pa_bm_block_tables(bm, 3, ids, MAXB, tables, lens), "pa_bm_block_tables")) return 1;
  dq = to_device(q1, sizeof(float) * 3 * HQ * D);
  dtables = to_device(tables, sizeof(tables));
  dlens = to_device(lens, sizeof(lens));
  if (!dq || !dtables || !dlens || !hip_ok(hipMalloc(&dout, sizeof(float) * 3 * HQ * D), "hipMalloc"))
    return 1;
  ws_bytes = pa_decode_workspace_size(3, HQ, HKV, D, 100, 32);
  if (ws_bytes > 0 && !hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc")) return 1;
  if (!pa_ok(pa_decode(dout, dq, PA_F32, 3, HQ, D, kpool, vpool, PA_F32, NB, BS, HKV, dtables, MAXB,
                       dlens, 100, 0.125f, 1.0f, 1.0f, 32, PA_DECODE_READ_ONCE, ws, ws_bytes, NULL),
             "pa_decode split-K"))
    return 1;
  if (!hip_ok(hipMemcpy(out1, dout, sizeof(float) * 3 * HQ * D, hipMemcpyDeviceToHost), "hipMemcpy"))
    return 1;
  print_f32("out1", out1, 3 * HQ * D);

  /* 2. fork, one token each with copy-on-write, one decode in one partition. */
  if (!pa_ok(pa_bm_fork(bm, 2, 3), "pa_bm_fork")) return 1;
  if (!pa_ok(pa_bm_append(bm, 2, ids2, slots2, cow, &ncow), "pa_bm_append")) return 1;
  print_i64("slots2", slots2, 2);
  print_i64("cow", cow, 2 * ncow);
  fill(kn, 2 * HKV * D);
  fill(vn, 2 * HKV * D);
  fill(q2, 2 * HQ * D);
  {
    void* dcow = to_device(cow, sizeof(int64_t) * 2 * (ncow > 0 ? ncow : 1));
    void* dkn = to_device(kn, sizeof(kn));
    void* dvn = to_device(vn, sizeof(vn));
    void* ds2 = to_device(slots2, sizeof(slots2));
    if (!dcow || !dkn || !dvn || !ds2) return 1;
    if (!pa_ok(pa_copy_blocks(kpool, vpool, PA_F32, NB, BS, HKV, D, dcow, ncow, NULL), "pa_copy_blocks"))
      return 1;
    if (!pa_ok(pa_cache_write(dkn, dvn, PA_F32, 2, kpool, vpool, PA_F32, NB, BS, HKV, D, ds2, 1.0f,
                              1.0f, NULL), "pa_cache_write 2"))
      return 1;
    if (!pa_ok(pa_bm_block_tables(bm, 2, ids2, MAXB, tables, lens), "pa_bm_block_tables 2")) return 1;
    if (!hip_ok(hipMemcpy(dtables, tables, sizeof(int32_t) * 2 * MAXB, hipMemcpyHostToDevice), "hipMemcpy") ||
        !hip_ok(hipMemcpy(dlens, lens, sizeof(int32_t) * 2, hipMemcpyHostToDevice), "hipMemcpy") ||
        !hip_ok(hipMemcpy(dq, q2, sizeof(q2), hipMemcpyHostToDevice), "hipMemcpy"))
      return 1;
    if (!pa_ok(pa_decode(dout, dq, PA_F32, 2, HQ, D, kpool, vpool, PA_F32, NB, BS, HKV, dtables, MAXB,
                         dlens, 101, 0.125f, 1.0f, 1.0f, 0, PA_DECODE_SHARED, NULL, 0, NULL),
               "pa_decode"))
      return 1;
    if (!hip_ok(hipMemcpy(out2, dout, sizeof(out2), hipMemcpyDeviceToHost), "hipMemcpy")) return 1;
    hipFree(dcow);
    hipFree(dkn);
    hipFree(dvn);
    hipFree(ds2);
  }
  print_f32("out2", out2, 2 * HQ * D);
  if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) return 1;

  hipFree(kpool);
  hipFree(vpool);
  hipFree(dk);
  hipFree(dv);
  hipFree(dslots);
  hipFree(dq);
  hipFree(dout);
  hipFree(dtables);
  hipFree(dlens);
  if (ws) hipFree(ws);
  free(k0);
  free(v0);
  free(q1);
  free(out1);
  pa_bm_destroy(bm);
  return 0;
}
