// pa_device.h — device-side building blocks shared by the gfx950 kernels:
// element traits of the K/V storage types, 16-byte vector access,
// wavefront reductions through DPP, and the fp8 / bf16 conversions.
//
// Written for CDNA4 (gfx950, wave64).  The DPP row is 16 lanes; one token
// row of a K/V tile (head_size elements) spans 4, 8 or 16 lanes (16 bytes
// per lane, 8 for fp8), so its dot products reduce inside a DPP row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Storage element tags.
struct F32 {};
struct BF16 {};
struct FP8 {};

template <typename T> struct Elem;
template <> struct Elem<F32>  { static constexpr int bytes = 4; using word = uint32_t; };
template <> struct Elem<BF16> { static constexpr int bytes = 2; using word = uint16_t; };
template <> struct Elem<FP8>  { static constexpr int bytes = 1; using word = uint8_t; };

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// --- conversions ------------------------------------------------------------
// Two bf16 packed in a dword -> two floats (bf16 is the top half of binary32).
__device__ __forceinline__ float bf16lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }

// Four OCP E4M3FN codes packed in a dword -> four floats (gfx950 converts
// the OCP encoding natively).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
}

// 16 bytes of storage -> EPL floats.
template <typename T> struct Vec;
template <> struct Vec<F32> {
  static constexpr int n = 4;
  __device__ __forceinline__ static void to_f32(const u32x4& v, float* o) {
    o[0] = u2f(v.x); o[1] = u2f(v.y); o[2] = u2f(v.z); o[3] = u2f(v.w);
  }
};
template <> struct Vec<BF16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void to_f32(const u32x4& v, float* o) {
    o[0] = bf16lo(v.x); o[1] = bf16hi(v.x); o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
    o[4] = bf16lo(v.z); o[5] = bf16hi(v.z); o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
  }
};
template <> struct Vec<FP8> {
  static constexpr int n = 16;
  __device__ __forceinline__ static void to_f32(const u32x4& v, float* o) {
    fp8x4_to_f32(v.x, o); fp8x4_to_f32(v.y, o + 4);
    fp8x4_to_f32(v.z, o + 8); fp8x4_to_f32(v.w, o + 12);
  }
};

// Four bf16 values (two packed words, low half first) widened to fp32.
__device__ __forceinline__ f32x4 bf16x4_to_f32x4(u32x2 w) {
  return f32x4{bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y)};
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = f2u(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float -> OCP E4M3FN code: saturate to +-448, round to nearest even,
// NaN -> 0x7F with the sign bit.  Built from the binary32 fields:
// magnitudes below 2^-6 are subnormal multiples of 2^-9, the rest keep
// their exponent and round the 23-bit fraction to 3 bits.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float x) {
  const uint32_t u = f2u(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7Fu | sign;
  float a = fminf(__builtin_fabsf(x), 448.0f);
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid 2^-9
    return (uint32_t)__builtin_rintf(a * 512.0f) | sign;   // exact product, RNE
  }
  const uint32_t ua = f2u(a);
  const int e = (int)(ua >> 23) - 127;       // -6 .. 8
  const uint32_t frac = ua & 0x7FFFFFu;
  const uint32_t keep = frac >> 20, rest = frac & 0xFFFFFu;
  const uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
  return ((uint32_t)((e + 7) << 3) + keep + up) | sign;
}

// --- cross-lane sums / maxima inside DPP rows --------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over groups of N consecutive lanes (N = 4, 8 or 16); every lane of a
// group receives the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "group must fit a DPP row");
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kRowMirror>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int m) {
  return __shfl_xor(x, m, kWave);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A load of K/V words: non-temporal (evict first) when NT, for a stream that
// reads every line once; an ordinary load when lines may be read again (a
// block shared by several sequences).
template <bool NT, typename V>
__device__ __forceinline__ V kv_load(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

}  // namespace pa
