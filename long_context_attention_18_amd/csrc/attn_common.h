// attn_common.h -- register-level helpers shared by the attention kernels (attend.hip, attention.hip).
#pragma once
#include "kernels.h"

namespace lca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// log2(e) / sqrt(128): logits stay unscaled (S = q.x); this one factor turns them into exp2 units
constexpr float kLog2eRsqrtD = 0.12751743074640293f;

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// value held by lane l ^ 16 / l ^ 32 (VALU lane swaps)
__device__ __forceinline__ float xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(((threadIdx.x >> 5) & 1) ? r[0] : r[1]);
}

// Float max without the NaN-quieting max the compiler puts before a max of values it cannot prove
// canonical (MFMA and lane-swap results): the logits here are never NaN.
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max / sum of x over lanes l and l ^ 16 (l ^ 32): a lane swap leaves the pair in its two outputs, so a
// symmetric operation needs no lane select
__device__ __forceinline__ float pair_max16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 8 E4M3FN codes (little-endian bytes) -> 8 bf16: v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts
// two codes exactly (every E4M3FN value is a bf16 value; checked for all 256 codes on MI355X)
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 c) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true));
  return o;
}

// two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed low first
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Load through a global-address-space pointer (a global_load, counted by vmcnt only).
template <typename T>
__device__ __forceinline__ T ldg(const void* p) {
  typedef const __attribute__((address_space(1))) T global_t;
  return *(global_t*)p;
}

// RoPE angle of position t and frequency f, reduced to [-pi, pi] in fp64 (2 pi as a double plus its
// remainder), then fp32 sin / cos: the rotated query is rounded to bf16, far coarser than either step
__device__ __forceinline__ void rope_angle(int64_t t, double f, float* sn, float* cs) {
  const double phi = (double)t * f;
  const double n = rint(phi * 0.15915494309189535);
  const double rr = (phi - n * 6.28318530717958623) - n * 2.4492935982947064e-16;
  sincosf((float)rr, sn, cs);
}

}  // namespace
}  // namespace lca
