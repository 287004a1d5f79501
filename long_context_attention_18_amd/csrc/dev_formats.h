// dev_formats.h -- device-side number formats and the pooling exp for gfx950.
//
// Storage formats named by the storage paragraph of "DeepSeek-V4: a
// million-token context that agents can actually use": FP8 KV entries, BF16
// RoPE dims, FP4 lightning indexer. The variants implemented: OCP FP8
// E4M3FN (bias 7, max 448, no infinities), bfloat16, OCP MX FP4 E2M1 with
// E8M0 block scales of 32 elements. Every encoder rounds to nearest, ties
// to even, directly from an fp64 value, and saturates where the format has
// no infinity. These run only in the compressor / window kernels (a few
// values per token), so clarity wins over speed here.
//
// The whole library is built with -ffp-contract=off: every `+ - * /` on
// doubles below is one IEEE-rounded operation, fma() is written where a
// fused operation is meant. That makes the fp64 pooling reproducible bit for
// bit on any IEEE host that runs the same operation sequence.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lca {

// exp for the pooling softmax: Cody & Waite additive range reduction
// (Software Manual for the Elementary Functions, 1980) and the degree-13
// Taylor polynomial of e^r on |r| <= ln2/2 in Horner form (truncation
// error r^14/14! < 4e-18). Constants: 1/ln2; ln2 split into a head with 32
// significant bits (n*head exact for |n| < 2^21) and the rounded remainder;
// Taylor coefficients 1/i!, all rounded to nearest.
__device__ __forceinline__ double pool_exp(double x) {
  if (x < -700.0) return 0.0;
  const double inv_ln2 = 0x1.71547652b82fep+0;
  const double ln2_hi = 0x1.62e42ff000000p-1;
  const double ln2_lo = -0x1.718432a1b0e26p-35;
  double n = rint(x * inv_ln2);
  double r = (x - n * ln2_hi) - n * ln2_lo;
  double p = 0x1.6124613a86d09p-33;       // 1/13!
  p = fma(p, r, 0x1.1eed8eff8d898p-29);   // 1/12!
  p = fma(p, r, 0x1.ae64567f544e4p-26);   // 1/11!
  p = fma(p, r, 0x1.27e4fb7789f5cp-22);   // 1/10!
  p = fma(p, r, 0x1.71de3a556c734p-19);   // 1/9!
  p = fma(p, r, 0x1.a01a01a01a01ap-16);   // 1/8!
  p = fma(p, r, 0x1.a01a01a01a01ap-13);   // 1/7!
  p = fma(p, r, 0x1.6c16c16c16c17p-10);   // 1/6!
  p = fma(p, r, 0x1.1111111111111p-7);    // 1/5!
  p = fma(p, r, 0x1.5555555555555p-5);    // 1/4!
  p = fma(p, r, 0x1.5555555555555p-3);    // 1/3!
  p = fma(p, r, 0.5);                     // 1/2!
  p = fma(p, r, 1.0);                     // 1/1!
  p = fma(p, r, 1.0);                     // 1/0!
  return ldexp(p, (int)n);
}

// Round |a| (finite, >= 0) to the grid of spacing 2^(max(ilogb(a), emin) - mbits):
// the representable magnitudes of a binary format with `mbits` stored
// mantissa bits and minimum normal exponent `emin`. Ties to even.
__device__ __forceinline__ double round_to_format(double a, int emin, int mbits, int* exp_out) {
  int e = (a == 0.0) ? emin : ilogb(a);
  if (e < emin) e = emin;
  double scaled = ldexp(a, mbits - e);   // exact: power-of-two scaling
  double r = rint(scaled);               // round half to even
  *exp_out = e;
  return r;                              // magnitude = r * 2^(e - mbits)
}

// FP8 E4M3FN code of v, saturating at +-448.
__device__ __forceinline__ uint32_t fp8_e4m3_encode(double v) {
  uint32_t sign = signbit(v) ? 0x80u : 0u;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7Eu;
  int e;
  double r = round_to_format(a, -6, 3, &e);   // r in [0, 16]
  uint32_t ri = (uint32_t)r;
  if (ri == 0) return sign;
  if (ri >= 16) { ri >>= 1; e += 1; }          // carried into the next binade
  if (ri < 8) return sign | ri;                 // subnormal (e == -6)
  return sign | ((uint32_t)(e + 7) << 3) | (ri - 8);
}

// bfloat16 bits of v (round to nearest even from fp64, overflow to inf).
__device__ __forceinline__ uint16_t bf16_encode(double v) {
  uint32_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return (uint16_t)sign;
  int e;
  double r = round_to_format(a, -126, 7, &e);  // r in [0, 256]
  uint32_t ri = (uint32_t)r;
  if (ri >= 256) { ri >>= 1; e += 1; }
  if (ri == 0) return (uint16_t)sign;
  if (ri < 128) return (uint16_t)(sign | ri);   // subnormal: exponent field 0
  if (e > 127) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | ((uint32_t)(e + 127) << 7) | (ri - 128));
}

// FP4 E2M1 code (bit 3 = sign) of v, saturating at +-6.
__device__ __forceinline__ uint32_t fp4_e2m1_encode(double v) {
  uint32_t sign = signbit(v) ? 8u : 0u;
  double a = fabs(v);
  if (a >= 6.0) return sign | 7u;
  int e;
  double r = round_to_format(a, 0, 1, &e);     // r in [0, 4]
  uint32_t ri = (uint32_t)r;
  if (ri >= 4) { ri >>= 1; e += 1; }
  if (ri == 0) return sign;
  if (ri < 2) return sign | 1u;                 // 0.5
  if (e > 2) return sign | 7u;                  // rounded up past 6
  return sign | ((uint32_t)(e + 1) << 1) | (ri - 2);
}

// MX block exponent for a block whose largest magnitude is amax (> 0):
// E = clamp(floor(log2 amax) - 2, -127, 127); the stored E8M0 byte is E + 127.
__device__ __forceinline__ int mx_block_exp(double amax) {
  int E = ilogb(amax) - 2;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Exact E4M3FN -> bfloat16 bit pattern (every E4M3FN value is a bf16 value;
// NaN codes are never stored). Branch-free: the 7 magnitude bits placed at
// fp32's exponent/mantissa boundary (E at bit 23, M at bit 20) read as
// 2^(E-127) * (1 + M/8), or M * 2^-129 for E = 0 (an fp32 subnormal); times
// 2^120 that is the E4M3 value, 2^(E-7) * (1 + M/8) or M * 2^-9, exactly.
__device__ __forceinline__ uint16_t e4m3_to_bf16(uint32_t c) {
  const float f = __uint_as_float((c & 0x7Fu) << 20) * 0x1p120f;
  return (uint16_t)(((c & 0x80u) << 8) | (__float_as_uint(f) >> 16));
}

}  // namespace lca
