// ingest.h -- per-token window entries and tail copies (the append step), shared by the append
// kernel and the candidate scan, which does a decode step's append in the same launch.
//
// Figure 3's sliding-window branch of "DeepSeek-V4: a million-token context that agents can
// actually use" and the KV-cache section of velog.io "DeepSeek V4 논문 정리" (separate window
// state, separately managed uncompressed tail).
#pragma once
#include "dev_formats.h"
#include "kernels.h"

namespace lca {

constexpr int kTailKv = 0, kTailGate = 128, kTailIk = 256, kTailIg = 320;

// BF16 input row of token p (absolute position) of sequence b, which held len tokens before this call:
// from the tail if an earlier call appended it, else from this call's input (row stride a.T).
// `slot` is p mod m when the caller knows it (a block's own positions: the index in the block), else -1.
__device__ __forceinline__ const uint16_t* token_row(const IngestArgs& a, int b, int64_t len, int64_t p,
                                                     const uint16_t* in, int width, int tail_off, int slot = -1) {
  if (p < len) {
    const size_t sl = slot >= 0 ? (size_t)slot : (size_t)(p % a.m);  // (a 64-bit division otherwise)
    return a.tail + ((size_t)b * a.m + sl) * a.tail_width + tail_off;
  }
  return in + ((size_t)b * a.T + (size_t)(p - len)) * width;
}

// Max of v over lane groups, with VALU lane moves instead of LDS-crossbar shuffles: DPP quad permutes
// (lane ^ 1, lane ^ 2) and row rotations (by 4, 8) give every lane its 16-lane row's max, and a
// v_permlane16_swap (rows 0 <-> 1, 2 <-> 3) or v_permlane32_swap (lane halves) pairs the rows. A
// double moves as its two 32-bit words; max is exact, so the grouping does not change the result.
template <int CTRL>
__device__ __forceinline__ double dpp_move(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double row_max(double v) {
  v = fmax(v, dpp_move<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  v = fmax(v, dpp_move<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  v = fmax(v, dpp_move<0x124>(v));  // row_ror:4
  return fmax(v, dpp_move<0x128>(v));  // row_ror:8
}
__device__ __forceinline__ double swap_max16(double v) {
  auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)__double2loint(v), (uint32_t)__double2loint(v), false, false);
  auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)__double2hiint(v), (uint32_t)__double2hiint(v), false, false);
  return fmax(__hiloint2double((int)hi[0], (int)lo[0]), __hiloint2double((int)hi[1], (int)lo[1]));
}
__device__ __forceinline__ double swap_max32(double v) {
  auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)__double2loint(v), (uint32_t)__double2loint(v), false, false);
  auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)__double2hiint(v), (uint32_t)__double2hiint(v), false, false);
  return fmax(__hiloint2double((int)hi[0], (int)lo[0]), __hiloint2double((int)hi[1], (int)lo[1]));
}

// max over the 64 lanes (every lane gets it)
__device__ __forceinline__ double wave_max(double v) { return swap_max32(swap_max16(row_max(v))); }

// max over lanes 0-31 and, separately, 32-63
__device__ __forceinline__ double half_wave_max(double v) { return swap_max16(row_max(v)); }

// RoPE-rotated value of channel 64+c of token p (pair (2i, 2i+1), i = c/2):
//   even: x0 cos - x1 sin;  odd: x0 sin + x1 cos;  angle p * inv_freq[i]; fp64.
// sin and cos of a RoPE angle x (0 <= x < 2^30: a position times an inverse frequency <= 1). Cody and
// Waite's reduction: k = the integer nearest x / (pi/2), r = x - k pi/2 with pi/2 split into three doubles
// (one fma each, so every product is exact before its one rounding; |r| <= pi/4 to within 2^-53). Then
// the Taylor series of sin through r^17 and of cos through r^18 (the first omitted terms stay below
// 1e-19 on |r| <= pi/4) in Horner form, and the quadrant k mod 4. About 1.5 ulp; no branch, no table.
__device__ __forceinline__ void rope_sincos(double x, double* sn, double* cs) {
  const double k = rint(x * 0x1.45f306dc9c883p-1);  // 2/pi
  double r = fma(-k, 0x1.921fb54442d18p+0, x);      // pi/2, first part
  r = fma(-k, 0x1.1a62633145c07p-54, r);            // second part
  r = fma(-k, -0x1.f1976b7ed8fbcp-110, r);          // third part
  const double z = r * r;
  double ps = 0x1.952c77030ad4ap-49;                // 1/17!
  ps = fma(ps, z, -0x1.ae7f3e733b81fp-41);          // -1/15!
  ps = fma(ps, z, 0x1.6124613a86d09p-33);           // 1/13!
  ps = fma(ps, z, -0x1.ae64567f544e4p-26);          // -1/11!
  ps = fma(ps, z, 0x1.71de3a556c734p-19);           // 1/9!
  ps = fma(ps, z, -0x1.a01a01a01a01ap-13);          // -1/7!
  ps = fma(ps, z, 0x1.1111111111111p-7);            // 1/5!
  ps = fma(ps, z, -0x1.5555555555555p-3);           // -1/3!
  const double s = fma(r * z, ps, r);
  double pc = -0x1.6827863b97d97p-53;               // -1/18!
  pc = fma(pc, z, 0x1.ae7f3e733b81fp-45);           // 1/16!
  pc = fma(pc, z, -0x1.93974a8c07c9dp-37);          // -1/14!
  pc = fma(pc, z, 0x1.1eed8eff8d898p-29);           // 1/12!
  pc = fma(pc, z, -0x1.27e4fb7789f5cp-22);          // -1/10!
  pc = fma(pc, z, 0x1.a01a01a01a01ap-16);           // 1/8!
  pc = fma(pc, z, -0x1.6c16c16c16c17p-10);          // -1/6!
  pc = fma(pc, z, 0x1.5555555555555p-5);            // 1/4!
  pc = fma(pc, z, -0.5);                            // -1/2!
  const double c = fma(z, pc, 1.0);
  const int q = (int)((long long)k & 3);
  *sn = q == 0 ? s : (q == 1 ? c : (q == 2 ? -s : -c));
  *cs = q == 0 ? c : (q == 1 ? -s : (q == 2 ? -c : s));
}

__device__ __forceinline__ double rope_channel(const uint16_t* kv_row, int c, int64_t p, const double* inv_freq) {
  int i = c >> 1;
  double x0 = (double)bf16_to_f32(kv_row[kNope + 2 * i]);
  double x1 = (double)bf16_to_f32(kv_row[kNope + 2 * i + 1]);
  double phi = (double)p * inv_freq[i];
  double sn, cs;
  rope_sincos(phi, &sn, &cs);
  return (c & 1) ? (x0 * sn + x1 * cs) : (x0 * cs - x1 * sn);
}

// Write one 196-byte entry from the lane's nope value xn (dim c) and RoPE
// value xr (dim 64+c): scale = fp32(amax / 448), code = E4M3FN(x / scale).
__device__ __forceinline__ void write_entry(double xn, double xr, int c, uint8_t* codes, float* scale,
                                            uint16_t* rope) {
  double amax = wave_max(fabs(xn));
  float s = (float)(amax / 448.0);
  bool zero = (amax == 0.0) || (s == 0.0f);
  uint32_t code = zero ? 0u : fp8_e4m3_encode(xn / (double)s);
  codes[c] = (uint8_t)code;
  rope[c] = bf16_encode(xr);
  if (c == 0) *scale = zero ? 0.0f : s;
}

// One unit of the append of sequence b, on the 64 lanes of a wave (lane c): unit < n_win writes the
// window entry of token a.first + unit (its kv, RoPE'd at its position, its own FP8 scale) into ring
// slot s mod R; the following units copy the BF16 inputs of the tokens of the block that is still
// incomplete after this call into the tail.
template <bool CSA>
__device__ __forceinline__ void append_unit(const IngestArgs& a, int b, int unit, int c) {
  int64_t len = a.len, first = a.first, end = a.len + a.T;
  int32_t n_win = a.n_win;
  if (a.seq_len) {  // ragged batch: this sequence's own window tokens and tail rows; units beyond them idle
    len = a.seq_len[b];
    end = len + ragged_T(a.seq_len, a.seq_T, a.seq_cap, b);
    first = end - a.ring > len ? end - a.ring : len;
    n_win = (int32_t)(end - first);
    int64_t tail_first = (end / a.m) * a.m;
    if (tail_first < len) tail_first = len;
    if (unit >= n_win + (int32_t)(end - tail_first)) return;
  }
  if (unit < n_win) {
    // window entry of token s: its own kv, RoPE'd at s, its own FP8 scale
    const int64_t s = first + unit;
    const uint16_t* kv = a.kv + ((size_t)b * a.T + (size_t)(s - len)) * kHeadDim;
    double xn = (double)bf16_to_f32(kv[c]);
    double xr = rope_channel(kv, c, s, a.inv_freq);
    const size_t e = (size_t)b * a.ring + (size_t)(s % a.ring);
    write_entry(xn, xr, c, a.win_codes + e * kNope, a.win_scale + e, a.win_rope + e * kRope);
    return;
  }
  // tail: tokens of the block that is still incomplete after this call
  int64_t tail_first = (end / a.m) * a.m;
  if (tail_first < len) tail_first = len;
  const int64_t p = tail_first + (unit - n_win);
  const size_t r = (size_t)b * a.T + (size_t)(p - len);
  uint16_t* dst = a.tail + ((size_t)b * a.m + (size_t)(p % a.m)) * a.tail_width;
  dst[kTailKv + c] = a.kv[r * kHeadDim + c];
  dst[kTailKv + 64 + c] = a.kv[r * kHeadDim + 64 + c];
  dst[kTailGate + c] = a.gate[r * kHeadDim + c];
  dst[kTailGate + 64 + c] = a.gate[r * kHeadDim + 64 + c];
  if (CSA) {
    dst[kTailIk + c] = a.ik[r * kIdxDim + c];
    dst[kTailIg + c] = a.ig[r * kIdxDim + c];
  }
}

}  // namespace lca
