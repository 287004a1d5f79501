// attention.hip -- CSA sparse / HCA dense attention with the sliding-window
// branch under one softmax, for gfx950.
//
// Figure 3 of "DeepSeek-V4: a million-token context that agents can actually
// use" (CSA: the selected compressed blocks plus a sliding-window branch over
// the recent uncompressed tokens) and Figure 4 / the HCA paragraph (every
// compressed block, densely, plus the same window). Per query t and head h:
//   keys  = {D1 entries: top-k list (CSA) or all j < (t+1)/m (HCA)}
//           + {window entries of positions max(0, t-W+1) .. t}
//   logit = RoPE(q_h, t) . x / sqrt(128),  K = V = the dequantised entry
//   out   = softmax over ALL keys (one normalisation) . x
//
// All query heads share the one KV head, so per query this is a
// [H x 128] x [128 x keys] product followed by [H x keys] x [keys x 128]:
// both run on v_mfma_f32_16x16x32_bf16 with heads as the M dimension. The
// FP8 codes and the BF16 RoPE dims are exact in bf16; the per-entry fp32
// scale is applied to the nope part of the logits (S = S_nope*scale +
// S_rope) and folded into P for the nope output dims (O_nope = (P*scale).C),
// so no dequantised copy is rounded. The rotated query is rounded to bf16.
//
// This kernel serves calls with many queries (chunked prefill); calls with
// fewer than 512 go to attend.hip. Grid: one workgroup per query (4 waves,
// 16 heads each) walks the key list 64 keys at a time: gathers the entries
// into LDS (key-major for Q.K^T, dim-major for P.V), keeps a running max /
// sum per head (online softmax) and writes the normalised output.
#include "dev_formats.h"
#include "kernels.h"

namespace lca {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int KC = kAttnKeys;   // 64 keys per iteration
constexpr int KD_STRIDE = 136;  // bf16 per Kd row (128 + 8 pad)
constexpr int VT_STRIDE = 72;   // bf16 per Vt row (64 + 8 pad)
constexpr int P_STRIDE = 72;

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint16_t* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Kd[KC * KD_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHeadDim * VT_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Pn[4 * 16 * P_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Pr[4 * 16 * P_STRIDE];
  __shared__ float kscale[KC];
  __shared__ int kvalid[KC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, col = lane & 15;
  const int q = blockIdx.x;
  const int b = q / a.Tq, tq = q % a.Tq;
  const int64_t t = query_t(a.seq_len, a.seq_T, a.len, a.Tq, b, tq);
  if (t < 0) return;  // ragged batch: no query in this row
  const int64_t N = min((t + 1) / a.m, a.max_blocks);  // 0 for the window-only layer
  const int64_t n_first = a.dense ? N : (int64_t)a.k;  // key slots before the window
  const int64_t total = n_first + a.W;
  const int64_t s_begin = 0, s_end = total;

  // ---- rotated query, as A operands: row = head (wave*16 + col), K-group kg, 4 K-steps of 32 dims
  const int head = wave * 16 + col;
  const bool head_ok = head < a.H;
  bf16x8 qa[4];
  {
    const uint16_t* qp = a.q + (((size_t)b * a.Tq + tq) * a.H + (head_ok ? head : 0)) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int d0 = ks * 32 + 8 * kg;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (head_ok) raw = *reinterpret_cast<const u32x4*>(qp + d0);
      if (ks >= 2 && head_ok) {
        uint16_t v[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          uint32_t w = raw[u];
          float x0 = bf16_to_f32((uint16_t)(w & 0xFFFFu));
          float x1 = bf16_to_f32((uint16_t)(w >> 16));
          const int pi = (d0 - kNope) / 2 + u;
          // angle t * f reduced to [-pi, pi] in fp64 with 2*pi as a double plus its remainder (error
          // about 1e-10 rad at a million positions), then fp32 sin/cos: the rotated query is rounded to
          // bf16, far coarser than either step
          const double phi = (double)t * a.inv_freq[pi];
          const double n = rint(phi * 0.15915494309189535);
          const double r = (phi - n * 6.28318530717958623) - n * 2.4492935982947064e-16;
          float s, c;
          sincosf((float)r, &s, &c);
          v[2 * u] = f32_to_bf16(x0 * c - x1 * s);
          v[2 * u + 1] = f32_to_bf16(x0 * s + x1 * c);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) raw[u] = (uint32_t)v[2 * u] | ((uint32_t)v[2 * u + 1] << 16);
      }
      qa[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  const float inv_sqrt_d = 0.08838834764831845f;  // 1/sqrt(128)
  float m_run[4], l_run[4];
  v4f O[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  const size_t blk_base = (size_t)b * a.max_blocks;
  const size_t win_base = (size_t)b * a.ring;
  uint16_t* Pn_w = Pn + wave * 16 * P_STRIDE;
  uint16_t* Pr_w = Pr + wave * 16 * P_STRIDE;

  for (int64_t c0 = s_begin; c0 < s_end; c0 += KC) {
    __syncthreads();
    // ---- gather 64 entries: thread -> (key kk, quarter pp) ; 16 codes + 16 rope values each
    {
      const int kk = tid >> 2, pp = tid & 3;
      const int64_t slot = c0 + kk;
      bool valid = slot < s_end;
      const uint8_t* codes = nullptr;
      const uint16_t* rope = nullptr;
      const float* scl = nullptr;
      if (valid) {
        if (slot < n_first) {
          int64_t j = a.dense ? slot : (int64_t)a.topk[((size_t)b * a.Tq + tq) * a.k + slot];
          valid = j >= 0 && j < N;
          if (valid) {
            codes = a.blk_codes + (blk_base + j) * kNope;
            rope = a.blk_rope + (blk_base + j) * kRope;
            scl = a.blk_scale + blk_base + j;
          }
        } else {
          int64_t s = t - a.W + 1 + (slot - n_first);
          valid = s >= 0;
          if (valid) {
            size_t e = win_base + (size_t)(s % a.ring);
            codes = a.win_codes + e * kNope;
            rope = a.win_rope + e * kRope;
            scl = a.win_scale + e;
          }
        }
      }
      u32x4 cw = {0u, 0u, 0u, 0u}, r0 = {0u, 0u, 0u, 0u}, r1 = {0u, 0u, 0u, 0u};
      if (valid) {
        cw = *reinterpret_cast<const u32x4*>(codes + pp * 16);
        r0 = *reinterpret_cast<const u32x4*>(rope + pp * 16);
        r1 = *reinterpret_cast<const u32x4*>(rope + pp * 16 + 8);
      }
      uint16_t cb[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) cb[u] = e4m3_to_bf16((cw[u >> 2] >> (8 * (u & 3))) & 0xFFu);
      u32x4 c_lo, c_hi;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c_lo[u] = (uint32_t)cb[2 * u] | ((uint32_t)cb[2 * u + 1] << 16);
        c_hi[u] = (uint32_t)cb[8 + 2 * u] | ((uint32_t)cb[8 + 2 * u + 1] << 16);
      }
      uint16_t* kd = Kd + kk * KD_STRIDE;
      *reinterpret_cast<u32x4*>(kd + pp * 16) = c_lo;
      *reinterpret_cast<u32x4*>(kd + pp * 16 + 8) = c_hi;
      *reinterpret_cast<u32x4*>(kd + kNope + pp * 16) = r0;
      *reinterpret_cast<u32x4*>(kd + kNope + pp * 16 + 8) = r1;
#pragma unroll
      for (int u = 0; u < 16; ++u) Vt[(pp * 16 + u) * VT_STRIDE + kk] = cb[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        Vt[(kNope + pp * 16 + u) * VT_STRIDE + kk] = (uint16_t)((r0[u >> 1] >> (16 * (u & 1))) & 0xFFFFu);
        Vt[(kNope + pp * 16 + 8 + u) * VT_STRIDE + kk] = (uint16_t)((r1[u >> 1] >> (16 * (u & 1))) & 0xFFFFu);
      }
      if (pp == 0) {
        kscale[kk] = valid ? *scl : 0.0f;
        kvalid[kk] = valid ? 1 : 0;
      }
    }
    __syncthreads();

    // ---- S = Q.K^T for this wave's 16 heads x 64 keys
    float S[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      v4f an = {0.0f, 0.0f, 0.0f, 0.0f}, ar = {0.0f, 0.0f, 0.0f, 0.0f};
      const uint16_t* krow = Kd + (kt * 16 + col) * KD_STRIDE + 8 * kg;
      an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0], lds_bf16x8(krow), an, 0, 0, 0);
      an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1], lds_bf16x8(krow + 32), an, 0, 0, 0);
      ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[2], lds_bf16x8(krow + 64), ar, 0, 0, 0);
      ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[3], lds_bf16x8(krow + 96), ar, 0, 0, 0);
      const int key = kt * 16 + col;
      const float sc = kscale[key];
      const bool ok = kvalid[key] != 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) S[kt][i] = ok ? (an[i] * sc + ar[i]) * inv_sqrt_d : -INFINITY;
    }
    // ---- online softmax per head row (rows 4kg+i live in the 16 lanes of group kg)
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = fmaxf(fmaxf(S[0][i], S[1][i]), fmaxf(S[2][i], S[3][i]));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float m_new = fmaxf(m_run[i], mx);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      alpha[i] = __expf(m_run[i] - m_use);
      float rs = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        float pv = __expf(S[kt][i] - m_use);
        S[kt][i] = pv;
        rs += pv;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) rs += __shfl_xor(rs, o, 64);
      l_run[i] = l_run[i] * alpha[i] + rs;
      m_run[i] = m_new;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[nt][i] *= alpha[i];
    // P (rope dims) and P*scale (nope dims) as bf16 A operands, via LDS
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = kt * 16 + col;
      const float sc = kscale[key];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Pr_w[(4 * kg + i) * P_STRIDE + key] = f32_to_bf16(S[kt][i]);
        Pn_w[(4 * kg + i) * P_STRIDE + key] = f32_to_bf16(S[kt][i] * sc);
      }
    }
    __syncthreads();
    // ---- O += P.V : A rows = heads, K = keys; B columns = dims
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint16_t* prow = (nt < 4 ? Pn_w : Pr_w) + col * P_STRIDE + 8 * kg;
      const uint16_t* vrow = Vt + (nt * 16 + col) * VT_STRIDE + 8 * kg;
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_bf16x8(prow), lds_bf16x8(vrow), O[nt], 0, 0, 0);
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_bf16x8(prow + 32), lds_bf16x8(vrow + 32), O[nt], 0, 0, 0);
    }
  }

  // ---- output: lane holds O[nt][i] = (head wave*16 + 4kg + i, dim nt*16 + col)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = wave * 16 + 4 * kg + i;
    if (h >= a.H) continue;
    const float inv = 1.0f / l_run[i];
    uint16_t* o = a.out + (((size_t)b * a.Tq + tq) * a.H + h) * kHeadDim;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt * 16 + col] = f32_to_bf16(O[nt][i] * inv);
    if (a.lse && col == 0) a.lse[((size_t)b * a.Tq + tq) * a.H + h] = m_run[i] + __logf(l_run[i]);
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int32_t B, hipStream_t s) {
  const unsigned nq = (unsigned)(B * a.Tq);
  hipLaunchKernelGGL(attn_kernel, dim3(nq), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lca
