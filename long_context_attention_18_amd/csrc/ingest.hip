// ingest.hip -- KV compressor and sliding-window / tail append for gfx950.
//
// Compressor: the CSA paragraph and Figure 3 of "DeepSeek-V4: a
// million-token context that agents can actually use" (softmax-gated
// pooling with a learned positional bias, every 4 tokens into one entry),
// the HCA paragraph and Figure 4 (the same at 128x). Window / tail: Figure
// 3's sliding-window branch and the KV-cache section of velog.io
// "DeepSeek V4 논문 정리" (separate window state, separately managed
// uncompressed tail).
//
// One 64-lane wave per compressed block (or per window token). Lane c owns
// channel c of the 64 "nope" dims, channel 64+c of the RoPE dims and, for
// CSA, channel c of the indexer stream. The pooling is fp64 with the
// library's own exp so that the FP8 / FP4 codes are reproducible bit for bit;
// this is a few thousand flops per block, far off any roofline (decode
// writes at most one block per m tokens).
#include "dev_formats.h"
#include "ingest.h"
#include "kernels.h"

namespace lca {

namespace {

// Blocks of at most kPoolCache tokens (CSA: 4): one wave per position (wave i loads position i's inputs,
// its RoPE rotation and, once the maxima are known, its exps), the position terms meet in LDS, and wave 0
// sums them in ascending position order -- the same operations in the same order as the three passes
// below, so the same bits, with the loads, the fp64 sincos and the exps of the positions side by side
// instead of in one wave's dependency chain.
constexpr int kPoolCache = 4;

struct PoolLds {
  double x[3][kPoolCache][64];  // gate + bias (nope, RoPE, indexer), then the position's exp
  double v[3][kPoolCache][64];  // value: kv nope dim, RoPE'd kv dim, indexer key dim
};

// Wave w (< m) of the workgroup; every wave of the workgroup calls it (barriers). Wave 0 gets the pooled
// values of its channel c.
template <bool CSA>
__device__ __forceinline__ void pool_waves(const IngestArgs& a, PoolLds& P, int b, int64_t len, int64_t j, int w,
                                           int c, double& y_n, double& y_r, double& y_i) {
  const int m = a.m;
  if (w < m) {
    const int64_t p = j * m + w;
    const uint16_t* g = token_row(a, b, len, p, a.gate, kHeadDim, kTailGate, w);
    const uint16_t* kv = token_row(a, b, len, p, a.kv, kHeadDim, kTailKv, w);
    P.x[0][w][c] = (double)bf16_to_f32(g[c]) + (double)a.bias[w * kHeadDim + c];
    P.x[1][w][c] = (double)bf16_to_f32(g[kNope + c]) + (double)a.bias[w * kHeadDim + kNope + c];
    P.v[0][w][c] = (double)bf16_to_f32(kv[c]);
    P.v[1][w][c] = rope_channel(kv, c, p, a.inv_freq);
    if (CSA) {
      const uint16_t* gi = token_row(a, b, len, p, a.ig, kIdxDim, kTailIg, w);
      const uint16_t* ki = token_row(a, b, len, p, a.ik, kIdxDim, kTailIk, w);
      P.x[2][w][c] = (double)bf16_to_f32(gi[c]) + (double)a.idx_bias[w * kIdxDim + c];
      P.v[2][w][c] = (double)bf16_to_f32(ki[c]);
    }
  }
  __syncthreads();
  double e0 = 0.0, e1 = 0.0, e2 = 0.0;
  if (w < m) {
    // the per-channel maxima (order-free), then this position's exps
    double mu[3] = {-INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int i = 0; i < kPoolCache; ++i)
      if (i < m)
#pragma unroll
        for (int s = 0; s < 3; ++s)
          if (s < 2 || CSA) mu[s] = fmax(mu[s], P.x[s][i][c]);
    e0 = pool_exp(P.x[0][w][c] - mu[0]);
    e1 = pool_exp(P.x[1][w][c] - mu[1]);
    if (CSA) e2 = pool_exp(P.x[2][w][c] - mu[2]);
  }
  __syncthreads();  // every wave has read the gate values the exps overwrite
  if (w < m) {
    P.x[0][w][c] = e0;
    P.x[1][w][c] = e1;
    if (CSA) P.x[2][w][c] = e2;
  }
  __syncthreads();
  y_n = 0.0;
  y_r = 0.0;
  y_i = 0.0;
  if (w != 0) return;
  double S_n = 0.0, S_r = 0.0, S_i = 0.0;
#pragma unroll
  for (int i = 0; i < kPoolCache; ++i) {
    if (i < m) {
      S_n = S_n + P.x[0][i][c];
      S_r = S_r + P.x[1][i][c];
      if (CSA) S_i = S_i + P.x[2][i][c];
    }
  }
#pragma unroll
  for (int i = 0; i < kPoolCache; ++i) {
    if (i < m) {
      y_n = fma(P.x[0][i][c] / S_n, P.v[0][i][c], y_n);
      y_r = fma(P.x[1][i][c] / S_r, P.v[1][i][c], y_r);
      if (CSA) y_i = fma(P.x[2][i][c] / S_i, P.v[2][i][c], y_i);
    }
  }
}

// m <= kPoolCache: m waves per block (pool_waves); otherwise one wave over the block's m positions
// The block's entry from its pooled values (wave 0 of the workgroup: lane c holds nope dim c, RoPE dim
// 64+c and, for CSA, indexer dim c)
template <bool CSA>
__device__ __forceinline__ void finish_block(const IngestArgs& a, int b, int64_t j, int c, double y_n, double y_r,
                                             double y_i) {
  const size_t e = (size_t)b * a.max_blocks + (size_t)j;
  write_entry(y_n, y_r, c, a.blk_codes + e * kNope, a.blk_scale + e, a.blk_rope + e * kRope);
  if (CSA) {
    // MX-FP4 indexer key: lanes 0..31 form scale block 0, lanes 32..63 block 1
    double amax = half_wave_max(fabs(y_i));
    int E = (amax == 0.0) ? -127 : mx_block_exp(amax);
    uint32_t code = (amax == 0.0) ? 0u : fp4_e2m1_encode(ldexp(y_i, -E));
    // the next lane's code (row_shl:1; the pairs (2i, 2i+1) never cross a 16-lane row)
    uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)code, 0x101, 0xf, 0xf, false);
    if ((c & 1) == 0) a.idx_codes[e * 32 + (c >> 1)] = (uint8_t)(code | (hi << 4));
    if ((c & 31) == 0) a.idx_scale[e * 2 + (c >> 5)] = (uint8_t)((amax == 0.0) ? 0 : E + 127);
  }
}

// Blocks of at most kPoolCache tokens: a wave per position (pool_waves)
template <bool CSA>
__global__ __launch_bounds__(64 * kPoolCache) void compress_kernel(IngestArgs a) {
  __shared__ PoolLds P;
  const int c = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int m = a.m;
  const int64_t len = a.seq_len ? a.seq_len[b] : a.len;
  const int64_t j = (a.seq_len ? len / m : a.first) + blockIdx.x;
  // ragged batch: the blocks this sequence's own tokens complete (the grid covers the most of any)
  if (a.seq_len && j >= (len + ragged_T(a.seq_len, a.seq_T, a.seq_cap, b)) / m) return;
  double y_n, y_r, y_i;
  pool_waves<CSA>(a, P, b, len, j, w, c, y_n, y_r, y_i);
  if (w == 0) finish_block<CSA>(a, b, j, c, y_n, y_r, y_i);
}

// Longer blocks (HCA: 128 tokens): kLongWaves waves, wave w over positions w, w + kLongWaves, ..., one
// stream (nope, RoPE, indexer) after the other. Per stream: the positions' gate + bias and their maximum
// (the maximum is free of order); each position's exp into LDS; wave 0 sums the exps in ascending
// position order; each position's weight (exp / sum) and value into LDS; wave 0 takes the weighted sum
// with one fma per position in ascending order. The same operations in the same order as one wave
// walking the positions, so the same bits; the loads, exps, divisions and sincos of the positions run
// side by side instead of one position after the other.
constexpr int kLongWaves = 8;
constexpr int kLongMaxM = 128;
constexpr int kLongPer = kLongMaxM / kLongWaves;  // positions per wave

struct LongPoolLds {
  double t[kLongMaxM][64];  // a stream's exps, then its weights
  double v[kLongMaxM][64];  // a stream's values
  double part[kLongWaves][64];
  double sum[64];
};

template <bool CSA>
__global__ __launch_bounds__(64 * kLongWaves) void compress_long_kernel(IngestArgs a) {
  __shared__ LongPoolLds P;
  const int c = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int m = a.m;
  const int64_t len = a.seq_len ? a.seq_len[b] : a.len;
  const int64_t j = (a.seq_len ? len / m : a.first) + blockIdx.x;
  if (a.seq_len && j >= (len + ragged_T(a.seq_len, a.seq_T, a.seq_cap, b)) / m) return;  // ragged batch, as above
  const int64_t p0 = j * m;
  double y[3] = {0.0, 0.0, 0.0};
#pragma unroll 1
  for (int st = 0; st < (CSA ? 3 : 2); ++st) {
    // gate + bias of this wave's positions, and their maximum
    double x[kLongPer];
    double mu = -INFINITY;
#pragma unroll
    for (int u = 0; u < kLongPer; ++u) {
      const int i = w + u * kLongWaves;
      x[u] = 0.0;
      if (i < m) {
        const int64_t p = p0 + i;
        if (st < 2) {
          const uint16_t* g = token_row(a, b, len, p, a.gate, kHeadDim, kTailGate, i);
          const int col = st == 0 ? c : kNope + c;
          x[u] = (double)bf16_to_f32(g[col]) + (double)a.bias[i * kHeadDim + col];
        } else {
          const uint16_t* gi = token_row(a, b, len, p, a.ig, kIdxDim, kTailIg, i);
          x[u] = (double)bf16_to_f32(gi[c]) + (double)a.idx_bias[i * kIdxDim + c];
        }
        mu = fmax(mu, x[u]);
      }
    }
    P.part[w][c] = mu;
    __syncthreads();
#pragma unroll
    for (int ww = 0; ww < kLongWaves; ++ww) mu = fmax(mu, P.part[ww][c]);
#pragma unroll
    for (int u = 0; u < kLongPer; ++u) {
      const int i = w + u * kLongWaves;
      if (i < m) P.t[i][c] = pool_exp(x[u] - mu);
    }
    __syncthreads();
    if (w == 0) {
      double S = 0.0;
#pragma unroll 16
      for (int i = 0; i < m; ++i) S = S + P.t[i][c];  // (unrolled: the LDS reads go out ahead of the adds)
      P.sum[c] = S;
    }
    __syncthreads();
    const double S = P.sum[c];
#pragma unroll 4
    for (int u = 0; u < kLongPer; ++u) {
      const int i = w + u * kLongWaves;
      if (i < m) {
        const int64_t p = p0 + i;
        P.t[i][c] = P.t[i][c] / S;
        if (st < 2) {
          const uint16_t* kv = token_row(a, b, len, p, a.kv, kHeadDim, kTailKv, i);
          P.v[i][c] = st == 0 ? (double)bf16_to_f32(kv[c]) : rope_channel(kv, c, p, a.inv_freq);
        } else {
          const uint16_t* ki = token_row(a, b, len, p, a.ik, kIdxDim, kTailIk, i);
          P.v[i][c] = (double)bf16_to_f32(ki[c]);
        }
      }
    }
    __syncthreads();
    if (w == 0) {
      double acc = 0.0;
#pragma unroll 16
      for (int i = 0; i < m; ++i) acc = fma(P.t[i][c], P.v[i][c], acc);
      y[st] = acc;
    }
    __syncthreads();  // wave 0 has read the arrays the next stream overwrites
  }
  if (w == 0) finish_block<CSA>(a, b, j, c, y[0], y[1], y[2]);
}

template <bool CSA>
__global__ __launch_bounds__(64) void append_kernel(IngestArgs a) {
  append_unit<CSA>(a, blockIdx.y, blockIdx.x, threadIdx.x);
}

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_compress(const IngestArgs& a, bool csa, int64_t n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  dim3 grid((unsigned)n_blocks, (unsigned)a.B);
  if (a.m > kLongMaxM) return hipErrorInvalidValue;
  if (a.m <= kPoolCache) {
    const dim3 threads(64u * (unsigned)a.m);  // a wave per position
    if (csa) hipLaunchKernelGGL(compress_kernel<true>, grid, threads, 0, s, a);
    else hipLaunchKernelGGL(compress_kernel<false>, grid, threads, 0, s, a);
  } else {
    if (csa) hipLaunchKernelGGL(compress_long_kernel<true>, grid, dim3(64 * kLongWaves), 0, s, a);
    else hipLaunchKernelGGL(compress_long_kernel<false>, grid, dim3(64 * kLongWaves), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_append(const IngestArgs& a, bool csa, int32_t n_tail, hipStream_t s) {
  int64_t n = (int64_t)a.n_win + n_tail;
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)n, (unsigned)a.B);
  if (csa) hipLaunchKernelGGL(append_kernel<true>, grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL(append_kernel<false>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

// Zero `bytes` (a multiple of 16, 16-byte aligned) with a kernel rather than
// a runtime memset, so the work can sit inside a captured graph.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace lca
