// indexer.hip -- CSA lightning indexer and exact per-query top-k for gfx950.
//
// The CSA paragraph of "DeepSeek-V4: a million-token context that agents can
// actually use": an FP4 lightning indexer, a ReLU-scored multi-head dot
// product, picks the top-k compressed blocks for each query.
//
// score (per query, per visible block j):
//   s_h     = fp32(<MXFP4(qI_h), key_j>)          h < H_I (<= 8)
//   score_j = fmaf chain over h of w_h * max(s_h, 0), from +0; -0 -> +0
// top-k: the min(k, N) largest (score, -j), output in ascending j.
//
// Kernel 1 (score): the per-head dot products are a [H_I x 64] x [64 x N]
// product in MXFP4, run on the gfx950 scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 operands and E8M0 scales. The
// indexer has a single 64-dim key head, so K=128 would be half empty; we
// pack two blocks into one K=128 column instead: A row (h, p) holds q_h in
// K-groups 2p, 2p+1 and zeros elsewhere, B column n holds blocks 2n and 2n+1
// back to back. C[(h,p)][n] is then q_h . key_{2n+p}: 16 rows x 16 columns =
// 8 heads x 32 blocks per instruction, nothing wasted. Each product of E2M1
// values is exact and every 32-element group sum is exact; the instruction
// adds two scaled exact terms, and one correctly rounded fp32 addition of two
// exact terms is the fp32 rounding of the exact dot product. The keys stream
// straight from HBM into the B operand (34 B per block, 16-B loads, fully
// coalesced), so the kernel is a pure HBM stream. The head combine is done in
// the MFMA output layout: lanes of row-group 0/2 hold heads 0..3, row-group
// 1/3 heads 4..7, and one cross-lane move continues the fmaf chain.
// Each workgroup also histograms the top 12 bits of the ordered score key in
// LDS and emits a lower bound T_c below which fewer than k' of its scores lie
// ("at least k' scores of this chunk are >= T_c").
//
// Kernel 2 (scan): L = the r-th largest T_c, r = ceil(G/2) chunks, k' =
// ceil(k/r): at least r*k' >= k scores are >= L, so every winner is >= L.
// Scores >= L are appended to a per-query candidate list (a few times k).
//
// Kernel 3 (select): radix select over the 64-bit keys (score_key << 32 |
// ~j) of the candidates in LDS (or over all N scores if the list overflowed),
// then a bitonic sort of the winners' indices. Exact for any input.
#include "dev_formats.h"
#include "kernels.h"

namespace lca {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float relu(float x) { return x > 0.0f ? x : 0.0f; }

__device__ __forceinline__ int64_t visible_blocks(const ScoreArgs& a, int tq) {
  int64_t t = a.len - a.Tq + tq;
  return (t + 1) / a.m;
}

// exclusive prefix sum of `v` over the 256 threads of a workgroup; *total gets the sum
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wave) off += wsum[w];
    tot += wsum[w];
  }
  *total = tot;
  return off + incl - v;
}

__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t thr_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = blockIdx.y;
  const int b = q / a.Tq, tq = q % a.Tq;
  const int64_t N = visible_blocks(a, tq);
  const int64_t j_begin = (int64_t)blockIdx.x * kScoreChunk;
  // this call's candidate counter starts at zero (the scan kernel runs after this one)
  if (blockIdx.x == 0 && tid == 0) a.cand_cnt[q] = 0;
  if (j_begin >= N) return;
  for (int i = tid; i < kHistBins; i += 256) hist[i] = 0;
  if (tid == 0) thr_s = 0;

  // ---- A operand: MXFP4 query. Lane: row r = lane%16 = (p, h) = (r/8, r%8), K-group g = lane/16.
  const int r = lane & 15, g = lane >> 4, p = r >> 3, h = r & 7, half = g & 1;
  uint32_t av[4] = {0u, 0u, 0u, 0u};
  int sa = 127;
  if ((g >> 1) == p && h < a.HI) {
    const uint16_t* src = a.qI + (((size_t)b * a.Tq + tq) * a.HI + h) * kIdxDim + half * 32;
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)bf16_to_f32(src[i])));
    if (amax == 0.0) {
      sa = 0;
    } else {
      int E = mx_block_exp(amax);
      sa = E + 127;
      for (int i = 0; i < 32; ++i) {
        uint32_t code = fp4_e2m1_encode(ldexp((double)bf16_to_f32(src[i]), -E));
        av[i >> 3] |= code << (4 * (i & 7));
      }
    }
  }
  const v8i A = {(int)av[0], (int)av[1], (int)av[2], (int)av[3], 0, 0, 0, 0};
  // head weights of the four output rows this lane holds: rows 4g+i = (p' = g/2, h' = 4(g%2)+i)
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int hh = 4 * (g & 1) + i;
    wv[i] = hh < a.HI ? a.w[((size_t)b * a.Tq + tq) * a.HI + hh] : 0.0f;
  }
  __syncthreads();

  const size_t kbase = (size_t)b * a.max_blocks;
  uint32_t* keys = a.keys + (size_t)q * a.max_blocks;
  const uint8_t* codes = a.idx_codes + kbase * 32;
  const uint8_t* scl = a.idx_scale + kbase * 2;
  for (int it = 0; it < kScoreIters; ++it) {
    const int64_t j0 = j_begin + ((int64_t)wave * kScoreIters + it) * 32;
    if (j0 >= N) break;
    // B operand: column n = lane%16 -> blocks j0+2n, j0+2n+1; K-group g -> (block 2n + g/2, half g%2)
    const int64_t jb = j0 + 2 * (lane & 15) + (g >> 1);
    uint4 bv = make_uint4(0u, 0u, 0u, 0u);
    int sb = 0;
    if (jb < N) {
      bv = *reinterpret_cast<const uint4*>(codes + jb * 32 + half * 16);
      sb = scl[jb * 2 + half];
    }
    const v8i Bv = {(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bv, acc, 4, 4, 0, sa, 0, sb);
    // lane holds C[4g+i][lane%16]: block jb (p' = g/2), heads 4(g%2)+i
    float e = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) e = fmaf(wv[i], relu(acc[i]), e);
    float s = __shfl_up(e, 16, 64);  // heads 0..3 of the same block, from row-group g-1
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(wv[i], relu(acc[i]), s);
    if ((g & 1) && jb < N) {
      if (s == 0.0f) s = 0.0f;
      uint32_t key = order_key(s);
      keys[jb] = key;
      atomicAdd(&hist[key >> 20], 1u);
    }
  }
  __syncthreads();

  // ---- chunk lower bound: lowest key of the histogram bin holding the k'-th largest score
  const int64_t G_q = (N + kScoreChunk - 1) / kScoreChunk;
  const int64_t rr = (G_q + 1) / 2;
  const uint32_t kp = (uint32_t)((a.k + rr - 1) / rr);
  const int top = kHistBins - 16 * tid;  // this thread's bins: [top-16, top), scanned downwards
  uint32_t cnt = 0;
  for (int i = 1; i <= 16; ++i) cnt += hist[top - i];
  uint32_t total;
  uint32_t excl = block_excl_scan(cnt, wsum, &total);
  if (total >= kp && excl < kp && excl + cnt >= kp) {
    uint32_t c = excl;
    for (int i = 1; i <= 16; ++i) {
      c += hist[top - i];
      if (c >= kp) {
        thr_s = (uint32_t)(top - i) << 20;
        break;
      }
    }
  }
  __syncthreads();
  if (tid == 0) a.thr[(size_t)q * a.G + blockIdx.x] = thr_s;
}

__global__ __launch_bounds__(256) void scan_kernel(ScoreArgs a) {
  __shared__ uint32_t sthr[2048];
  __shared__ uint32_t L_s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int q = blockIdx.y;
  const int tq = q % a.Tq;
  const int64_t N = visible_blocks(a, tq);
  if (N <= a.k) return;  // the select kernel takes every visible block
  const int64_t start = (int64_t)blockIdx.x * kScanPerWG;
  if (start >= N) return;
  const int G_q = (int)((N + kScoreChunk - 1) / kScoreChunk);
  const int rr = (G_q + 1) / 2;
  if (tid == 0) L_s = 0;
  for (int i = tid; i < G_q; i += 256) sthr[i] = a.thr[(size_t)q * a.G + i];
  __syncthreads();
  for (int i = tid; i < G_q; i += 256) {
    uint32_t v = sthr[i];
    int rank = 0;
    for (int j = 0; j < G_q; ++j) {
      uint32_t u = sthr[j];
      rank += (u > v) || (u == v && j < i);
    }
    if (rank == rr - 1) L_s = v;
  }
  __syncthreads();
  const uint32_t L = L_s;
  const int64_t end = (start + kScanPerWG < N) ? start + kScanPerWG : N;
  const uint32_t* keys = a.keys + (size_t)q * a.max_blocks;
  uint64_t* cand = a.cand + (size_t)q * kCandCap;
  for (int64_t base = start; base < end; base += 256) {
    const int64_t j = base + tid;
    uint32_t key = 0;
    bool pred = false;
    if (j < end) {
      key = keys[j];
      pred = key >= L;
    }
    uint64_t mask = __ballot(pred);
    if (mask == 0) continue;
    uint32_t n = (uint32_t)__popcll(mask);
    uint32_t pos = 0;
    if (lane == 0) pos = atomicAdd(&a.cand_cnt[q], n);
    pos = __shfl(pos, 0, 64);
    uint32_t rank = (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    if (pred && pos + rank < (uint32_t)kCandCap)
      cand[pos + rank] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
  }
}

__global__ __launch_bounds__(512) void select_kernel(ScoreArgs a) {
  __shared__ uint64_t cs[kCandCap];
  __shared__ int32_t list[2048];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_digit, sel_above, sel_count, n_win;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = blockIdx.x;
  const int tq = q % a.Tq;
  const int64_t N = visible_blocks(a, tq);
  int32_t* out = a.topk + (size_t)q * a.k;
  if (N <= a.k) {
    for (int i = tid; i < a.k; i += 512) out[i] = (i < N) ? i : -1;
    return;
  }
  const uint32_t total = a.cand_cnt[q];
  const bool fast = total <= (uint32_t)kCandCap;
  const int64_t n = fast ? (int64_t)total : N;
  const uint32_t* keys = a.keys + (size_t)q * a.max_blocks;
  if (fast) {
    const uint64_t* cand = a.cand + (size_t)q * kCandCap;
    for (int64_t i = tid; i < n; i += 512) cs[i] = cand[i];
  }
  if (tid == 0) n_win = 0;
  __syncthreads();
  auto elem = [&](int64_t i) -> uint64_t {
    if (fast) return cs[i];
    return ((uint64_t)keys[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
  };

  // radix select of the k-th largest 64-bit key, 8 bits at a time, stopping
  // as soon as the bin that holds it is taken whole
  uint64_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)a.k;  // N > k here
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += 512) {
      uint64_t e = elem(i);
      if ((e & mask) == prefix) atomicAdd(&hist[(uint32_t)(e >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane covers bins 255-4*lane .. 252-4*lane (descending)
      uint32_t c4 = 0;
      for (int i = 0; i < 4; ++i) c4 += hist[255 - 4 * lane - i];
      uint32_t incl = c4;
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      uint32_t excl = incl - c4;
      if (excl < need && incl >= need) {
        uint32_t c = excl;
        for (int i = 0; i < 4; ++i) {
          uint32_t d = 255 - 4 * lane - i;
          if (c + hist[d] >= need) {
            sel_digit = d;
            sel_above = c;
            sel_count = hist[d];
            break;
          }
          c += hist[d];
        }
      }
    }
    __syncthreads();
    const uint32_t d = sel_digit;
    need -= sel_above;
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)0xFF << shift;
    if (sel_count == need) break;
  }
  // winners: every element whose determined bits are >= the selected prefix
  for (int64_t i = tid; i < n; i += 512) {
    uint64_t e = elem(i);
    if ((e & mask) >= prefix) {
      uint32_t s = atomicAdd(&n_win, 1u);
      if (s < 2048u) list[s] = (int32_t)(0xFFFFFFFFu - (uint32_t)(e & 0xFFFFFFFFu));
    }
  }
  __syncthreads();
  const int kk = a.k;
  int n2 = 1;
  while (n2 < kk) n2 <<= 1;
  for (int i = kk + tid; i < n2; i += 512) list[i] = 0x7FFFFFFF;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += 512) {
        int lo = 2 * i - (i & (stride - 1));
        int hi = lo + stride;
        bool asc = (lo & size) == 0;
        int32_t x = list[lo], y = list[hi];
        if ((x > y) == asc) {
          list[lo] = y;
          list[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < kk; i += 512) out[i] = list[i];
}

}  // namespace

hipError_t launch_index_score(const ScoreArgs& a, int32_t B, hipStream_t s) {
  const int64_t N_last = a.len / a.m;  // visible blocks of the last query (t = len-1)
  if (N_last <= a.k) return hipSuccess;  // every visible block is selected; no scores needed
  const unsigned nq = (unsigned)(B * a.Tq);
  unsigned g1 = (unsigned)((N_last + kScoreChunk - 1) / kScoreChunk);
  hipLaunchKernelGGL(score_kernel, dim3(g1, nq), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_select(const ScoreArgs& a, int32_t B, hipStream_t s) {
  const int64_t N_last = a.len / a.m;
  const unsigned nq = (unsigned)(B * a.Tq);
  if (N_last > a.k) {
    unsigned g2 = (unsigned)((N_last + kScanPerWG - 1) / kScanPerWG);
    hipLaunchKernelGGL(scan_kernel, dim3(g2, nq), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(select_kernel, dim3(nq), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace lca
