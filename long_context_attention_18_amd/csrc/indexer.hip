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
// coalesced), so the kernel is a pure HBM stream. That argument needs the two
// terms J_b * 2^(S_b - 256) (J_b < 2^13 in magnitude, S_b = sum of the two
// E8M0 bytes of half b) to fit fp32's 24 bits together: measured on MI355X,
// the instruction is not round-to-nearest once they do not. So every block
// whose bytes give |S_0 - S_1| > 10, or a term outside fp32's normal range,
// is flagged (a ballot over the wave) and rescored exactly in fp64 from the
// codes -- the same sums in the same order as the definition. With real data
// the flag never fires; it keeps the top-k exact for any input.
// The head combine is done in
// the MFMA output layout: lanes of row-group 0/2 hold heads 0..3, row-group
// 1/3 heads 4..7, and one cross-lane move continues the fmaf chain.
// Each workgroup also counts, per bin of the top 12 bits of the ordered
// score key, its scores from its maximum down to a quarter of it, and adds
// those ~17 bins to a per-query global histogram.
//
// Kernel 2 (scan): L = the bottom of the highest bin at which the global
// histogram, summed from the top, reaches k. A bin's count can only be short
// (a chunk leaves out scores below its own cut), so at least k scores are >=
// L and every winner is >= L. Each workgroup compacts its scores >= L, in
// index order, into its own segment (wave ballots + one LDS prefix scan).
//
// Kernel 3 (select, select.h): one workgroup per query gathers the
// candidates into LDS in index order (or takes all N scores when there are
// too many), radix-selects the k-th largest 64-bit key (score_key << 32 |
// ~j) and writes the winners by an order-preserving compaction, so the
// output is ascending without a sort. Exact for any input.
//
// Calls with many queries (chunked prefill) take other shapes of kernel 1:
// 512+ queries, a workgroup per 8 chunks of a query (one set-up, one
// histogram); 2048+ queries that see at most kTileMaxBlocks blocks, query
// tiles (tile_kernel: 8 queries per workgroup on the 32x32x64 MFMA), which
// also do kernel 2's work, and kernel 3's for the combined call.
#include "dev_formats.h"
#include "ingest.h"
#include "kernels.h"
#include "select.h"
#include "attend_core.h"

namespace lca {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// bits(s) ^ 0xFFFFFFFF for a negative s, bits(s) | 0x80000000 otherwise: unsigned keys order like the floats
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float relu(float x) { return x > 0.0f ? x : 0.0f; }

// twice the E2M1 value of a code: magnitudes {0, 1, 2, 3, 4, 6, 8, 12}, bit 3 the sign
__device__ __forceinline__ int e2m1_x2(uint32_t c) {
  int m = (int)(c & 7u);
  int v = m < 4 ? m : (m < 6 ? 2 * m - 4 : 4 * m - 16);
  return (c & 8u) ? -v : v;
}

// Exact score of one block from its FP4 codes: per head, the two 32-element
// halves as integer dot products J_b of doubled values, the value
// J_0 * 2^(S_0 - 256) + J_1 * 2^(S_1 - 256) summed in fp64 and rounded once to
// fp32, then the ReLU-weighted fmaf chain over heads.
__device__ __forceinline__ float exact_block_score(const uint8_t* kc, int ks0, int ks1, const uint32_t* qcode /* [8][8] */,
                                                   const int* qscale /* [8][2] */, const float* w, int HI) {
  float acc = 0.0f;
  for (int h = 0; h < HI; ++h) {
    int J[2] = {0, 0};
    for (int c = 0; c < 64; ++c) {
      const int kq = e2m1_x2((kc[c >> 1] >> (4 * (c & 1))) & 15u);
      J[c >> 5] += e2m1_x2((qcode[h * 8 + (c >> 3)] >> (4 * (c & 7))) & 15u) * kq;
    }
    double D = 0.0;
    D = D + ldexp((double)J[0], qscale[h * 2 + 0] + ks0 - 256);
    D = D + ldexp((double)J[1], qscale[h * 2 + 1] + ks1 - 256);
    float sh = (float)D;
    acc = fmaf(w[h], sh > 0.0f ? sh : 0.0f, acc);
  }
  return acc == 0.0f ? 0.0f : acc;
}

// blocks visible to query row tq of sequence b (0 for a row without a query)
__device__ __forceinline__ int64_t visible_blocks(const ScoreArgs& a, int b, int tq) {
  const int64_t t = query_t(a.seq_len, a.seq_T, a.seq_cap, a.len, a.Tq, b, tq);
  return t < 0 ? 0 : (t + 1) / a.m;
}

// exclusive prefix sum of `v` over the threads of a workgroup of kScoreWaves waves (every caller's);
// *total gets the sum. The waves' sums are read all at once, branch-free.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kScoreWaves; ++w) {
    const uint32_t x = wsum[w];
    off += w < wave ? x : 0u;
    tot += x;
  }
  *total = tot;
  return off + incl - v;
}

// FP4 E2M1 code of v (fp32) by comparisons: the magnitude code counts the round-to-nearest-even
// decision points a passes (0.25 and 1.25, 2.5, 5 are ties that stay down; 0.75, 1.75, 3.5 ties that go up).
__device__ __forceinline__ uint32_t fp4_e2m1_code_cmp(float v) {
  const float a = fabsf(v);
  uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  // saturating: every a > 5 is code 7 (6.0). The query values x * 2^-E are exact in fp32 (a BF16 value
  // times a power of two), so this makes the fp64 encoder's decisions.
  return ((__float_as_uint(v) >> 28) & 8u) | m;
}

__device__ __forceinline__ float from_partner(float x, int odd_row) {
  // value of lane l ^ 16 (v_permlane16_swap: odd rows of the first operand <-> even rows of the second)
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(odd_row ? r[0] : r[1]);
}

__device__ __forceinline__ uint32_t from_partner_u(uint32_t x, int odd_row) {
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return odd_row ? r[0] : r[1];
}

// LDS of one score workgroup
struct ScoreLds {
  uint32_t hist[kHistBins];
  uint32_t qcode[8 * 8];  // quantised query [head][8 words of 8 codes]
  int qscale[8 * 2];      // its E8M0 bytes [head][half]
  int guard[6];           // block-scale bounds inside which the MFMA sum is exact
  uint32_t flag_blk[kScoreWaves][kScoreIters * 32];  // per wave: blocks to rescore exactly (offset in chunk)
  uint32_t n_flag[kScoreWaves];
  uint32_t wmax[kScoreWaves];
  uint32_t wcnt[kScoreWaves];  // per wave: its keys in the chunk's top bins
  uint32_t range;
  int lo;             // hist_cmin_bin's bin; the record floor's bin (-1: none)
  int lo_reached;     // hist_cmin_bin found its bin
  uint32_t lo_above;  // the count in the bins above it
  uint32_t lo_key;    // in-launch threshold: the record's floor key
  uint32_t sub[256];  // in-launch threshold: keys of the floor's bin by their next 8 bits
  int coop_last;         // this workgroup is the last of its query to arrive
  uint32_t coop_top;      // the last to arrive: the query's largest key
  uint32_t coop_bound;    // the last to arrive: the highest record floor
  uint32_t coop_lmin;     // the lowest record floor
  uint32_t coop_total;    // candidates over all records
};

// A workgroup's query: its MX-FP4 operands, head weights and exactness bounds (one per workgroup)
struct ScoreQuery {
  v8i A0, A1;
  int sA, sB;
  float wlo[4], whi[4];  // head weights 0..3 and 4..7 (0 for heads >= H_I)
  int dlo, dhi, k0lo, k0hi, k1lo, k1hi;
  const float* wq;
};

// A 16-byte non-temporal load (the key stream is read once per call: its lines need not stay cached).
__device__ __forceinline__ uint4 ld_stream16(const uint8_t* p) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const u4v x = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// All of a wave's key loads for one chunk (kScoreIters tiles x 16 B + 1 scale byte per lane), issued
// back to back in tile order (loads return in order, so the first tile pair can start as soon as its
// own data is in), non-temporal. FULL: the whole chunk is visible, so each address is one base plus a
// constant offset; otherwise each is clamped to the last visible block (always in bounds).
template <bool FULL, int ITERS = kScoreIters>
__device__ __forceinline__ void load_keys(const uint8_t* codes, const uint8_t* scl, int wave_j0, int n2, int half,
                                          int N, uint4 (&bvs)[ITERS], int (&sbs)[ITERS]) {
  if (FULL) {
    const uint8_t* cb = codes + (size_t)(wave_j0 + n2) * 32 + half * 16;
    const uint8_t* sb = scl + (size_t)(wave_j0 + n2) * 2 + half;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      bvs[it] = ld_stream16(cb + it * 32 * 32);
      sbs[it] = __builtin_nontemporal_load(sb + it * 32 * 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      int jb = wave_j0 + it * 32 + n2;
      jb = jb < N ? jb : N - 1;
      bvs[it] = ld_stream16(codes + (size_t)jb * 32 + half * 16);
      sbs[it] = __builtin_nontemporal_load(scl + (size_t)jb * 2 + half);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The MX-FP4 query and its exactness bounds, by one wave into LDS (the caller's barrier makes them
// visible), from this lane's slice qraw (lane -> head lane/8, dims 8*(lane%8)..+8): codes to
// qcode [head][8 words], E8M0 bytes to qscale [head][half], the six bounds to guard.
__device__ __forceinline__ void quantise_query_into(const ScoreArgs& a, uint4 qraw, uint32_t* qcode, int* qscale,
                                                    int* guard) {
  const int lane = threadIdx.x & 63;
  const int qh = lane >> 3, qpart = lane & 7;
  uint32_t word = 0, sbyte = 0;
  if (qh < a.HI) {
    float x[8];
    const uint32_t rw[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[2 * u] = __uint_as_float(rw[u] << 16);
      x[2 * u + 1] = __uint_as_float(rw[u] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));  // the four lanes of one 32-element block
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    if (amax > 0.0f) {
      int E = ilogbf(amax) - 2;
      E = E < -127 ? -127 : (E > 127 ? 127 : E);
      sbyte = (uint32_t)(E + 127);
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= fp4_e2m1_code_cmp(ldexpf(x[i], -E)) << (4 * i);
    }
  }
  qcode[qh * 8 + qpart] = word;
  if ((qpart & 3) == 0) qscale[qh * 2 + (qpart >> 2)] = (int)sbyte;
  // bounds: |S0 - S1| <= 10 and 130 <= S_b <= 370 for every live head, S_b = qs_b + ks_b.
  // Lane 8h holds head h's half-0 byte, lane 8h+4 its half-1 byte.
  const int q0 = __shfl((int)sbyte, (lane & 7) * 8, 64), q1 = __shfl((int)sbyte, (lane & 7) * 8 + 4, 64);
  const bool live = (lane & 7) < a.HI;
  int g0 = live ? -10 - (q0 - q1) : -100000, g1 = live ? 10 - (q0 - q1) : 100000;
  int g2 = live ? 130 - q0 : -100000, g3 = live ? 370 - q0 : 100000;
  int g4 = live ? 130 - q1 : -100000, g5 = live ? 370 - q1 : 100000;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    g0 = max(g0, __shfl_xor(g0, o, 64)); g1 = min(g1, __shfl_xor(g1, o, 64));
    g2 = max(g2, __shfl_xor(g2, o, 64)); g3 = min(g3, __shfl_xor(g3, o, 64));
    g4 = max(g4, __shfl_xor(g4, o, 64)); g5 = min(g5, __shfl_xor(g5, o, 64));
  }
  if (lane == 0) {
    guard[0] = g0; guard[1] = g1; guard[2] = g2; guard[3] = g3; guard[4] = g4; guard[5] = g5;
  }
}

__device__ __forceinline__ void quantise_query(const ScoreArgs& a, ScoreLds& S, uint4 qraw) {
  quantise_query_into(a, qraw, S.qcode, S.qscale, S.guard);
}

// After the barrier that follows quantise_query: the two A operands. Lane: row r = lane%16, K-group
// g = lane/16; row r holds (p, h) = (r/8, r%8) in operand A0 and (r/8, (r%8 + 4) % 8) in operand A1,
// its codes in K-groups 2p, 2p+1 only.
__device__ __forceinline__ void query_operands(const ScoreLds& S, ScoreQuery& Q) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4, p = r >> 3, odd = g & 1;
  const int hA = r & 7, hB = (hA + 4) & 7;
  uint32_t aA[4] = {0u, 0u, 0u, 0u}, aB[4] = {0u, 0u, 0u, 0u};
  Q.sA = 127;
  Q.sB = 127;
  if ((g >> 1) == p) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      aA[u] = S.qcode[hA * 8 + odd * 4 + u];
      aB[u] = S.qcode[hB * 8 + odd * 4 + u];
    }
    Q.sA = S.qscale[hA * 2 + odd];
    Q.sB = S.qscale[hB * 2 + odd];
  }
  Q.A0 = (v8i){(int)aA[0], (int)aA[1], (int)aA[2], (int)aA[3], 0, 0, 0, 0};
  Q.A1 = (v8i){(int)aB[0], (int)aB[1], (int)aB[2], (int)aB[3], 0, 0, 0, 0};
  Q.dlo = S.guard[0]; Q.dhi = S.guard[1]; Q.k0lo = S.guard[2]; Q.k0hi = S.guard[3]; Q.k1lo = S.guard[4];
  Q.k1hi = S.guard[5];
}

// One chunk's scores from its loaded keys: the key of every visible block to `keys`, this lane's key
// per tile pair to lane_keys (0 = no block); blocks outside the exactness bounds are rescored in fp64.
// Contains workgroup barriers: every thread of the workgroup calls it.
// keys: the query's global key row (written through); lkeys (or null): the workgroup's LDS key array,
// indexed by the block's offset from j_begin, which gets the keys too (the in-launch threshold).
template <bool FULL, int ITERS = kScoreIters>
__device__ __forceinline__ void score_pairs(const ScoreArgs& a, ScoreLds& S, const ScoreQuery& Q, const uint4 (&bvs)[ITERS],
                                            const int (&sbs)[ITERS], uint32_t* keys, const uint8_t* codes,
                                            const uint8_t* scl, int N, int j_begin, int wave_j0, int n2,
                                            uint32_t (&lane_keys)[ITERS / 2], uint32_t* lkeys = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int odd = (lane >> 4) & 1;
  if (lane == 0) S.n_flag[wave] = 0;  // this wave's own list: program order suffices
#pragma unroll
  for (int pr = 0; pr < ITERS / 2; ++pr) {
    const int tA = 2 * pr, tB = 2 * pr + 1;
    const bool liveA = FULL || wave_j0 + tA * 32 + n2 < N, liveB = FULL || wave_j0 + tB * 32 + n2 < N;
    const uint4 bA = liveA ? bvs[tA] : make_uint4(0u, 0u, 0u, 0u);
    const uint4 bB = liveB ? bvs[tB] : make_uint4(0u, 0u, 0u, 0u);
    const int sbA = liveA ? sbs[tA] : 0, sbB = liveB ? sbs[tB] : 0;
    const v8i BA = {(int)bA.x, (int)bA.y, (int)bA.z, (int)bA.w, 0, 0, 0, 0};
    const v8i BB = {(int)bB.x, (int)bB.y, (int)bB.z, (int)bB.w, 0, 0, 0, 0};
    v4f accA = {0.0f, 0.0f, 0.0f, 0.0f}, accB = {0.0f, 0.0f, 0.0f, 0.0f};
    accA = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.A0, BA, accA, 4, 4, 0, Q.sA, 0, sbA);
    accB = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.A1, BB, accB, 4, 4, 0, Q.sB, 0, sbB);
    // rows 4g..4g+3 of this lane: tile A gives heads 0..3 on even g, 4..7 on odd g; tile B the reverse.
    // Heads 0..3 first (fmaf chain from +0), then the partner lane (g^1) continues with heads 4..7.
    float e = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) e = fmaf(Q.wlo[i], relu(odd ? accB[i] : accA[i]), e);
    float sc = from_partner(e, odd);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc = fmaf(Q.whi[i], relu(odd ? accA[i] : accB[i]), sc);
    // this lane now holds the final score of block jb: tile A if g is odd, tile B if even
    const int jb = wave_j0 + (odd ? tA : tB) * 32 + n2;
    const uint32_t other = from_partner_u((uint32_t)sbA | ((uint32_t)sbB << 8), odd);
    const int own = odd ? sbA : sbB;
    const int oth = odd ? (int)(other & 0xFFu) : (int)(other >> 8);
    const int ks0 = odd ? oth : own, ks1 = odd ? own : oth;
    const int dk = ks0 - ks1;
    const bool bad = dk < Q.dlo || dk > Q.dhi || ks0 < Q.k0lo || ks0 > Q.k0hi || ks1 < Q.k1lo || ks1 > Q.k1hi;
    uint32_t key = 0;
    if (FULL || jb < N) {
      if (sc == 0.0f) sc = 0.0f;
      key = order_key(sc);
      // written through to memory (agent scope): the next launch reads it from other XCDs, and the
      // launch's end then has no dirty lines of it to write back
      __hip_atomic_store(&keys[jb], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lkeys) lkeys[jb - j_begin] = key;
      if (bad) S.flag_blk[wave][atomicAdd(&S.n_flag[wave], 1u)] = (uint32_t)(jb - j_begin);
    }
    lane_keys[pr] = key;
  }
  __syncthreads();
  // exact rescoring of the flagged blocks (none with real data); the reload below picks the new keys up
  uint32_t nf = 0;
  for (int w = 0; w < kScoreWaves; ++w) {
    const uint32_t n = S.n_flag[w];
    for (uint32_t f = tid; f < n; f += kScoreThreads) {
      const int jb = j_begin + (int)S.flag_blk[w][f];
      const float ex = exact_block_score(codes + (size_t)jb * 32, scl[(size_t)jb * 2], scl[(size_t)jb * 2 + 1],
                                         S.qcode, S.qscale, Q.wq, a.HI);
      __hip_atomic_store(&keys[jb], order_key(ex), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lkeys) lkeys[jb - j_begin] = order_key(ex);
    }
    nf += n;
  }
  if (nf != 0) {
    __syncthreads();
    __threadfence_block();
#pragma unroll
    for (int pr = 0; pr < ITERS / 2; ++pr) {
      const int jb = wave_j0 + ((odd ? 2 * pr : 2 * pr + 1)) * 32 + n2;
      if (FULL || jb < N) lane_keys[pr] = lkeys ? lkeys[jb - j_begin] : keys[jb];
    }
  }
}

// The workgroup's maximum key (all threads get it); `m` is this lane's
__device__ __forceinline__ uint32_t wg_max_key(ScoreLds& S, uint32_t m) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // inclusive prefix maximum through DPP (the steps of wave_incl_scan): lane 63 ends with the wave's
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x111, 0xf, 0xf, false));  // row_shr:1
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x112, 0xf, 0xf, false));  // row_shr:2
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x114, 0xf, 0xf, false));  // row_shr:4
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x118, 0xf, 0xf, false));  // row_shr:8
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x142, 0xa, 0xf, false));  // row_bcast:15
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x143, 0xc, 0xf, false));  // row_bcast:31
  if (lane == 63) S.wmax[wave] = m;
  __syncthreads();
  uint32_t kmax = 0;
#pragma unroll
  for (int w = 0; w < kScoreWaves; ++w) kmax = max(kmax, S.wmax[w]);
  return kmax;
}

// lo = the highest bin at which the LDS histogram, counted from the top, reaches cmin (S.lo; every
// thread calls it)
__device__ __forceinline__ int hist_cmin_bin(ScoreLds& S, uint32_t cmin) {
  const int tid = threadIdx.x;
  constexpr int kPerT = kHistBins / kScoreThreads;  // bins per thread
  if (tid == 0) {
    S.lo = 0;
    S.lo_reached = 0;
  }
  __syncthreads();
  const int hi_b = kHistBins - kPerT * tid;  // this thread: bins [hi_b - kPerT, hi_b), threads in descending order
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 1; i <= kPerT; ++i) cnt += S.hist[hi_b - i];
  uint32_t tot;
  const uint32_t excl = block_excl_scan(cnt, S.wmax, &tot);
  if (excl < cmin && excl + cnt >= cmin) {
    uint32_t c = excl;
    for (int i = 1; i <= kPerT; ++i) {
      const uint32_t above = c;
      c += S.hist[hi_b - i];
      if (c >= cmin) {
        S.lo = hi_b - i;
        S.lo_above = above;
        S.lo_reached = 1;
        break;
      }
    }
  }
  __syncthreads();
  return S.lo;
}

// The LDS histogram's bins lo .. top_bin into the query's global histogram
__device__ __forceinline__ void hist_publish(const ScoreArgs& a, ScoreLds& S, int q, int lo, int top_bin) {
  for (int i = lo + (int)threadIdx.x; i <= top_bin; i += kScoreThreads) {
    const uint32_t c = S.hist[i];
    if (c) atomicAdd(&q_hist(a, q)[i], c);
  }
}

// the query's head weights (0 for heads >= H_I)
__device__ __forceinline__ void load_weights(const ScoreArgs& a, int b, int tq, ScoreQuery& Q) {
  Q.wq = a.w + ((size_t)b * a.Tq + tq) * a.HI;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Q.wlo[i] = i < a.HI ? Q.wq[i] : 0.0f;
    Q.whi[i] = i + 4 < a.HI ? Q.wq[i + 4] : 0.0f;
  }
}

// The query's loads (its MX-FP4 slice for quantise_query, the head weights) into Q / qraw
__device__ __forceinline__ uint4 load_query(const ScoreArgs& a, int b, int tq, ScoreQuery& Q) {
  const int lane = threadIdx.x & 63;
  const int qh = lane >> 3, qpart = lane & 7;
  uint4 qraw = make_uint4(0u, 0u, 0u, 0u);
  if (qh < a.HI) qraw = *reinterpret_cast<const uint4*>(a.qI + (((size_t)b * a.Tq + tq) * a.HI + qh) * kIdxDim + qpart * 8);
  load_weights(a, b, tq, Q);
  return qraw;
}

// In-launch threshold: the chunk's record floor and largest key (*top), from the keys in registers; every
// thread calls it. The floor is the lowest key at which the chunk's count from the top still fits its record
// (pref_slots words): every nonzero key goes into the LDS histogram of the top 12 key bits, wave 0 finds the
// bin B where the count from the top first exceeds pref_slots (64 bins a round, from the largest key's bin
// down), and a histogram of B's keys by their next 8 bits gives the lowest boundary of those sub-bins at
// which the count still fits. No such bin: every key fits, floor 0. (A floor on whole bins sits above the
// query's k-th key whenever one chunk holds more than its record's worth of keys in a crowded bin that also
// holds the k-th.) Four barriers.
template <int NA, int NB>
__device__ __forceinline__ uint32_t coop_floor(const ScoreArgs& a, ScoreLds& S, const uint32_t (&ka)[NA],
                                               const uint32_t (&kb)[NB], uint32_t* top) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  (void)tid;
  const uint32_t need = (uint32_t)a.pref_slots + 1u;
  uint32_t m = 0;
#pragma unroll
  for (int pr = 0; pr < NA + NB; ++pr) {
    const uint32_t key = pr < NA ? ka[pr] : kb[pr - NA];
    m = max(m, key);
    if (key != 0) atomicAdd(&S.hist[key >> 20], 1u);
  }
  const uint32_t kmax = wg_max_key(S, m);  // (its barrier also completes the histogram)
  if (top) *top = kmax;
  if (wave == 0) {
    uint32_t above = 0;  // keys in the bins above this round's
    for (int hi = (int)(kmax >> 20); hi >= 0; hi -= 64) {
      const int bin = hi - lane;
      const uint32_t h = bin >= 0 ? S.hist[bin] : 0u;
      const uint32_t c = wave_incl_scan(h) + above;  // count of bins hi..bin
      const uint64_t over = __ballot(c >= need);
      if (over) {
        if (lane == __ffsll((long long)over) - 1) {
          S.lo = bin;
          S.lo_above = c - h;
        }
        break;
      }
      above = (uint32_t)__builtin_amdgcn_readlane((int)c, 63);
    }
  }
  __syncthreads();
  const int B = S.lo;
  if (B < 0) return 0u;
  const uint32_t room = need - 1u - S.lo_above;  // keys of B the record can take
#pragma unroll
  for (int pr = 0; pr < NA + NB; ++pr) {
    const uint32_t key = pr < NA ? ka[pr] : kb[pr - NA];
    if (key != 0 && (int)(key >> 20) == B) atomicAdd(&S.sub[(key >> 12) & 255u], 1u);
  }
  __syncthreads();
  if (wave == 0) {
    // lane l: sub-bins 255-4l .. 252-4l; the first whose count from the top exceeds room
    uint32_t h4[4], c4 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h4[i] = S.sub[255 - 4 * lane - i];
      c4 += h4[i];
    }
    const uint32_t incl = wave_incl_scan(c4);
    if (incl - c4 <= room && incl > room) {
      uint32_t c = incl - c4, sb = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (c + h4[i] > room) {
          sb = (uint32_t)(255 - 4 * lane - i);
          break;
        }
        c += h4[i];
      }
      const uint64_t f = ((uint64_t)(uint32_t)B << 20) + ((uint64_t)(sb + 1u) << 12);  // (B + 1) << 20 when sb = 255
      S.lo_key = f > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)f;  // all-ones: no candidates
    }
  }
  __syncthreads();
  return S.lo_key;
}

// One score workgroup's chunk: kScoreChunk blocks from j_begin (few-query calls: every workgroup one
// chunk). The keys' loads go out before the query is quantised.
// lkeys (in-launch threshold): the workgroup's LDS key array -- the chunk's keys at offsets 0..2047,
// the folded chunk's from kScoreChunk on -- which gets every key too. Returns the lowest bin published.
template <bool FULL>
__device__ __forceinline__ int score_chunk(const ScoreArgs& a, ScoreLds& S, int q, int b, int tq, int N, int j_begin,
                                           int j_tail, uint32_t* lkeys = nullptr, uint32_t* top = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  ScoreQuery Q;
  const uint4 qraw = load_query(a, b, tq, Q);
  const size_t kbase = (size_t)b * a.max_blocks;
  uint32_t* keys = q_keys(a, q);
  const uint8_t* codes = a.idx_codes + kbase * 32;
  const uint8_t* scl = a.idx_scale + kbase * 2;
  const int wave_j0 = j_begin + wave * kScoreIters * 32;
  const int n2 = 2 * (lane & 15) + ((lane >> 4) >> 1);  // block of this lane inside a 32-block tile
  uint4 bvs[kScoreIters];
  int sbs[kScoreIters];
  load_keys<FULL>(codes, scl, wave_j0, n2, (lane >> 4) & 1, N, bvs, sbs);
  // a folded last chunk (blocks j_tail..N-1, at most half a chunk: kTailIters tiles per wave), loaded
  // with this one and scored after it into the same histogram
  constexpr int kTailIters = kScoreIters / 2;
  const bool has_tail = j_tail >= 0 && j_tail < N;
  const int wave_t0 = j_tail + wave * kTailIters * 32;
  uint4 tvs[kTailIters];
  int tsb[kTailIters];
  if (has_tail) load_keys<false, kTailIters>(codes, scl, wave_t0, n2, (lane >> 4) & 1, N, tvs, tsb);
  for (int i = tid; i < kHistBins; i += kScoreThreads) S.hist[i] = 0;
  if (a.coop && tid < 256) S.sub[tid] = 0;
  if (a.coop && tid == 0) S.lo = -1;
  if (wave == 0) quantise_query(a, S, qraw);
  __syncthreads();  // quantised query and bounds visible
  query_operands(S, Q);
  uint32_t lane_keys[kScoreIters / 2];
  score_pairs<FULL>(a, S, Q, bvs, sbs, keys, codes, scl, N, j_begin, wave_j0, n2, lane_keys, lkeys);
  uint32_t tail_keys[kTailIters / 2];
#pragma unroll
  for (int pr = 0; pr < kTailIters / 2; ++pr) tail_keys[pr] = 0u;
  if (has_tail) {
    __syncthreads();  // every wave has read the first chunk's flag lists
    score_pairs<false, kTailIters>(a, S, Q, tvs, tsb, keys, codes, scl, N, j_tail, wave_t0, n2, tail_keys,
                                   lkeys ? lkeys + kScoreChunk : nullptr);
  }
  if (a.coop) return (int)coop_floor(a, S, lane_keys, tail_keys, top);
  // ---- top of this chunk into the query's global histogram (top 12 key bits): the chunk max's bin
  // and the 16 bins below it (down to a quarter of the max), or, when those hold fewer than cmin of the
  // chunk's keys, every bin down to where the chunk's count from the top reaches cmin. Counts in a bin
  // only ever undercount, so the bin where the global count from the top reaches k is a lower bound of
  // the k-th largest key; cmin (twice a chunk's share of k) keeps that bound tight when the scores
  // bunch up, e.g. all <= 0 (every indexer weight negative): the max is then 0 and the keys of negative
  // scores lie far below its bin.
  uint32_t m = 0;
#pragma unroll
  for (int pr = 0; pr < kScoreIters / 2; ++pr) m = max(m, lane_keys[pr]);
#pragma unroll
  for (int pr = 0; pr < kTailIters / 2; ++pr) m = max(m, tail_keys[pr]);
  const uint32_t kmax = wg_max_key(S, m);
  const int top_bin = (int)(kmax >> 20);
  const int low_bin = top_bin >= 16 ? top_bin - 16 : 0;
  uint32_t in_range = 0;  // this lane's keys in bins low_bin..top_bin
#pragma unroll
  for (int pr = 0; pr < (kScoreIters + kTailIters) / 2; ++pr) {
    const uint32_t key = pr < kScoreIters / 2 ? lane_keys[pr] : tail_keys[pr - kScoreIters / 2];
    if (key != 0 && (int)(key >> 20) >= low_bin) {
      atomicAdd(&S.hist[key >> 20], 1u);
      ++in_range;
    }
  }
  in_range = wave_incl_scan(in_range);  // lane 63: the wave's count
  if (lane == 63) S.wcnt[wave] = in_range;
  __syncthreads();  // the histogram adds and the counts are visible
  uint32_t range = 0;
#pragma unroll
  for (int w = 0; w < kScoreWaves; ++w) range += S.wcnt[w];
  int lo = low_bin;
  const uint32_t need = (uint32_t)a.cmin;
  const bool all_in = range < need && low_bin > 0;
  if (all_in) {
    // the rest of the chunk's keys, then the highest bin at which the count from the top reaches cmin
#pragma unroll
    for (int pr = 0; pr < (kScoreIters + kTailIters) / 2; ++pr) {
      const uint32_t key = pr < kScoreIters / 2 ? lane_keys[pr] : tail_keys[pr - kScoreIters / 2];
      if (key != 0 && (int)(key >> 20) < low_bin) atomicAdd(&S.hist[key >> 20], 1u);
    }
    lo = hist_cmin_bin(S, (uint32_t)a.cmin);
  }
  hist_publish(a, S, q, lo, top_bin);
  return lo;
}

// A workgroup over chunks chunk0, chunk0 + step, ... of its query (many-query calls, where one
// workgroup per chunk would repeat the query's set-up and histogram for every 2048 blocks): the query
// is quantised once, every key of its chunks is counted in the LDS histogram, and the histogram is
// published once, from the workgroup's maximum's bin down by 16 bins or to cmin keys.
__device__ __forceinline__ void score_multi(const ScoreArgs& a, ScoreLds& S, int q, int b, int tq, int N, int chunk0,
                                            int step) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  ScoreQuery Q;
  const uint4 qraw = load_query(a, b, tq, Q);
  const size_t kbase = (size_t)b * a.max_blocks;
  uint32_t* keys = q_keys(a, q);
  const uint8_t* codes = a.idx_codes + kbase * 32;
  const uint8_t* scl = a.idx_scale + kbase * 2;
  const int n2 = 2 * (lane & 15) + ((lane >> 4) >> 1);
  const int half = (lane >> 4) & 1;
  for (int i = tid; i < kHistBins; i += kScoreThreads) S.hist[i] = 0;
  if (wave == 0) quantise_query(a, S, qraw);
  __syncthreads();
  query_operands(S, Q);
  uint32_t m = 0;
  for (int c = chunk0; c * kScoreChunk < N; c += step) {
    const int j_begin = c * kScoreChunk;
    const int wave_j0 = j_begin + wave * kScoreIters * 32;
    uint4 bvs[kScoreIters];
    int sbs[kScoreIters];
    uint32_t lane_keys[kScoreIters / 2];
    if (j_begin + kScoreChunk <= N) {
      load_keys<true>(codes, scl, wave_j0, n2, half, N, bvs, sbs);
      score_pairs<true>(a, S, Q, bvs, sbs, keys, codes, scl, N, j_begin, wave_j0, n2, lane_keys);
    } else {
      load_keys<false>(codes, scl, wave_j0, n2, half, N, bvs, sbs);
      score_pairs<false>(a, S, Q, bvs, sbs, keys, codes, scl, N, j_begin, wave_j0, n2, lane_keys);
    }
#pragma unroll
    for (int pr = 0; pr < kScoreIters / 2; ++pr) {
      const uint32_t key = lane_keys[pr];
      m = max(m, key);
      if (key != 0) atomicAdd(&S.hist[key >> 20], 1u);
    }
    __syncthreads();  // every wave has read the flag lists: the next chunk may reuse them
  }
  const uint32_t kmax = wg_max_key(S, m);  // (its barrier also orders the histogram adds before the reads)
  const int top_bin = (int)(kmax >> 20);
  const int low_bin = top_bin >= 16 ? top_bin - 16 : 0;
  if (wave == 0) {
    uint32_t v = (lane <= top_bin - low_bin) ? S.hist[low_bin + lane] : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o, 64);
    if (lane == 0) S.range = v;
  }
  __syncthreads();
  const int lo = (S.range < (uint32_t)a.cmin && low_bin > 0) ? hist_cmin_bin(S, (uint32_t)a.cmin) : low_bin;
  hist_publish(a, S, q, lo, top_bin);
}

// blockIdx.x: a chunk of the query (a.chunk_step = 0) or the first of the chunks x, x + step, ...
__global__ __launch_bounds__(kScoreThreads, 4) void score_kernel(ScoreArgs a) {  // <= 128 VGPRs: 2 per CU
  __shared__ ScoreLds S;
  const int q = blockIdx.y;
  const int b = q / a.Tq, tq = q % a.Tq;
  const int N = (int)visible_blocks(a, b, tq);
  const int c0 = blockIdx.x;
  if (c0 * kScoreChunk >= N) return;
  if (a.chunk_step > 0) {
    score_multi(a, S, q, b, tq, N, c0, a.chunk_step);
    return;
  }
  const int j_begin = c0 * kScoreChunk;
  const int j_tail = a.fold_tail && c0 == 0 ? (int)gridDim.x * kScoreChunk : -1;  // the chunk the grid leaves out
  if (j_begin + kScoreChunk <= N) score_chunk<true>(a, S, q, b, tq, N, j_begin, j_tail);
  else score_chunk<false>(a, S, q, b, tq, N, j_begin, j_tail);
}

// ---- In-launch threshold and selection (decode-sized calls) -----------------------------------------------
//
// No workgroup waits for another. Each score workgroup writes its keys to the query's key row and one
// record per chunk: a header (the chunk's largest key, its floor bin lo, its candidate count) and its
// candidates, the keys of bins >= lo in block order (zero-padded; a score's key is never 0), lo as low as
// cmin candidates -- twice its share of k plus 16 -- still fit. Then it counts itself in at the query's
// counter and ends. The last to arrive has every other workgroup's writes complete behind the counter: it
// reads all records (one round of coalesced loads, kept in registers) and takes F = the highest floor.
// Every record holds all of its keys >= F, so the candidates >= F are exactly the query's keys >= F; when
// there are at least k of them they hold the top-k: a radix select on their 32-bit keys (LDS histograms
// only), then the winners straight from the loaded records in block order, equal keys by lower block
// first. Otherwise (a chunk with far more than its share of the winners), it takes the keys above a lower
// bound from the key row in memory instead: the lowest floor, which every candidate clears, so that with k
// candidates in all at least k keys do (else every key). Everything one workgroup writes for another goes
// through memory at agent scope (the XCDs' L2s are not coherent), and a workgroup's writes complete before
// it counts itself in.

struct CoopLds {
  union {
    struct {
      ScoreLds sc;
      uint32_t keys[kScoreChunk + kScoreChunk / 2];  // every visible block's key: the chunk, then the folded one
    } s;
    SelectLds sel;  // the last workgroup selects
  } u;
};

__device__ __forceinline__ void st_agent64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A record: the keys at LDS offsets 0..n-1 (blocks j0..j0+n-1) >= the floor key L, in block order,
// zero-padded to R words (the caller's floor keeps them within R), and its header (the floor key, the bin
// of the workgroup's largest key, the count). Every thread calls it.
__device__ __forceinline__ void coop_record(const uint32_t* lk, int n, int64_t j0, uint32_t L, uint32_t top,
                                            uint64_t* hdr, uint64_t* cand, int R, uint32_t* wsum) {
  constexpr int kPer = kScoreChunk / kScoreThreads;  // consecutive blocks per thread
  const int i0 = (int)threadIdx.x * kPer;
  uint32_t kv[kPer];
  uint32_t c = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    kv[u] = i0 + u < n ? lk[i0 + u] : 0u;
    c += (i0 + u < n && kv[u] >= L) ? 1u : 0u;
  }
  uint32_t total;
  uint32_t pos = block_excl_scan(c, wsum, &total);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (i0 + u < n && kv[u] >= L) {
      const uint32_t j = (uint32_t)(j0 + i0 + u);
      st_agent64(&cand[pos], ((uint64_t)kv[u] << 32) | (uint64_t)(0xFFFFFFFFu - j));
      ++pos;
    }
  }
  for (int i = (int)total + (int)threadIdx.x; i < R; i += kScoreThreads) st_agent64(&cand[i], 0ull);
  if (threadIdx.x == 0) st_agent64(hdr, ((uint64_t)L << 32) | ((uint64_t)(top >> 20) << 16) | total);
  __syncthreads();  // wsum is reused by the next call
}

// The last to arrive, over every key of the query's row in memory: the keys >= the lower bound L in block
// order into LDS (loads in batches of 16 keys per thread), then the selection in LDS; or, when more than
// fit, the selection over every key straight from memory.
__device__ __forceinline__ uint32_t coop_select_row(const ScoreArgs& a, SelectLds& S, int q, int N, uint32_t L,
                                                    int32_t* out, int32_t* out2) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* keys = q_keys(a, q);
  for (int i = tid; i < kRadixBins; i += kScoreThreads) S.hist[i] = 0u;
  if (tid == 0) {
    S.small_n = 0u;
    S.sel_count = 0u;  // candidates so far
  }
  if (tid < 64) S.small[tid] = 0ull;
  __syncthreads();
  constexpr int kBatch = 16 * kScoreThreads;  // keys per batch: 16 consecutive per thread
  uint64_t lo = ~0ull, hi = 0;
  bool fits = true;
  for (int j0 = 0; j0 < N && fits; j0 += kBatch) {
    uint32_t kv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = j0 + tid * 16 + u;
      kv[u] = j < N ? __hip_atomic_load(&keys[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    }
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) c += (j0 + tid * 16 + u < N && kv[u] >= L) ? 1u : 0u;
    const uint32_t base = S.sel_count;
    uint32_t total;
    uint32_t pos = block_excl_scan(c, S.wsum, &total);
    if (base + total <= (uint32_t)kCandCap) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int j = j0 + tid * 16 + u;
        if (j < N && kv[u] >= L) {
          const uint64_t e = ((uint64_t)kv[u] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
          S.cs[base + pos++] = e;
          lo = e < lo ? e : lo;
          hi = e > hi ? e : hi;
        }
      }
    }
    __syncthreads();  // every thread has read sel_count and wsum
    if (tid == 0) S.sel_count = base + total;
    __syncthreads();
    fits = S.sel_count <= (uint32_t)kCandCap;
  }
  const uint32_t n = S.sel_count;
  if (fits && n >= (uint32_t)a.k) {
    (void)lane;
    (void)wave;
    return select_core<true>(a, S, (int64_t)n, lo, hi, [&](int64_t i) -> uint64_t { return S.cs[i]; }, out,
                             out2);
  }
  // more candidates than the LDS holds: every key, straight from memory
  auto elem = [&](int64_t i) -> uint64_t {
    const uint32_t k = __hip_atomic_load(&keys[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
  };
  lo = ~0ull;
  hi = 0;
  for (int i = tid; i < N; i += kScoreThreads) {
    const uint64_t e = elem(i);
    lo = e < lo ? e : lo;
    hi = e > hi ? e : hi;
  }
  __syncthreads();
  return select_core<true>(a, S, (int64_t)N, lo, hi, elem, out, out2);
}

// The last workgroup of a query to arrive: the selection into the workspace list (and topk), over NL
// loaded record words per thread. Predicates are combined without short-circuit and LDS reads issued
// together, so that no wave waits on one LDS round trip per loaded word.
template <int NL>
__device__ __forceinline__ void coop_select(const ScoreArgs& a, CoopLds& L, int q, int N) {
  ScoreLds& S = L.u.s.sc;
  SelectLds& T = L.u.sel;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = (N + kScoreChunk - 1) / kScoreChunk;  // records (one per chunk)
  const int R = a.pref_slots;
  const int n_words = G * R;
  const uint64_t* hdr = q_rec(a, q);
  const uint64_t* cw = hdr + kRecHdrSlots;
  // ---- one round of loads: the headers (thread t: record t) and every record's words (wave w, load u,
  // lane l: word 64 (NL w + u) + l, so each wave holds a contiguous run of the words, in block order along
  // (u, lane))
  const uint64_t h = tid < G ? ld_agent64(&hdr[tid]) : 0ull;
  uint64_t v[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int w = 64 * (NL * wave + u) + lane;
    v[u] = w < n_words ? ld_agent64(&cw[w]) : 0ull;
  }
  // ---- headers: the highest and lowest floor, the largest key and the count over all records
  if (wave * 64 < G) {
    const bool hv = tid < G;
    const uint64_t f = h >> 32;  // the record's floor key
    uint64_t fmin = hv ? f : ~0ull, fmax = hv ? f : 0ull;
    wave_minmax_u64(fmin, fmax);
    // an upper bound of the record's keys: the end of its largest key's bin
    uint64_t dummy = ~0ull, top = hv ? ((((h >> 16) & 0xFFFull) << 20) | 0xFFFFFull) : 0ull;
    wave_minmax_u64(dummy, top);
    const uint32_t cnt = wave_incl_scan(hv ? (uint32_t)h & 0xFFFFu : 0u);
    if (lane == 63) {
      atomicMax(&S.coop_bound, (uint32_t)fmax);
      atomicMin(&S.coop_lmin, (uint32_t)fmin);
      atomicMax(&S.coop_top, (uint32_t)top);
      atomicAdd(&S.coop_total, cnt);
    }
  }
  for (int i = tid; i < kRadixBins; i += kScoreThreads) T.hist[i] = 0u;  // (beyond the score LDS)
  __syncthreads();
  const uint32_t F = S.coop_bound;  // the highest floor key
  int32_t* out = q_list(a, q);
  int32_t* out2 = a.topk ? a.topk + (size_t)q * a.k : nullptr;
  uint32_t n = 0;
  bool fast = F != 0xFFFFFFFFu;  // (all ones: a record holds no key, its top bin alone overflowing it)
  if (fast) {
    // ---- radix select of the k-th largest key among the candidates (keys >= Fk, all <= the largest key
    // Kt, so they share the bits above the highest bit in which Fk and Kt differ), kRadixBits at a time,
    // until the digit bin that holds it is taken whole or the bits run out (equal keys). The first pass
    // also counts the candidates.
    const uint32_t Fk = F ? F : 1u, Kt = S.coop_top;
    int hb = 31 - __clz(Fk ^ Kt);
    hb = hb < 0 ? 0 : hb;
    uint32_t mask = hb >= 31 ? 0u : ~((2u << hb) - 1u);
    uint32_t prefix = Fk & mask;
    uint32_t need = (uint32_t)a.k;
    for (int shift = hb - (kRadixBits - 1); shift > -kRadixBits; shift -= kRadixBits) {
      const int sh = shift < 0 ? 0 : shift;  // the last digit may be narrower
      const uint32_t dmask = shift < 0 ? ((1u << (shift + kRadixBits)) - 1u) : (uint32_t)(kRadixBins - 1);
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const uint32_t key = (uint32_t)(v[u] >> 32);
        if ((key >= Fk) & ((key & mask) == prefix)) atomicAdd(&T.hist[(key >> sh) & dmask], 1u);
      }
      __syncthreads();
      // counts from the top: thread t holds bins 2047-4t .. 2044-4t (cleared for the next pass)
      uint32_t h4[4], c4 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h4[i] = T.hist[kRadixBins - 1 - 4 * tid - i];
        c4 += h4[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) T.hist[kRadixBins - 1 - 4 * tid - i] = 0u;
      const uint32_t excl = excl_scan_512(c4, T.wsum);
      if (shift == hb - (kRadixBits - 1)) {  // the first pass: every candidate counted
        uint32_t C = 0;
#pragma unroll
        for (int w = 0; w < kScoreWaves; ++w) C += T.wsum[w];
        if (C < (uint32_t)a.k) {
          fast = false;
          break;
        }
      }
      if (excl < need && excl + c4 >= need) {
        uint32_t c = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (c + h4[i] >= need) {
            T.sel_digit = (uint32_t)(kRadixBins - 1 - 4 * tid - i);
            T.sel_above = c;
            T.sel_count = h4[i];
            break;
          }
          c += h4[i];
        }
      }
      __syncthreads();
      need -= T.sel_above;
      prefix |= T.sel_digit << sh;
      mask |= dmask << sh;
      if (T.sel_count == need) break;
    }
    if (fast) {
      // ---- the winners in block order: the candidates above the boundary bin, and of those in it (equal
      // keys once the bits ran out) the first `need`. Each wave counts both kinds over its run of words
      // (ballots), the waves exchange their counts once, and each lane's position is its wave's offset
      // plus the count of winners before it in the wave's run.
      uint64_t mg[NL], me[NL];
      uint32_t cg = 0, ce = 0;
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const uint32_t key = (uint32_t)(v[u] >> 32);
        const bool in = key >= Fk;
        mg[u] = __ballot(in & ((key & mask) > prefix));
        me[u] = __ballot(in & ((key & mask) == prefix));
        cg += (uint32_t)__popcll(mg[u]);
        ce += (uint32_t)__popcll(me[u]);
      }
      if (lane == 0) S.flag_blk[1][wave] = cg | (ce << 16);  // at most 64 NL < 2^16 each
      __syncthreads();
      uint32_t bg = 0, be = 0, ng = 0, ne = 0;
#pragma unroll
      for (int w = 0; w < kScoreWaves; ++w) {
        const uint32_t x = S.flag_blk[1][w];
        if (w < wave) {
          bg += x & 0xFFFFu;
          be += x >> 16;
        }
        ng += x & 0xFFFFu;
        ne += x >> 16;
      }
      const uint64_t lm = (1ull << lane) - 1ull;
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const bool gt = (mg[u] >> lane) & 1ull, eq = (me[u] >> lane) & 1ull;
        const uint32_t gb = bg + (uint32_t)__popcll(mg[u] & lm);
        const uint32_t eb = be + (uint32_t)__popcll(me[u] & lm);
        if (gt | (eq & (eb < need))) {
          const uint32_t pos = gb + (eb < need ? eb : need);
          const int32_t jb = (int32_t)(0xFFFFFFFFu - (uint32_t)v[u]);
          if (pos < (uint32_t)a.k) {
            __hip_atomic_store(&out[pos], jb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (out2) out2[pos] = jb;
          }
        }
        bg += (uint32_t)__popcll(mg[u]);
        be += (uint32_t)__popcll(me[u]);
      }
      n = ng + (ne < need ? ne : need);
      n = n < (uint32_t)a.k ? n : (uint32_t)a.k;
    }
  }
  if (!fast) {
    // fewer than k keys >= F (a crowded chunk): a lower bound of the k-th key, then the key row
    const uint32_t Lkey = S.coop_total >= (uint32_t)a.k ? S.coop_lmin : 0u;
    __syncthreads();
    n = coop_select_row(a, T, q, N, Lkey, out, out2);
  }
  for (int i = (int)n + tid; i < a.k; i += kScoreThreads) {  // only if fewer than k were found
    __hip_atomic_store(&out[i], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (out2) out2[i] = -1;
  }
}

// grid (max(n_cols, B), B*Tq [+ 1]): x = chunk of query y; the extra last row (app_units > 0) writes the
// step's append, workgroup x for sequence x.
// Score workgroup (query q, chunk column c0) of the one-launch indexer. token != 0 (the step launch): the
// last to arrive also publishes the list, once every thread's list stores have completed, by storing token
// into the query's ready word, which the attention workgroups of the same launch wait for.
template <int NL>
__device__ __forceinline__ void index_select_wg(const ScoreArgs& a, CoopLds& L, int q, int c0, uint32_t token) {
  const int tid = threadIdx.x;
  const int b = q / a.Tq, tq = q % a.Tq;
  if (query_t(a.seq_len, a.seq_T, a.seq_cap, a.len, a.Tq, b, tq) < 0) return;  // ragged batch: no query in this row
  const int N = (int)visible_blocks(a, b, tq);
  if (N <= a.k) {
    // every visible block is selected: no scores; the attention takes them all without a list
    if (c0 == 0 && a.topk) {
      int32_t* o = a.topk + (size_t)q * a.k;
      for (int i = tid; i < a.k; i += kScoreThreads) o[i] = i < N ? i : -1;
    }
    return;
  }
  if (c0 * kScoreChunk >= N) return;
  const int j_begin = c0 * kScoreChunk;
  // the chunk the grid leaves out goes to a column that differs from query to query (two workgroups with
  // the extra chunk on one compute unit would end last)
  const int fold_col = (int)(((unsigned)q * 37u) % (unsigned)a.n_cols);
  const int j_tail = a.fold_tail && c0 == fold_col ? a.n_cols * kScoreChunk : -1;
  ScoreLds& S = L.u.s.sc;
  uint32_t top;  // the chunk's largest key
  const uint32_t lo = (uint32_t)(j_begin + kScoreChunk <= N
                                     ? score_chunk<true>(a, S, q, b, tq, N, j_begin, j_tail, L.u.s.keys, &top)
                                     : score_chunk<false>(a, S, q, b, tq, N, j_begin, j_tail, L.u.s.keys, &top));
  // this workgroup's record (the folded chunk's in its own record, after the others)
  uint64_t* hdr = q_rec(a, q);
  uint64_t* cw = hdr + kRecHdrSlots;
  const int R = a.pref_slots;
  coop_record(L.u.s.keys, min(kScoreChunk, N - j_begin), j_begin, lo, top, hdr + c0, cw + (size_t)c0 * R, R,
              S.wmax);
  if (j_tail >= 0 && j_tail < N)
    coop_record(L.u.s.keys + kScoreChunk, N - j_tail, j_tail, lo, top, hdr + a.n_cols, cw + (size_t)a.n_cols * R,
                R, S.wmax);
  if (tid == 0) {  // the last to arrive: the selection's LDS counters
    S.coop_top = 0u;
    S.coop_bound = 0u;
    S.coop_lmin = ~0u;
    S.coop_total = 0u;
  }
  // count in (this thread's key and record writes complete first); the last to arrive goes on
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* sync = q_sync(a, q);
  const int n_act = min(a.n_cols, (N + kScoreChunk - 1) / kScoreChunk);  // this query's score workgroups
  if (tid == 0)
    S.coop_last = __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (uint32_t)(n_act - 1);
  __syncthreads();
  if (!S.coop_last) return;
  if (tid == 0) __hip_atomic_store(sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next call
  coop_select<NL>(a, L, q, N);
  if (token != 0u) {
    __builtin_amdgcn_s_waitcnt(0);  // this thread's list stores have completed
    __syncthreads();
    if (tid == 0) __hip_atomic_store(sync + kSyncReady, token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// grid (max(n_cols, B), B*Tq [+ 1]): x = chunk of query y; the extra last row (app_units > 0) writes the
// step's append, workgroup x for sequence x.
template <int NL>
__global__ __launch_bounds__(kScoreThreads, 4) void index_select_kernel(ScanArgs args) {  // <= 128 VGPRs
  __shared__ CoopLds L;
  if (args.app_units > 0 && (int)blockIdx.y == (int)gridDim.y - 1) {
    const int b = blockIdx.x;
    if (b < args.app.B)
      for (int unit = (int)(threadIdx.x >> 6); unit < args.app_units; unit += kScoreWaves)
        append_unit<true>(args.app, b, unit, threadIdx.x & 63);
    return;
  }
  if ((int)blockIdx.x >= args.a.n_cols) return;
  index_select_wg<NL>(args.a, L, (int)blockIdx.y, (int)blockIdx.x, 0u);
}

// ---- The CSA decode step in one launch: the indexer above and the attention over its lists ---------------
//
// Workgroups [0, n_idx) are the score workgroups of index_select_kernel (query-major, n_cols a query, the
// count rounded up to a multiple of 8 so that the attention's ids keep their XCD); the rest are attention
// workgroups (query, 16-head group, key split), placed as attend_kernel places them. An attention workgroup
// that needs its query's list (the query sees more than k blocks) waits for the token its query's last score
// workgroup stores once the list is complete, then loads its split's slice of the list with agent-scope
// loads. The wait cannot deadlock: score workgroups never wait, and the attention workgroups come last in
// the grid (they are dispatched after every score workgroup, and while they wait they hold fewer compute
// units than the grid's score workgroups can run on). It is bounded all the same (kStepWaitTicks of the
// 100 MHz clock): a workgroup that gives up attends no keys and poisons its partial, so the query's output
// rows are NaN rather than silently wrong. The step's append (window entries, tail) is written by the
// attention workgroups that read the window, as in the dense attention launch.
struct StepAttnLds {
  AttnWaveLds w;
  int32_t list[kStepListMax];  // this split's slice of the list
  int last;                    // this workgroup merges the splits
  uint32_t timed_out;
  float cos_t[32], sin_t[32];
};

__device__ __forceinline__ bool wait_token(const uint32_t* word, uint32_t token) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != token) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > kStepWaitTicks) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Attention workgroup (query q, head group hg, key split) of the step launch.
__device__ __forceinline__ void step_attend(const StepArgs& sa, StepAttnLds& S, int q, int hg, int split) {
  const AttendArgs& args = sa.att;
  const AttnArgs& a = args.t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int b = q / a.Tq, tq = q % a.Tq;
  const int64_t t = query_t(a.seq_len, a.seq_T, a.seq_cap, a.len, a.Tq, b, tq);
  if (t < 0) return;  // ragged batch: no query in this row
  const int64_t N = min((t + 1) / a.m, a.max_blocks);
  Keys K;
  K.win_codes = a.win_codes;
  K.blk_codes = a.blk_codes;
  K.win_rope = a.win_rope;
  K.blk_rope = a.blk_rope;
  K.win_scale = a.win_scale;
  K.blk_scale = a.blk_scale;
  K.ring = (uint32_t)a.ring;
  K.list = S.list;
  K.win_row = (size_t)b * a.ring;
  K.blk_row = (size_t)b * a.max_blocks;
  K.n_win = (int)((int64_t)a.W < t + 1 ? (int64_t)a.W : t + 1);
  K.win_base = (uint32_t)((t - K.n_win + 1) % a.ring);
  K.j_max = N > 0 ? N - 1 : 0;
  // the selection's list (k winners when N > k); a query that sees at most k blocks takes them all
  K.use_list = N > a.k;
  K.n_list = (int)(N > a.k ? (int64_t)a.k : N);
  if (tid < 32) {
    float sn, cs;
    rope_angle(t, a.inv_freq[tid], &sn, &cs);
    S.cos_t[tid] = cs;
    S.sin_t[tid] = sn;
  }
  const int head = hg * 16 + r;
  const bool head_ok = head < a.H;
  u32x4 qraw[4];
  {
    const uint16_t* qp = a.q + (((size_t)b * a.Tq + tq) * a.H + (head_ok ? head : 0)) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qraw[ks] = head_ok ? *reinterpret_cast<const u32x4*>(qp + ks * 32 + 8 * g) : (u32x4){0u, 0u, 0u, 0u};
  }
  const int n_keys = K.n_win + K.n_list;
  const int splits = args.splits;
  const int per_split = ((n_keys + splits * 16 - 1) / (splits * 16)) * 16;
  const int s_begin = split * per_split;
  int s_end = min(s_begin + per_split, n_keys);
  if (args.app_units > 0) {
    // the step's append: every workgroup whose slots reach into the window writes all of its sequence's
    // new window entries (the same bytes from each) and reads them back after the fence and barrier below;
    // the tail copies (with the indexer's inputs) go to head group 0 of split 0. One wave per unit.
    const bool reads_window = s_begin < K.n_win;
    const bool writes_tail = hg == 0 && split == 0;
    for (int unit = wave; unit < args.app_units; unit += kWaves)
      if (unit < args.app.n_win ? reads_window : writes_tail) append_unit<true>(args.app, b, unit, lane);
    __threadfence_block();
  }
  K.list0 = 0;
  if (K.use_list) {
    if (tid == 0) S.timed_out = wait_token(q_sync(args.s, q) + kSyncReady, sa.token) ? 0u : 1u;
    __syncthreads();
    const int l0 = min(max(s_begin - K.n_win, 0), K.n_list), l1 = min(max(s_end - K.n_win, 0), K.n_list);
    const int32_t* lp = q_list(args.s, q);
    for (int i = l0 + tid; i < l1; i += kScoreThreads)
      S.list[i - l0] = __hip_atomic_load(&lp[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    K.list0 = l0;
  } else if (tid == 0) {
    S.timed_out = 0u;
  }
  __syncthreads();
  const bool poison = S.timed_out != 0u;
  if (poison) s_end = s_begin;
  bf16x8 qb[4];
  rotate_query(qraw, S.cos_t, S.sin_t, g, qb);
  float m_run, l_run;
  v4f O[8];
  attend_slots<1>(K, s_begin, s_end, per_split, qb, S.w, wave, r, g, m_run, l_run, O);
  attend_finish(args, S.w, &S.last, q, hg, split, m_run, l_run, O, poison);
}

template <int NL>
__global__ __launch_bounds__(kScoreThreads, 4) void csa_step_kernel(StepArgs sa) {  // <= 128 VGPRs
  __shared__ union {
    CoopLds idx;
    StepAttnLds att;
  } U;
  const int lin = (int)blockIdx.x;
  if (lin < sa.n_idx) {
    const int cols = sa.idx.a.n_cols;
    const int q = lin / cols, c0 = lin - q * cols;
    if (q < sa.n_queries) index_select_wg<NL>(sa.idx.a, U.idx, q, c0, sa.token);
    return;
  }
  // the attention workgroups: consecutive logical ids (the head groups of a (query, split)) inside one XCD's
  // share, as in attend_kernel; n_idx is a multiple of 8, so la % 8 is the XCD
  const unsigned total = (unsigned)sa.n_att, la = (unsigned)(lin - sa.n_idx);
  const unsigned xcd = la % 8u, pos = la / 8u;
  const unsigned logical = xcd * (total / 8u) + min(xcd, total % 8u) + pos;
  const int hgs = (sa.att.t.H + 15) / 16;
  const unsigned per_q = (unsigned)(hgs * sa.att.splits);
  const int q = (int)(logical / per_q);
  const int hg = (int)(logical % per_q) % hgs;
  const int split = (int)(logical % per_q) / hgs;
  step_attend(sa, U.att, q, hg, split);
}

// ---- Many-query calls (chunked prefill): query tiles on the 32x32x64 scaled MFMA ------------------------
//
// A workgroup takes kTileQueries consecutive queries of one sequence and every block any of them sees, so
// each key it loads serves all of them. Per 32-block tile a wave runs two
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands (queries 0-3, then 4-7): K is the 64-dim key (lanes
// 0-31 hold dims 0-31, lanes 32-63 dims 32-63, each with its own E8M0 byte), B column n is block n of the
// tile, and A row r is one (query, head) pair, placed so that the output lands where the head sum wants
// it: output register i of lane l holds row 8 (i/4) + 4 (l/32) + i%4, so row r is given query
// (r/16) + 2 ((r/4) % 2) and head 4 ((r/8) % 2) + r%4, and lane l then holds in registers 0-7 all eight
// heads of query 2 (l/32) and in registers 8-15 those of query 2 (l/32) + 1. The fmaf chain over heads
// runs in one lane, in the definition's order, with no lane exchange. Every product term is useful, and
// the exactness argument of the score kernel holds unchanged (each output is the same two scaled exact
// terms; the same bounds flag the blocks that need the fp64 rescoring).
// Pass 1 counts every score of the workgroup's queries in per-query LDS histograms (4096 bins of the top
// 12 key bits, two 16-bit counts per word: a query sees at most kTileMaxBlocks blocks), which give each
// query the exact bin L at which the count from the top reaches k, and the number of keys in bins >= L.
// Pass 2 scores again (the same instructions, so the same keys) and writes every key >= L, in index
// order, into the candidate segments the selection reads (wave ballots and one LDS count exchange per
// round of kTileWaves tiles). No per-block score goes to memory, unless the call asks for them
// (write_keys) or a query's candidates would not fit the selection's LDS (its keys then serve the
// selection's path over every block).
struct TileLds {
  uint32_t hist[kTileQueries][kHistBins / 2];  // bin 2i in the low half of word i, bin 2i+1 in the high half
  uint32_t qcode[kTileQueries][64];
  int qscale[kTileQueries][16];
  int guard[kTileQueries][6];
  alignas(16) uint32_t cnt[2][kTileWaves][8];  // pass 2: candidates per (wave, lane slot j + 4 half) of a round
  alignas(16) float wts[kTileQueries][8];      // head weights (0 beyond H_I), read per tile: registers are short
  uint32_t Lkey[kTileQueries];
  uint32_t ncand[kTileQueries];                // keys in bins >= L
  uint32_t countL[kTileQueries];               // keys in bin L
  uint32_t bcnt[kTileQueries];                 // pass 2: bin-L candidates gathered in LDS so far
  int32_t Nq[kTileQueries];                    // blocks the query scores (0: none)
};

// query of the tile held by slot j (0-3) of a lane in half `half` (lanes 0-31: 0, 1, 4, 5; 32-63: 2, 3, 6, 7)
__device__ __forceinline__ int tile_slot_query(int j, int half) { return (j & 1) + 2 * half + 4 * (j >> 1); }

// This lane's MFMA query operands, the blocks its four queries see and the bounds all queries satisfy
struct TileQuery {
  v8i A0, A1;
  int sA0, sA1;
  int N[4];
  int g[6];
};

// ReLU on the bit pattern: every negative float (and -0) has a negative int pattern, so max(int, 0) maps
// it to +0 and keeps every positive float; one integer max instead of a NaN-quieting float max pair
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Keys of block jb (the lane's column) for this lane's four queries, from its loaded key slice; 0 where
// the query does not see the block. Every lane of the wave calls it (MFMA and lane swap).
template <bool CHECK>
__device__ __forceinline__ void tile_keys(const ScoreArgs& a, const TileLds& S, const TileQuery& Q, const uint8_t* codes,
                                          uint4 kb, int ks, int jb, int jc, uint32_t (&key)[4]) {
  const int half = (threadIdx.x >> 5) & 1;
  const v8i B = {(int)kb.x, (int)kb.y, (int)kb.z, (int)kb.w, 0, 0, 0, 0};
  v16f c[2];
  c[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Q.A0, B, (v16f){}, 4, 4, 0, Q.sA0, 0, ks);
  c[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Q.A1, B, (v16f){}, 4, 4, 0, Q.sA1, 0, ks);
  auto rs = __builtin_amdgcn_permlane32_swap((uint32_t)ks, (uint32_t)ks, false, false);
  const int ko = (int)(half ? rs[0] : rs[1]);  // the other half's scale byte of the same block
  const int ks0 = half ? ko : ks, ks1 = half ? ks : ko;
  const int dk = ks0 - ks1;
  const bool ok_all = dk >= Q.g[0] && dk <= Q.g[1] && ks0 >= Q.g[2] && ks0 <= Q.g[3] && ks1 >= Q.g[4] &&
                      ks1 <= Q.g[5];
  float e[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = tile_slot_query(j, half);
    const float4 wa = *reinterpret_cast<const float4*>(&S.wts[q][0]);
    const float4 wb = *reinterpret_cast<const float4*>(&S.wts[q][4]);
    const int base = 8 * (j & 1);
    const v16f& cj = c[j >> 1];
    float x = 0.0f;  // starts at +0, so it never becomes -0
    x = fmaf(wa.x, relu_bits(cj[base + 0]), x);
    x = fmaf(wa.y, relu_bits(cj[base + 1]), x);
    x = fmaf(wa.z, relu_bits(cj[base + 2]), x);
    x = fmaf(wa.w, relu_bits(cj[base + 3]), x);
    x = fmaf(wb.x, relu_bits(cj[base + 4]), x);
    x = fmaf(wb.y, relu_bits(cj[base + 5]), x);
    x = fmaf(wb.z, relu_bits(cj[base + 6]), x);
    x = fmaf(wb.w, relu_bits(cj[base + 7]), x);
    e[j] = x;
  }
  if (!ok_all) {
    // a block outside some query's exactness bounds: those queries' scores in fp64 (never with real data;
    // one rolled loop keeps this path's registers out of the main path's)
    const int tq0 = blockIdx.x * kTileQueries;
#pragma unroll 1
    for (int j = 0; j < 4; ++j) {
      const int q = tile_slot_query(j, half);
      const int* g = S.guard[q];
      if (dk < g[0] || dk > g[1] || ks0 < g[2] || ks0 > g[3] || ks1 < g[4] || ks1 > g[5]) {
        const int tq = tq0 + q < a.Tq ? tq0 + q : a.Tq - 1;
        const float x = exact_block_score(codes + (size_t)jc * 32, ks0, ks1, S.qcode[q], S.qscale[q],
                                          a.w + ((size_t)blockIdx.y * a.Tq + tq) * a.HI, a.HI);
        e[0] = j == 0 ? x : e[0];
        e[1] = j == 1 ? x : e[1];
        e[2] = j == 2 ? x : e[2];
        e[3] = j == 3 ? x : e[3];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) key[j] = (!CHECK || jb < Q.N[j]) ? order_key(e[j]) : 0u;
}

// tile_keys, with the per-query visibility test only for a tile that reaches past the fewest blocks a
// scoring query of the workgroup sees (Nmin); a query that scores nothing needs no zero keys
__device__ __forceinline__ void tile_keys_at(const ScoreArgs& a, const TileLds& S, const TileQuery& Q, const uint8_t* codes,
                                             uint4 kb, int ks, int t, int Nmin, int jc, uint32_t (&key)[4]) {
  const int jb = t * 32 + (threadIdx.x & 31);
  if (t * 32 + 32 <= Nmin) tile_keys<false>(a, S, Q, codes, kb, ks, jb, jc, key);
  else tile_keys<true>(a, S, Q, codes, kb, ks, jb, jc, key);
}

// This lane's key slice of block jb (clamped to the last block any query sees: always in bounds)
__device__ __forceinline__ void tile_load(const uint8_t* codes, const uint8_t* scl, int jb, int Nmax, uint4& kb, int& ks,
                                          int& jc) {
  const int half = (threadIdx.x >> 5) & 1;
  jc = jb < Nmax ? jb : Nmax - 1;
  kb = *reinterpret_cast<const uint4*>(codes + (size_t)jc * 32 + half * 16);
  ks = scl[(size_t)jc * 2 + half];
}

// Pass 3 of the combined call, one wave per query (row tq of sequence b, tile slot q): the query's top-k
// list from its candidates. Every candidate in a bin above L is a winner; of the countL keys in bin L,
// the `need` = k - (ncand - countL) largest (64-bit key, then lower index) are, found by a radix
// select over the bin's keys (8-bit digits below the bin's 12 bits, from the LDS copy pass 2 gathered,
// or, when the bin was too full for it, from the candidates in memory) until the digit's bin is taken
// whole or holds at most 64 keys, which are ranked directly. The winners then go out in index order
// (the candidates' order) with ballot prefix counts. The query's 8 KB of histogram words are the
// wave's scratch: the bin-L copy (kTileBoundCap keys), the segment offsets, the digit bins.
__device__ __forceinline__ void tile_select(const ScoreArgs& a, TileLds& S, int b, int tq, int q) {
  const int lane = threadIdx.x & 63;
  if (tq >= a.Tq) return;
  const int64_t t = query_t(a.seq_len, a.seq_T, a.seq_cap, a.len, a.Tq, b, tq);
  if (t < 0) return;  // ragged: no query in this row
  const int64_t N = (t + 1) / a.m;
  const int qg = b * a.Tq + tq;
  int32_t* out = a.topk + (size_t)qg * a.k;
  if (N <= a.k) {  // every visible block, then -1
    for (int i = lane; i < a.k; i += 64) out[i] = (i < N) ? i : -1;
    return;
  }
  uint32_t* wl = &S.hist[q][0];
  const uint64_t* blist = reinterpret_cast<const uint64_t*>(wl);  // words [0, 2 kTileBoundCap)
  uint32_t* pref = wl + 2 * kTileBoundCap;                         // G + 1 segment offsets
  uint32_t* rbin = pref + kTilePrefWords;                          // 256 digit bins (8-byte aligned)
  uint64_t* small = reinterpret_cast<uint64_t*>(rbin);             // or 64 keys to rank (aliases rbin)
  const uint64_t* cand = q_cand(a, qg);
  const int G = (int)((N + kTileSeg - 1) / kTileSeg);
  // segment offsets (exclusive prefix of the counts pass 2 wrote), in rounds of 64 segments
  uint32_t total = 0;
  for (int s0 = 0; s0 < G; s0 += 64) {
    const uint32_t c = s0 + lane < G ? q_seg(a, qg)[s0 + lane] : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (s0 + lane < G) pref[s0 + lane] = total + incl - c;
    total += (uint32_t)__shfl((int)incl, 63, 64);
  }
  if (lane == 0) pref[G] = total;
  // candidate e of flat index i (index order): its segment by binary search over the offsets
  auto flat = [&](uint32_t i) -> uint64_t {
    int lo = 0, hi = G;  // pref[lo] <= i < pref[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pref[mid] <= i) lo = mid;
      else hi = mid;
    }
    return cand[(size_t)lo * kTileSeg + (i - pref[lo])];
  };
  const uint32_t Lbin = S.Lkey[q] >> 20;
  const uint32_t countL = S.countL[q];
  uint32_t need = (uint32_t)a.k - (S.ncand[q] - countL);  // 1 <= need <= countL
  const bool in_lds = countL <= (uint32_t)kTileBoundCap;
  const uint32_t n_src = in_lds ? countL : total;
  auto src = [&](uint32_t i) -> uint64_t { return in_lds ? blist[i] : flat(i); };
  // radix select of the need-th largest key of bin L: (e & mask) == prefix selects the current bin
  uint64_t prefix = (uint64_t)Lbin << 52, mask = 0xFFF0000000000000ull;
  uint32_t cnt = countL;
  // (keys are unique, so the 52 bits below the bin settle it by sh = -4; the bound only guards the loop)
  for (int sh = 44; cnt != need && sh > -12; sh -= 8) {
    const uint64_t dmask = sh >= 0 ? 0xFFull : (0xFFull >> -sh);  // the last digit: bits 3..0
    const int shc = sh >= 0 ? sh : 0;
    if (cnt <= 64) {
      // at most 64 keys left: gather them and rank directly (keys are unique)
      small[lane] = 0ull;  // unused slots rank below every key
      uint32_t ns = 0;
      for (uint32_t i0 = 0; i0 < n_src; i0 += 64) {
        const uint32_t i = i0 + lane;
        const uint64_t e = i < n_src ? src(i) : 0ull;
        const bool m = i < n_src && (e & mask) == prefix;
        const uint64_t bm = __ballot(m);
        const uint32_t at = ns + __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
        if (m && at < 64u) small[at] = e;
        ns += (uint32_t)__popcll(bm);
      }
      const uint64_t mine = small[lane];
      uint32_t rank = 0;
#pragma unroll
      for (int m = 0; m < 64; ++m) rank += small[m] > mine ? 1u : 0u;
      const uint64_t th = __ballot(lane < (int)cnt && rank == need - 1);
      prefix = (uint64_t)__shfl((long long)mine, th ? (int)__builtin_ctzll(th) : 0, 64);
      mask = ~0ull;
      break;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) rbin[lane + 64 * u] = 0u;
    for (uint32_t i = lane; i < n_src; i += 64) {
      const uint64_t e = src(i);
      if ((e & mask) == prefix) atomicAdd(&rbin[(uint32_t)((e >> shc) & dmask)], 1u);
    }
    // digit whose count from the top reaches need: lane l holds bins 255-4l .. 252-4l
    uint32_t h4[4], c4 = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      h4[u] = rbin[255 - 4 * lane - u];
      c4 += h4[u];
    }
    const uint32_t incl = wave_incl_scan(c4);
    const uint32_t excl = incl - c4;
    uint32_t dsel = 0, above = 0, cd = 0;
    if (excl < need && incl >= need) {
      uint32_t run = excl;
      for (int u = 0; u < 4; ++u) {
        if (run + h4[u] >= need) {
          dsel = 255u - 4u * lane - u;
          above = run;
          cd = h4[u];
          break;
        }
        run += h4[u];
      }
    }
    const uint64_t owner = __ballot(excl < need && incl >= need);
    const int ol = owner ? (int)__builtin_ctzll(owner) : 0;
    dsel = (uint32_t)__shfl((int)dsel, ol, 64);
    above = (uint32_t)__shfl((int)above, ol, 64);
    cd = (uint32_t)__shfl((int)cd, ol, 64);
    need -= above;
    prefix |= (uint64_t)dsel << shc;
    mask |= dmask << shc;
    cnt = cd;
  }
  // winners: (e & mask) >= prefix (every key of a higher bin or digit, and the bin's chosen ones), out in
  // index order
  uint32_t pos = 0;
  for (uint32_t i0 = 0; i0 < total; i0 += 256) {  // 256 candidates per round, their loads issued together
    uint64_t e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = i0 + 64u * u + (uint32_t)lane;
      e[u] = i < total ? flat(i) : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = i0 + 64u * u + (uint32_t)lane;
      const bool w = i < total && (e[u] & mask) >= prefix;
      const uint64_t bm = __ballot(w);
      const uint32_t p = pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
      if (w && p < (uint32_t)a.k) out[p] = (int32_t)(0xFFFFFFFFu - (uint32_t)(e[u] & 0xFFFFFFFFu));
      pos += (uint32_t)__popcll(bm);
    }
  }
  for (uint32_t i = pos + lane; i < (uint32_t)a.k; i += 64) out[i] = -1;  // only if fewer than k were found
}

__global__ __launch_bounds__(kTileWaves * 64, 4) void tile_kernel(ScoreArgs a) {
  __shared__ TileLds S;
  constexpr int kThreads = kTileWaves * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int b = blockIdx.y;
  const int tq0 = blockIdx.x * kTileQueries;
  // the blocks each query scores: all it sees when it selects (N > k) or the call keeps every key, else
  // none (the selection writes the list of a query with N <= k)
  if (tid < kTileQueries) {
    const int tq = tq0 + tid;
    const int64_t N = tq < a.Tq ? visible_blocks(a, b, tq) : 0;
    S.Nq[tid] = (N > a.k || a.write_keys) ? (int32_t)N : 0;
  }
  if (tid < kTileQueries * 8) {
    const int q = tid >> 3, h = tid & 7;
    const int tq = tq0 + q < a.Tq ? tq0 + q : a.Tq - 1;
    S.wts[q][h] = h < a.HI ? a.w[((size_t)b * a.Tq + tq) * a.HI + h] : 0.0f;
  }
  for (int i = tid; i < kTileQueries * kHistBins / 2; i += kThreads) (&S.hist[0][0])[i] = 0u;
  // wave w quantises query w (a query that scores nothing gets bounds nothing fails)
  if (wave < kTileQueries) {
    const int tq = tq0 + wave < a.Tq ? tq0 + wave : a.Tq - 1;
    ScoreQuery Qs;
    const uint4 qraw = load_query(a, b, tq, Qs);
    quantise_query_into(a, qraw, S.qcode[wave], S.qscale[wave], S.guard[wave]);
  }
  __syncthreads();
  if (tid < kTileQueries && S.Nq[tid] == 0) {
    S.guard[tid][0] = -100000; S.guard[tid][1] = 100000; S.guard[tid][2] = -100000;
    S.guard[tid][3] = 100000; S.guard[tid][4] = -100000; S.guard[tid][5] = 100000;
  }
  __syncthreads();
  int Nmax = 0, Nmin = 0x7FFFFFFF;
#pragma unroll
  for (int q = 0; q < kTileQueries; ++q) {
    Nmax = max(Nmax, (int)S.Nq[q]);
    if (S.Nq[q] > 0) Nmin = min(Nmin, (int)S.Nq[q]);
  }
  if (Nmax == 0) {  // no query of the tile scores anything; the combined call still wants their lists
    if (a.topk && a.tile_select) tile_select(a, S, b, tq0 + wave, wave);
    return;
  }

  TileQuery Q;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    int v = S.guard[0][i];
#pragma unroll
    for (int q = 1; q < kTileQueries; ++q) v = (i & 1) ? min(v, S.guard[q][i]) : max(v, S.guard[q][i]);
    Q.g[i] = v;
  }
  {
    // A row lane%32 = r: query (r/16) + 2 ((r/4) % 2) (+4 in A1), head 4 ((r/8) % 2) + r%4; this lane's
    // half of the 64 dims
    const int r = lane & 31;
    const int qi = (r >> 4) + 2 * ((r >> 2) & 1), h = 4 * ((r >> 3) & 1) + (r & 3);
    uint32_t x[4], y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[u] = S.qcode[qi][h * 8 + half * 4 + u];
      y[u] = S.qcode[qi + 4][h * 8 + half * 4 + u];
    }
    Q.A0 = (v8i){(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
    Q.A1 = (v8i){(int)y[0], (int)y[1], (int)y[2], (int)y[3], 0, 0, 0, 0};
    Q.sA0 = S.qscale[qi][h * 2 + half];
    Q.sA1 = S.qscale[qi + 4][h * 2 + half];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) Q.N[j] = S.Nq[tile_slot_query(j, half)];
  const size_t kbase = (size_t)b * a.max_blocks;
  const uint8_t* codes = a.idx_codes + kbase * 32;
  const uint8_t* scl = a.idx_scale + kbase * 2;
  const int nt = (Nmax + 31) / 32;

  // ---- pass 1: histograms (the next tile's key slice is loaded before this one is scored)
  {
    uint4 kb;
    int ks, jc;
    int t = wave;
    if (t < nt) tile_load(codes, scl, t * 32 + (lane & 31), Nmax, kb, ks, jc);
    for (; t < nt; t += kTileWaves) {
      uint4 kb2 = kb;
      int ks2 = ks, jc2 = jc;
      if (t + kTileWaves < nt) tile_load(codes, scl, (t + kTileWaves) * 32 + (lane & 31), Nmax, kb2, ks2, jc2);
      uint32_t key[4];
      tile_keys_at(a, S, Q, codes, kb, ks, t, Nmin, jc, key);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (key[j] != 0u) {
          const uint32_t bin = key[j] >> 20;
          atomicAdd(&S.hist[tile_slot_query(j, half)][bin >> 1], 1u << ((bin & 1u) << 4));
        }
      }
      kb = kb2;
      ks = ks2;
      jc = jc2;
    }
  }
  __syncthreads();
  // ---- per query (wave w: query w): the bin where the count from the top reaches k
  if (wave < kTileQueries && S.Nq[wave] > a.k) {
    const uint32_t* hq = S.hist[wave];
    const uint32_t kk = (uint32_t)a.k;
    const int top = kHistBins / 2 - 32 * lane;  // this lane: words top-32 .. top-1 (64 bins), from the top
    uint32_t c = 0;
#pragma unroll
    for (int i = 1; i <= 32; ++i) {
      const uint32_t v = hq[top - i];
      c += (v & 0xFFFFu) + (v >> 16);
    }
    const uint32_t incl = wave_incl_scan(c);
    const uint32_t excl = incl - c;
    if (excl < kk && incl >= kk) {
      uint32_t run = excl;
      for (int i = 1; i <= 32; ++i) {
        const uint32_t v = hq[top - i];
        run += v >> 16;
        if (run >= kk) {
          S.Lkey[wave] = (uint32_t)(2 * (top - i) + 1) << 20;
          S.countL[wave] = v >> 16;
          break;
        }
        run += v & 0xFFFFu;
        if (run >= kk) {
          S.Lkey[wave] = (uint32_t)(2 * (top - i)) << 20;
          S.countL[wave] = v & 0xFFFFu;
          break;
        }
      }
      S.ncand[wave] = run;
      S.bcnt[wave] = 0u;
    }
  }
  __syncthreads();

  // ---- pass 2: candidates (key >= L) in index order. Wave w writes segments w, w + kTileWaves, ... of
  // kTileSeg blocks each, in block order, so it needs no other wave's counts.
  // this lane's queries' workspace rows (valid only where the query scores)
  auto qrow = [&](int j) { return b * a.Tq + tq0 + tile_slot_query(j, half); };
  uint32_t Lk[4];
  bool sel[4], ovf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = tile_slot_query(j, half);
    sel[j] = Q.N[j] > a.k;  // only a query that selects has candidates
    // valid keys are never 0, so key >= max(L, 1) also leaves out the blocks a query does not see; no
    // key of a finite score reaches 0xFFFFFFFF
    Lk[j] = sel[j] ? max(S.Lkey[q], 1u) : 0xFFFFFFFFu;
    ovf[j] = Q.N[j] > 0 && (a.write_keys || (sel[j] && S.ncand[q] > (uint32_t)kCandCap));
  }
  // the combined call selects here (pass 3): the keys of bin L, if they fit, are also gathered into
  // the query's LDS scratch (its histogram's words, free once the thresholds are known)
  const bool sel_here = a.topk != nullptr && a.tile_select != 0;
  bool blst[4];
  uint32_t Lb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = tile_slot_query(j, half);
    blst[j] = sel_here && sel[j] && S.countL[q] <= (uint32_t)kTileBoundCap;
    Lb[j] = S.Lkey[q] >> 20;
  }
  constexpr int kSegTiles = kTileSeg / 32;
  static_assert(kTileSeg % 32 == 0, "a candidate segment is whole tiles");
  const int nseg = (Nmax + kTileSeg - 1) / kTileSeg;
  for (int sg = wave; sg < nseg; sg += kTileWaves) {
    const int t0 = sg * kSegTiles, t1 = min(t0 + kSegTiles, nt);
    uint32_t run[4] = {0u, 0u, 0u, 0u};
    uint4 kb;
    int ks, jc;
    tile_load(codes, scl, t0 * 32 + (lane & 31), Nmax, kb, ks, jc);
    for (int t = t0; t < t1; ++t) {
      const int jb = t * 32 + (lane & 31);
      uint4 kb2 = kb;
      int ks2 = ks, jc2 = jc;
      if (t + 1 < t1) tile_load(codes, scl, jb + 32, Nmax, kb2, ks2, jc2);
      uint32_t key[4];
      tile_keys_at(a, S, Q, codes, kb, ks, t, Nmin, jc, key);
      kb = kb2;
      ks = ks2;
      jc = jc2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool c = key[j] >= Lk[j];
        const uint64_t m = __ballot(c);
        const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
        // candidates of this half before this lane, and in this half
        const uint32_t nlo = (uint32_t)__popc(lo);
        const uint32_t pre = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u)) - (half ? nlo : 0u);
        if (c) {
          const uint64_t e = ((uint64_t)key[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)jb);
          q_cand(a, qrow(j))[(size_t)sg * kTileSeg + run[j] + pre] = e;
          if (blst[j] && (key[j] >> 20) == Lb[j]) {
            const int q = tile_slot_query(j, half);
            const uint32_t at = atomicAdd(&S.bcnt[q], 1u);  // < countL <= kTileBoundCap: pass 1 counted these keys
            if (at < (uint32_t)kTileBoundCap) reinterpret_cast<uint64_t*>(&S.hist[q][0])[at] = e;
          }
        }
        run[j] += half ? (uint32_t)__popc(hi) : nlo;
        if (ovf[j] && jb < Q.N[j]) q_keys(a, qrow(j))[jb] = key[j];
      }
    }
    if ((lane & 31) == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (sel[j]) q_seg(a, qrow(j))[sg] = run[j];
    }
  }
  if (sel_here) {
    __syncthreads();  // every wave's candidates, segment counts and bin-L lists are written
    tile_select(a, S, b, tq0 + wave, wave);
  }
}

// Candidate scan: every key >= L (the bound the query's global histogram gives) is written, in index
// order, to this workgroup's segment of the candidate row; the segment's count goes to seg. A query with
// at most k visible blocks gets its whole list (and its histogram cleared) here.
// APPEND: the launch has one more row of workgroups (blockIdx.y == B*Tq) that writes a decode step's
// window entries and tail copies (the append), one workgroup per sequence, one unit per wave. The
// score kernel before it reads neither the window ring nor the tail, and the attention after it
// needs the new window entries: this launch is a free slot for that work.
template <bool APPEND>
__global__ __launch_bounds__(512) void scan_kernel(ScanArgs args) {
  const ScoreArgs& a = args.a;
  if (APPEND && (int)blockIdx.y == (int)gridDim.y - 1) {
    const int b = blockIdx.x;
    if (b < args.app.B)
      for (int unit = (int)(threadIdx.x >> 6); unit < args.app_units; unit += 8)
        append_unit<true>(args.app, b, unit, threadIdx.x & 63);
    return;
  }
  constexpr int kPer = kScanPerWG / 512;  // keys per thread: j = start + u*512 + tid
  __shared__ uint32_t wsum[8];
  __shared__ uint32_t L_s;
  __shared__ uint32_t cnt_s[kPer * 8];    // candidates per (u, wave), then their exclusive offsets
  __shared__ uint32_t total_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = blockIdx.y;
  const int tq = q % a.Tq;
  if (query_t(a.seq_len, a.seq_T, a.seq_cap, a.len, a.Tq, q / a.Tq, tq) < 0) return;  // ragged: no query in this row
  const int64_t N = visible_blocks(a, q / a.Tq, tq);
  if (N <= a.k) {
    // every visible block is selected; one workgroup writes the list and clears the histogram
    if (blockIdx.x == 0) {
      if (a.topk) {
        int32_t* out = a.topk + (size_t)q * a.k;
        for (int i = tid; i < a.k; i += 512) out[i] = (i < N) ? i : -1;
      }
      for (int i = tid; i < kHistBins; i += 512) q_hist(a, q)[i] = 0u;
    }
    return;
  }
  const int64_t start = (int64_t)blockIdx.x * kScanPerWG;
  if (start >= N) return;
  // this workgroup's keys first (they do not depend on the threshold), then the chunk bounds
  const int64_t end = (start + kScanPerWG < N) ? start + kScanPerWG : N;
  const uint32_t* keys = q_keys(a, q);
  uint32_t kv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t j = start + (int64_t)u * 512 + tid;
    kv[u] = keys[j < end ? j : end - 1];
  }
  // L = the lowest key of the highest bin at which the query's global histogram, counted from the top,
  // reaches k (every winner is >= L; no such bin: L = 0, every block a candidate)
  if (tid == 0) L_s = 0;
  {
    const int top = kHistBins - 8 * tid;
    uint32_t hv[8];
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 1; i <= 8; ++i) {
      hv[i - 1] = q_hist(a, q)[top - i];
      cnt += hv[i - 1];
    }
    uint32_t tot;
    const uint32_t excl = block_excl_scan(cnt, wsum, &tot);
    const uint32_t kk = (uint32_t)a.k;
    if (excl < kk && excl + cnt >= kk) {
      uint32_t c = excl;
      for (int i = 1; i <= 8; ++i) {
        c += hv[i - 1];
        if (c >= kk) {
          L_s = (uint32_t)(top - i) << 20;
          break;
        }
      }
    }
  }
  __syncthreads();
  const uint32_t L = L_s;
  // candidates (key >= L) keep index order: (u, wave, lane) order is ascending j
  uint64_t masks[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t j = start + (int64_t)u * 512 + tid;
    masks[u] = __ballot(j < end && kv[u] >= L);
    if (lane == 0) cnt_s[u * 8 + wave] = (uint32_t)__popcll(masks[u]);
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of the kPer*8 counts in (u, wave) order; two per lane
    uint32_t c0 = cnt_s[2 * lane], c1 = cnt_s[2 * lane + 1];
    const uint32_t incl = wave_incl_scan(c0 + c1);
    uint32_t excl = incl - c0 - c1;
    cnt_s[2 * lane] = excl;
    cnt_s[2 * lane + 1] = excl + c0;
    if (lane == 63) total_s = incl;
  }
  __syncthreads();
  uint64_t* seg = q_cand(a, q) + start;  // this workgroup's segment
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if ((masks[u] >> lane) & 1ull) {
      const uint32_t pos = cnt_s[u * 8 + wave] + (uint32_t)__popcll(masks[u] & lt);
      const uint32_t j = (uint32_t)(start + (int64_t)u * 512 + tid);
      seg[pos] = ((uint64_t)kv[u] << 32) | (uint64_t)(0xFFFFFFFFu - j);
    }
  }
  if (tid == 0) q_seg(a, q)[blockIdx.x] = total_s;
}

// Selection: one workgroup per query gathers the ordered candidates and radix-selects the k largest.
// Every scan workgroup has read the histogram by now, so it is cleared here for the next call.
__global__ __launch_bounds__(512) void select_kernel(ScoreArgs a) {
  __shared__ SelectLds S;
  const int q = blockIdx.x;
  const int b = q / a.Tq, tq = q % a.Tq;
  const int64_t N = visible_blocks(a, b, tq);
  if (N <= a.k) {
    // query tiles leave no scan to write the list of a query that sees at most k blocks
    if (a.tiles && query_t(a.seq_len, a.seq_T, a.seq_cap, a.len, a.Tq, b, tq) >= 0) {
      int32_t* out = a.topk + (size_t)q * a.k;
      for (int i = threadIdx.x; i < a.k; i += 512) out[i] = (i < N) ? i : -1;
    }
    return;
  }
  if (!a.tiles)  // query tiles never count into the global histograms
    for (int i = threadIdx.x; i < kHistBins; i += 512) q_hist(a, q)[i] = 0u;
  int32_t* out = a.topk + (size_t)q * a.k;
  const uint32_t n = select_query(a, q, N, S, out);
  for (int i = (int)n + (int)threadIdx.x; i < a.k; i += 512) out[i] = -1;  // only if fewer than k were found
}

}  // namespace

hipError_t launch_index_score(const ScoreArgs& a, int32_t B, hipStream_t s) {
  const int64_t N_last = a.len / a.m;  // visible blocks of the last query (t = len-1)
  if (N_last <= a.k) return hipSuccess;  // every visible block is selected; no scores needed
  const unsigned nq = (unsigned)(B * a.Tq);
  // a workgroup per chunk, or (many queries) chunk_step workgroups per query, each over every
  // chunk_step-th chunk
  if (a.tiles) {
    const unsigned gx = (unsigned)((a.Tq + kTileQueries - 1) / kTileQueries);
    hipLaunchKernelGGL(tile_kernel, dim3(gx, (unsigned)B), dim3(kTileWaves * 64), 0, s, a);
    return hipGetLastError();
  }
  unsigned g1 = a.chunk_step > 0 ? (unsigned)a.chunk_step : (unsigned)((N_last + kScoreChunk - 1) / kScoreChunk);
  if (a.fold_tail && a.chunk_step == 0 && g1 >= 2) g1 -= 1;  // workgroup 0 scores the last chunk
  hipLaunchKernelGGL(score_kernel, dim3(g1, nq), dim3(kScoreThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_index_select(const ScanArgs& args, int32_t B, hipStream_t s) {
  const unsigned nq = (unsigned)(B * args.a.Tq);
  const unsigned cols = (unsigned)(args.a.n_cols > 0 ? args.a.n_cols : 1);
  const bool app = args.app_units > 0;
  const unsigned gx = app && (unsigned)B > cols ? (unsigned)B : cols;
  // record words per thread of the last workgroup: the most any query of the call has
  const int64_t words = (int64_t)(cols + (args.a.fold_tail ? 1 : 0)) * args.a.pref_slots;
  if (words <= 9 * kScoreThreads)
    hipLaunchKernelGGL(index_select_kernel<9>, dim3(gx, nq + (app ? 1u : 0u)), dim3(kScoreThreads), 0, s, args);
  else if (words <= kPrefMaxLoads * kScoreThreads)
    hipLaunchKernelGGL(index_select_kernel<kPrefMaxLoads>, dim3(gx, nq + (app ? 1u : 0u)), dim3(kScoreThreads), 0,
                       s, args);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_csa_step(const StepArgs& sa, hipStream_t s) {
  const unsigned grid = (unsigned)(sa.n_idx + sa.n_att);
  const int64_t words = (int64_t)(sa.idx.a.n_cols + (sa.idx.a.fold_tail ? 1 : 0)) * sa.idx.a.pref_slots;
  if (words <= 9 * kScoreThreads)
    hipLaunchKernelGGL(csa_step_kernel<9>, dim3(grid), dim3(kScoreThreads), 0, s, sa);
  else if (words <= kPrefMaxLoads * kScoreThreads)
    hipLaunchKernelGGL(csa_step_kernel<kPrefMaxLoads>, dim3(grid), dim3(kScoreThreads), 0, s, sa);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_topk_select(const ScoreArgs& a, int32_t B, hipStream_t s, bool with_select,
                              const IngestArgs* app, int32_t app_units) {
  const int64_t N_last = a.len / a.m;
  const unsigned nq = (unsigned)(B * a.Tq);
  unsigned g2 = (unsigned)((N_last + kScanPerWG - 1) / kScanPerWG);
  if (g2 < 1) g2 = 1;
  ScanArgs args{};
  args.a = a;
  if (a.tiles) {
    // the score launch wrote the candidates (and, for the combined call, the lists); a decode step's
    // append never comes with query tiles
    if (app && app_units > 0) return hipErrorInvalidValue;
    if (with_select && !a.tile_select) hipLaunchKernelGGL(select_kernel, dim3(nq), dim3(512), 0, s, a);
    return hipGetLastError();
  }
  if (app && app_units > 0) {
    args.app = *app;
    args.app_units = app_units;
    const unsigned gx = g2 > (unsigned)B ? g2 : (unsigned)B;
    hipLaunchKernelGGL(scan_kernel<true>, dim3(gx, nq + 1), dim3(512), 0, s, args);
  } else {
    hipLaunchKernelGGL(scan_kernel<false>, dim3(g2, nq), dim3(512), 0, s, args);
  }
  if (with_select) hipLaunchKernelGGL(select_kernel, dim3(nq), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace lca
