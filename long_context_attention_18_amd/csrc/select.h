// select.h -- exact top-k selection of one query from its ordered candidates (gfx950, 512 threads).
//
// The CSA paragraph of "DeepSeek-V4: a million-token context that agents can
// actually use": each query keeps the k compressed blocks its indexer scores
// highest. Ties go to the lower block index, so the order is the 64-bit key
// (score_key << 32 | ~j), which is unique per block.
//
// Input: the candidates the scan left in index order, one segment per scan
// workgroup (every key >= a lower bound of the k-th key), or, when there are
// more than fit in LDS, every visible block's key. Radix select finds the
// k-th largest 64-bit key, 11 bits at a time from the highest bit in which the
// elements differ, until the bin that holds it is taken whole or holds at most
// 64 elements, which one wave then ranks directly; an order-preserving
// compaction writes the winners in ascending block index to `out` (global or
// LDS), without a sort.
#pragma once
#include "kernels.h"

namespace lca {

constexpr int kRadixBits = 11;  // digit width of the radix select: 2048 LDS bins
constexpr int kRadixBins = 1 << kRadixBits;

struct SelectLds {
  uint64_t cs[kCandCap];
  uint32_t seg_off[kMaxSegs + 1];  // G2_q <= kMaxSegs segments
  uint32_t hist[kRadixBins];
  uint32_t wsum[8];
  uint32_t sel_digit, sel_above, sel_count, flat_needed;
  uint64_t red_lo[8], red_hi[8];
  uint64_t small[64];  // a boundary bin of at most 64 elements, ranked directly
  uint32_t small_n;
  uint64_t sel_thresh;
};

// One step of an inclusive prefix min (lo) / max (hi) of 64-bit values over the wave, through DPP on the
// two 32-bit halves; lanes the move does not reach keep the neutral value (all ones for min, 0 for max)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void minmax_step(uint64_t& lo, uint64_t& hi) {
  const uint32_t l0 = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)lo, CTRL, ROW_MASK, 0xf, false);
  const uint32_t l1 = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)(lo >> 32), CTRL, ROW_MASK, 0xf, false);
  const uint32_t h0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)hi, CTRL, ROW_MASK, 0xf, false);
  const uint32_t h1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(hi >> 32), CTRL, ROW_MASK, 0xf, false);
  const uint64_t ol = ((uint64_t)l1 << 32) | l0, oh = ((uint64_t)h1 << 32) | h0;
  lo = ol < lo ? ol : lo;
  hi = oh > hi ? oh : hi;
}

// the wave's minimum and maximum end in lane 63 (the steps of wave_incl_scan)
__device__ __forceinline__ void wave_minmax_u64(uint64_t& lo, uint64_t& hi) {
  minmax_step<0x111, 0xf>(lo, hi);  // row_shr:1
  minmax_step<0x112, 0xf>(lo, hi);  // row_shr:2
  minmax_step<0x114, 0xf>(lo, hi);  // row_shr:4
  minmax_step<0x118, 0xf>(lo, hi);  // row_shr:8
  minmax_step<0x142, 0xa>(lo, hi);  // row_bcast:15 -> rows 1, 3
  minmax_step<0x143, 0xc>(lo, hi);  // row_bcast:31 -> rows 2, 3
}

// exclusive prefix sum over the 512 threads of the workgroup (thread order); every thread calls it
__device__ __forceinline__ uint32_t excl_scan_512(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {  // all 8 read at once (a loop to `wave` would wait for each read in turn)
    const uint32_t x = wsum[w];
    off += w < wave ? x : 0u;
  }
  return off + incl - v;
}

// The k-th largest of n elements (elem(i): the i-th; lo / hi: this thread's smallest and largest of the
// ones it read) by radix select: on return the winners are exactly the elements e with (e & mask) >=
// prefix. S.hist must be zero, S.small_n zero and S.small[] zero on entry (left zero again). Every thread
// calls it.
template <class Elem>
__device__ inline void radix_bound(SelectLds& S, int64_t n, uint64_t lo, uint64_t hi, Elem elem, uint32_t k,
                                   uint64_t* prefix_out, uint64_t* mask_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* hist = S.hist;
  uint32_t* wsum = S.wsum;
  wave_minmax_u64(lo, hi);
  if (lane == 63) {
    S.red_lo[wave] = lo;
    S.red_hi[wave] = hi;
  }
  __syncthreads();

  // every element a winner (n == k): no selection
  uint64_t prefix = 0, mask = 0;
  if (n > (int64_t)k) {
    uint64_t glo = S.red_lo[0], ghi = S.red_hi[0];
    for (int w = 1; w < 8; ++w) {
      glo = S.red_lo[w] < glo ? S.red_lo[w] : glo;
      ghi = S.red_hi[w] > ghi ? S.red_hi[w] : ghi;
    }
    // radix select of the k-th largest 64-bit key (score key, then lower index first), kRadixBits at a
    // time from the highest bit in which the elements differ (keys are unique and n > k >= 1, so some
    // bit differs), stopping as soon as the bin that holds it is taken whole
    const int hb = 63 - __clzll((long long)(glo ^ ghi));
    const uint64_t common = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
    prefix = glo & common;
    mask = common;
    uint32_t need = k;
    for (int shift = hb - (kRadixBits - 1); shift > -kRadixBits; shift -= kRadixBits) {
      const int sh = shift < 0 ? 0 : shift;  // the last digit may be narrower
      const uint64_t dmask = shift < 0 ? ((1ull << (shift + kRadixBits)) - 1ull) : (uint64_t)(kRadixBins - 1);
      for (int64_t i = tid; i < n; i += 512) {
        const uint64_t e = elem(i);
        if ((e & mask) == prefix) atomicAdd(&hist[(uint32_t)((e >> sh) & dmask)], 1u);
      }
      __syncthreads();
      // counts from the top: thread t holds bins 2047-4t .. 2044-4t
      uint32_t h4[4], c4 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h4[j] = hist[kRadixBins - 1 - 4 * tid - j];
        hist[kRadixBins - 1 - 4 * tid - j] = 0u;  // cleared for the next pass (its adds follow two barriers)
        c4 += h4[j];
      }
      const uint32_t excl = excl_scan_512(c4, wsum);
      if (excl < need && excl + c4 >= need) {
        uint32_t c = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (c + h4[j] >= need) {
            S.sel_digit = (uint32_t)(kRadixBins - 1 - 4 * tid - j);
            S.sel_above = c;
            S.sel_count = h4[j];
            break;
          }
          c += h4[j];
        }
      }
      __syncthreads();
      const uint32_t d = S.sel_digit;
      need -= S.sel_above;
      prefix |= (uint64_t)d << sh;
      mask |= dmask << sh;
      if (S.sel_count == need) break;
      if (S.sel_count <= 64) {
        // a small boundary bin: gather its elements and find the need-th largest by direct ranking
        // (keys are unique, so exactly one element has need-1 larger ones) instead of another pass
        for (int64_t i = tid; i < n; i += 512) {
          const uint64_t e = elem(i);
          if ((e & mask) == prefix) S.small[atomicAdd(&S.small_n, 1u)] = e;
        }
        __syncthreads();
        if (wave == 0) {
          // all 64 slots, unrolled: the LDS reads go out together instead of one round trip per element
          const uint32_t c = S.sel_count;
          const uint64_t mine = S.small[lane];
          uint32_t rank = 0;
#pragma unroll
          for (int m = 0; m < 64; ++m) rank += S.small[m] > mine ? 1u : 0u;
          if (lane < (int)c && rank == need - 1) S.sel_thresh = mine;
        }
        __syncthreads();
        prefix = S.sel_thresh;  // the winners are exactly the elements >= the need-th largest of the bin
        mask = ~0ull;
        break;
      }
    }
  }
  *prefix_out = prefix;
  *mask_out = mask;
}

// The selection proper, over n elements in index order (elem(i): the i-th; lo / hi: this thread's
// smallest and largest of the ones it read): radix select of the k-th largest, then the winners in index
// order to out (and out2). Returns the number of winners written (min(k, n)). Every thread calls it.
// kAgentOut: out is written with agent-scope stores (a list that workgroups on other XCDs read in the same
// launch).
template <bool kAgentOut = false, class Elem>
__device__ inline uint32_t select_core(const ScoreArgs& a, SelectLds& S, int64_t n, uint64_t lo, uint64_t hi,
                                       Elem elem, int32_t* out, int32_t* out2) {
  const int tid = threadIdx.x;
  uint32_t* wsum = S.wsum;
  uint64_t prefix, mask;
  radix_bound(S, n, lo, hi, elem, (uint32_t)a.k, &prefix, &mask);
  // winners (determined bits >= prefix), written in index order: each thread owns a contiguous run
  const int64_t per = (n + 511) / 512;
  const int64_t i0 = (int64_t)tid * per;
  const int64_t i1 = (i0 + per < n) ? i0 + per : n;
  uint32_t mine = 0;
  for (int64_t i = i0; i < i1; ++i) mine += ((elem(i) & mask) >= prefix) ? 1u : 0u;
  uint32_t pos = excl_scan_512(mine, wsum);
  uint32_t n_win = 0;
  for (int w = 0; w < 8; ++w) n_win += wsum[w];
  for (int64_t i = i0; i < i1; ++i) {
    const uint64_t e = elem(i);
    if ((e & mask) >= prefix) {
      if (pos < (uint32_t)a.k) {
        const int32_t j = (int32_t)(0xFFFFFFFFu - (uint32_t)(e & 0xFFFFFFFFu));
        if constexpr (kAgentOut) __hip_atomic_store(&out[pos], j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else out[pos] = j;
        if (out2) out2[pos] = j;
      }
      ++pos;
    }
  }
  return n_win < (uint32_t)a.k ? n_win : (uint32_t)a.k;
}

// Returns the number of winners written (min(k, N) whenever N > k). The candidate lower bound is only
// a hint: with fewer than k candidates (a histogram left dirty by a score call without its selection)
// or more than fit in LDS, the selection takes the path over every visible block and stays exact.
// Winners go to out (and out2 when not null) in ascending block order.
__device__ inline uint32_t select_query(const ScoreArgs& a, int q, int64_t N, SelectLds& S, int32_t* out,
                                        int32_t* out2 = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t* cs = S.cs;
  uint32_t* seg_off = S.seg_off;
  uint32_t* hist = S.hist;
  uint32_t* wsum = S.wsum;

  // One round of loads: every segment's count and, speculatively, its first `covered` slots (always in
  // bounds: a segment has room for seg_sz candidates, and the workspace continues after the last
  // query's); only a fuller segment needs a second round. Segments: kScanPerWG blocks (candidate scan)
  // or kTileSeg (query tiles).
  const int seg_sz = a.tiles ? kTileSeg : kScanPerWG;
  const int G2_q = (int)((N + seg_sz - 1) / seg_sz);
  constexpr int kSpecPerLane = 16;  // speculative loads per thread
  const uint64_t* cand = q_cand(a, q);
  const int lanes_per_seg = G2_q <= 32 ? 16 : (G2_q <= 64 ? 8 : 0);  // speculation only for few segments
  // slots per segment the speculative loads place: the first 256 (16 threads per segment) or 128 (8)
  const uint32_t covered = (uint32_t)(lanes_per_seg * kSpecPerLane);
  uint64_t spec[kSpecPerLane];
  const int my_seg = lanes_per_seg ? tid / lanes_per_seg : 0;
  const int my_sub = lanes_per_seg ? tid % lanes_per_seg : 0;
  const int per_lane = lanes_per_seg ? kSpecPerLane : 0;
  if (lanes_per_seg && my_seg < G2_q) {
#pragma unroll
    for (int r = 0; r < kSpecPerLane; ++r)
      if (r < per_lane) spec[r] = cand[(size_t)my_seg * seg_sz + my_sub + r * lanes_per_seg];
  }
  if (tid == 0) S.flat_needed = 0u;
  // the first radix pass's bins and the small-bin state, cleared now (the barriers below order them)
  for (int i = tid; i < kRadixBins; i += 512) hist[i] = 0u;
  if (tid == 0) S.small_n = 0u;
  if (tid < 64) S.small[tid] = 0ull;  // unused slots rank below every element
  if (G2_q <= 64) {
    // one wave holds every segment count: its scan needs no workgroup barrier before the offsets
    if (wave == 0) {
      const uint32_t c = lane < G2_q ? q_seg(a, q)[lane] : 0u;
      const uint32_t incl = wave_incl_scan(c);
      if (lane < G2_q) seg_off[lane] = incl - c;
      if (lane == 63) seg_off[G2_q] = incl;
      if (c > covered) S.flat_needed = 1u;
    }
    __syncthreads();
  }
  for (int g0 = 0; G2_q > 64 && g0 < G2_q; g0 += 512) {
    const int gi = g0 + tid;
    const uint32_t c = gi < G2_q ? q_seg(a, q)[gi] : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t base = g0 == 0 ? 0u : seg_off[g0];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t x = wsum[w];
      base += w < wave ? x : 0u;
    }
    if (gi < G2_q) seg_off[gi] = base + incl - c;
    if (tid == 511) seg_off[g0 + 512 < G2_q ? g0 + 512 : G2_q] = base + incl;
    if (c > covered) S.flat_needed = 1u;
    __syncthreads();
  }
  const uint32_t total = seg_off[G2_q];
  const bool fast = total >= (uint32_t)a.k && total <= (uint32_t)kCandCap;
  const int64_t n = fast ? (int64_t)total : N;
  const uint32_t* keys = q_keys(a, q);
  // element i in index order: the ordered candidates, or (slow path) every visible block
  auto elem = [&](int64_t i) -> uint64_t {
    if (fast) return cs[i];
    return ((uint64_t)keys[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
  };
  // gather into LDS (fast path), keeping each thread's smallest and largest element
  uint64_t lo = ~0ull, hi = 0;
  if (fast) {
    if (lanes_per_seg && my_seg < G2_q) {
      const uint32_t c = seg_off[my_seg + 1] - seg_off[my_seg];
#pragma unroll
      for (int r = 0; r < kSpecPerLane; ++r) {
        const uint32_t i = my_sub + r * lanes_per_seg;
        if (r < per_lane && i < c) {
          cs[seg_off[my_seg] + i] = spec[r];
          lo = spec[r] < lo ? spec[r] : lo;
          hi = spec[r] > hi ? spec[r] : hi;
        }
      }
    }
    if (S.flat_needed) {
      // segments longer than the speculated slots: flat gather, segment found by binary search
      for (uint32_t i = tid; i < total; i += 512) {
        int l = 0, h = G2_q - 1;
        while (l < h) {
          const int mid = (l + h + 1) >> 1;
          if (seg_off[mid] <= i) l = mid;
          else h = mid - 1;
        }
        const uint32_t off = i - seg_off[l];
        if (off >= covered) {
          const uint64_t e = cand[(size_t)l * seg_sz + off];
          cs[i] = e;
          lo = e < lo ? e : lo;
          hi = e > hi ? e : hi;
        }
      }
    }
  } else {
    for (int64_t i = tid; i < n; i += 512) {
      const uint64_t e = elem(i);
      lo = e < lo ? e : lo;
      hi = e > hi ? e : hi;
    }
  }
  return select_core(a, S, n, lo, hi, elem, out, out2);
}

}  // namespace lca
