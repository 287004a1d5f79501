// attend.hip -- one-launch attention for a few queries (decode), for gfx950.
//
// Figure 3 of "DeepSeek-V4: a million-token context that agents can actually
// use" (CSA: the selected compressed blocks plus a sliding-window branch) and
// Figure 4 / the HCA paragraph (every compressed block plus the window), with
// one softmax over all of a query's keys:
//   logit = RoPE(q_h, t) . x / sqrt(128),  K = V = the dequantised entry.
//
// A workgroup owns one query, 16 of its heads and a share of its keys (all
// of them, or one of up to 4 key splits when the call has few queries): its
// 8 waves take contiguous ranges of 32-key chunks, each keeps an online
// softmax for the 16 heads, and the 8 wave states are merged in LDS. With
// splits, each workgroup writes a partial and the last of a (query, group)
// to finish merges them, in the same launch. With few queries the
// step is latency-bound, and this keeps it to one launch. Each wave takes a
// contiguous range of the key slots and issues the gathers of up to kRound
// chunks at once (random reads: one memory latency per round).
//
// Modes: LIST (the caller's top-k list), LIST_WS (the list the indexer's
// in-launch selection left in the workspace: the decode step's path), DENSE
// (HCA: every visible block) and SELECT (CSA after a separate score call: the
// workgroup first runs the exact top-k selection of its query from the scan's
// candidates, select.h, into LDS, then attends over the result).
//
// Key slots: the window first, then the compressed entries (the softmax does
// not depend on the order).
//
// MFMA layout (v_mfma_f32_16x16x32_bf16; lane l = 16 g + r):
//   S^T = K . Q^T   A = 16 keys x 32 dims, straight from the gathered entry
//                   (lane: key r, dims 8g..8g+7 of the K-step); B = Q^T
//                   (lane: head r, same dims); out lane: head r, keys 4g+v.
//   O^T = V^T . P^T A = V^T (lane: dim r of the tile, 8 keys), read from the
//                   wave's key-major LDS copy of the chunk by gfx950's
//                   transposing LDS read (ds_read_b64_tr_b16: lane 4a + e of
//                   a 16-lane group gets element e of the 8-byte rows lanes a,
//                   a+4, a+8, a+12 address; each lane addresses the key its K
//                   index needs); B = P^T (lane: head r, keys 8g..8g+7).
// Within a 32-key chunk, MFMA K index 8g + 2v + tt is key 4g+v of 16-key tile
// tt, so each lane's B operand for P^T is exactly the 8 logits it holds. The
// FP8 codes and BF16 RoPE dims are exact in bf16; the fp32 scale multiplies
// the nope logits and is folded into P for the nope output dims.
#include "attn_common.h"
#include "dev_formats.h"
#include "ingest.h"
#include "kernels.h"
#include "select.h"
#include "attend_core.h"

namespace lca {

namespace {

constexpr int kRound = 4;      // chunks a wave gathers at once (VGPR budget: five spill)

struct AttendLds {
  union {
    SelectLds sel;  // selection
    AttnWaveLds w;  // the keys, then the wave merge
  } u;
  int32_t list[kMaxTopk];  // compressed entries to attend (block indices)
  int last;                // this workgroup merges the splits
  float cos_t[32], sin_t[32];
};

template <int MODE>
__global__ __launch_bounds__(512) void attend_kernel(AttendArgs args) {
  __shared__ AttendLds S;
  const AttnArgs& a = args.t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int hgs = (a.H + 15) / 16;
  // XCD-aware placement: the launch's workgroups go round-robin over the 8 XCDs in linear id order, and
  // the head groups of one (query, split) gather the same key rows, so they take consecutive logical
  // indices inside one XCD's share (its L2 then serves the rows once instead of once per group)
  int hg, split, q;
  {
    const unsigned total = gridDim.x * gridDim.y;
    const unsigned lin = blockIdx.x + gridDim.x * blockIdx.y;
    const unsigned xcd = lin % 8u, pos = lin / 8u;
    const unsigned logical = xcd * (total / 8u) + min(xcd, total % 8u) + pos;
    const unsigned per_q = gridDim.x;  // hgs x splits
    q = (int)(logical / per_q);
    hg = (int)(logical % per_q) % hgs;
    split = (int)(logical % per_q) / hgs;
  }
  const int b = q / a.Tq, tq = q % a.Tq;
  const int64_t t = query_t(a.seq_len, a.seq_T, a.seq_cap, a.len, a.Tq, b, tq);
  if (args.adv_len) {
    // lengths on the device: every workgroup counts itself in once each of its waves holds its length (the
    // load complete), and the last one advances every sequence's length for the next step
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (wave == 0) {
      uint32_t old = 0;
      if (lane == 0)
        old = __hip_atomic_fetch_add(args.adv_cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = (uint32_t)__builtin_amdgcn_readfirstlane((int)old);
      if (old == gridDim.x * gridDim.y - 1u) {
        if (lane == 0) __hip_atomic_store(args.adv_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int nb = (int)(gridDim.y / (unsigned)a.Tq);
        for (int bb = lane; bb < nb; bb += 64)
          args.adv_len[bb] = a.seq_len[bb] + ragged_T(a.seq_len, a.seq_T, a.seq_cap, bb);
      }
    }
  }
  if (t < 0) return;  // ragged batch: no query in this row
  // visible blocks; max_blocks bounds them (0 for the window-only layer, which has no compressed stream)
  const int64_t N = min((t + 1) / a.m, a.max_blocks);
  const bool do_select = MODE == kAttendSelect && N > a.k;

  Keys K;
  K.win_codes = a.win_codes;
  K.blk_codes = a.blk_codes;
  K.win_rope = a.win_rope;
  K.blk_rope = a.blk_rope;
  K.win_scale = a.win_scale;
  K.blk_scale = a.blk_scale;
  K.ring = (uint32_t)a.ring;
  K.list = S.list;
  K.list0 = 0;
  K.win_row = (size_t)b * a.ring;
  K.blk_row = (size_t)b * a.max_blocks;
  K.n_win = (int)((int64_t)a.W < t + 1 ? (int64_t)a.W : t + 1);
  K.win_base = (uint32_t)((t - K.n_win + 1) % a.ring);
  K.j_max = N > 0 ? N - 1 : 0;
  if (MODE == kAttendDense) {
    K.n_list = (int)N;
    K.use_list = false;
  } else if (MODE == kAttendList) {
    K.n_list = a.k;
    K.use_list = true;
  } else if (MODE == kAttendListWs) {
    // the in-launch selection's list (k winners when N > k); a query that sees at most k blocks takes them all
    K.use_list = N > a.k;
    K.n_list = (int)(N > a.k ? (int64_t)a.k : N);
  } else {
    K.n_list = (int)(N < a.k ? N : (int64_t)a.k);
    K.use_list = do_select;
  }
  // RoPE angles of position t: reduced to [-pi, pi] in fp64 (2 pi as a double plus its remainder),
  // then fp32 sin / cos; the rotated query is rounded to bf16, far coarser than either step
  if (tid < 32) {
    float sn, cs;
    rope_angle(t, a.inv_freq[tid], &sn, &cs);
    S.cos_t[tid] = cs;
    S.sin_t[tid] = sn;
  }
  // query rows (head hg*16 + r, dims 32 ks + 8 g ..), loaded now, rotated after the barrier
  const int head = hg * 16 + r;
  const bool head_ok = head < a.H;
  u32x4 qraw[4];
  {
    const uint16_t* qp = a.q + (((size_t)b * a.Tq + tq) * a.H + (head_ok ? head : 0)) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qraw[ks] = head_ok ? *reinterpret_cast<const u32x4*>(qp + ks * 32 + 8 * g) : (u32x4){0u, 0u, 0u, 0u};
  }
  if (MODE == kAttendList) {
    // the caller's list, valid entries (0 <= j < N) only, in order
    const int32_t* lp = a.topk + ((size_t)b * a.Tq + tq) * a.k;
    uint32_t* wsum = S.u.sel.wsum;
    int n = 0;
    for (int base = 0; base < a.k; base += 512) {
      const int i = base + tid;
      const int32_t j = i < a.k ? lp[i] : -1;
      const bool ok = j >= 0 && (int64_t)j < N;
      const uint64_t m = __ballot(ok);
      if (lane == 0) wsum[wave] = (uint32_t)__popcll(m);
      __syncthreads();
      int pos = n + (int)__popcll(m & ((1ull << lane) - 1ull));
      int tot = 0;
      for (int w = 0; w < kWaves; ++w) {
        const int c = (int)wsum[w];
        if (w < wave) pos += c;
        tot += c;
      }
      if (ok) S.list[pos] = j;
      n += tot;
      __syncthreads();
    }
    K.n_list = n;
  }
  if (MODE == kAttendListWs && K.use_list) {
    const int32_t* lp = q_list(args.s, q);
    for (int i = tid; i < a.k; i += 512) S.list[i] = lp[i];
  }
  if (do_select) {
    const ScoreArgs& sa = args.s;
    if (hg == 0 && split == 0)  // every scan workgroup has read this query's histogram: clear it for the next call
      for (int i = tid; i < kHistBins; i += 512) q_hist(sa, q)[i] = 0u;
    K.n_list = (int)select_query(sa, q, N, S.u.sel, S.list);
  }
  // this workgroup: key slots [s_begin, s_end) of its split (the window's slots first)
  const int n_keys = K.n_win + K.n_list;
  const int splits = args.splits;
  const int per_split = ((n_keys + splits * 16 - 1) / (splits * 16)) * 16;
  const int s_begin = split * per_split;
  const int s_end = min(s_begin + per_split, n_keys);
  if (MODE == kAttendDense && args.app_units > 0) {
    // The step's append, in this launch: the window entries of the new tokens, which the newest window
    // slots read. Every workgroup whose slot range reaches into the window writes all of its sequence's
    // new entries (the same bytes from each; a ring slot holds nothing else any query of the call
    // reads) and reads them back after the fence and barrier below, so no workgroup depends on
    // another's writes. The tail copies go to head group 0 of split 0 (nothing here reads the tail).
    // One wave per unit.
    const bool reads_window = s_begin < K.n_win;
    const bool writes_tail = hg == 0 && split == 0;
    for (int unit = wave; unit < args.app_units; unit += kWaves)
      if (unit < args.app.n_win ? reads_window : writes_tail) append_unit<false>(args.app, b, unit, lane);
    __threadfence_block();
  }
  __syncthreads();
  if (do_select && hg == 0 && split == 0 && args.s.topk) {
    int32_t* o = args.s.topk + (size_t)q * a.k;
    for (int i = tid; i < a.k; i += 512) o[i] = S.list[i];
  }
  if (MODE == kAttendSelect && !do_select && args.s.tiles && hg == 0 && split == 0 && args.s.topk) {
    // query tiles leave no scan to write the list of a query that sees at most k blocks
    int32_t* o = args.s.topk + (size_t)q * a.k;
    for (int i = tid; i < a.k; i += 512) o[i] = (int64_t)i < N ? i : -1;
  }

  bf16x8 qb[4];
  rotate_query(qraw, S.cos_t, S.sin_t, g, qb);
  float m_run = -INFINITY, l_run = 0.0f;
  v4f O[8];
  attend_slots<kRound>(K, s_begin, s_end, per_split, qb, S.u.w, wave, r, g, m_run, l_run, O);
  attend_finish(args, S.u.w, &S.last, q, hg, split, m_run, l_run, O);
}

}  // namespace

hipError_t launch_attend(const AttendArgs& args, int32_t B, int mode, hipStream_t s) {
  const unsigned nq = (unsigned)(B * args.t.Tq);
  const unsigned gx = (unsigned)((args.t.H + 15) / 16 * args.splits);
  if (mode == kAttendSelect) hipLaunchKernelGGL(attend_kernel<kAttendSelect>, dim3(gx, nq), dim3(512), 0, s, args);
  else if (mode == kAttendListWs) hipLaunchKernelGGL(attend_kernel<kAttendListWs>, dim3(gx, nq), dim3(512), 0, s, args);
  else if (mode == kAttendDense) hipLaunchKernelGGL(attend_kernel<kAttendDense>, dim3(gx, nq), dim3(512), 0, s, args);
  else hipLaunchKernelGGL(attend_kernel<kAttendList>, dim3(gx, nq), dim3(512), 0, s, args);
  return hipGetLastError();
}

}  // namespace lca
