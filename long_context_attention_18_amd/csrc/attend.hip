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

namespace lca {

namespace {

constexpr int kWaves = 8;
constexpr int kChunk = 32;     // keys per wave step: two 16-key tiles
constexpr int kKdStride = 136;  // bf16 per key-major LDS row (128 dims + 8 pad)
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
constexpr int kRound = 4;      // chunks a wave gathers at once (VGPR budget: five spill)

struct AttendLds {
  union {
    SelectLds sel;  // selection
    struct {
      uint16_t kd[kWaves][kChunk * kKdStride];    // per-wave key-major copy of its current chunk
      float scl[kWaves][2][16];                   // per-wave key scales of the chunk's two tiles
    } b;
    struct {
      float o[kWaves][16][kHeadDim + 4];  // row stride 132 floats: conflict-free 16-B accesses
      float m[kWaves][16], l[kWaves][16];
    } c;
  } u;
  int32_t list[kMaxTopk];  // compressed entries to attend (block indices)
  int last;                // this workgroup merges the splits
  float cos_t[32], sin_t[32];
};

// One 32-key chunk's raw gathered data, as lane (r, g) holds it: key r of tiles 0 and 1.
struct Raw {
  u32x2 c0[2], c1[2];  // FP8 codes, dims 8g..8g+7 and 32+8g..32+8g+7
  u32x4 r0[2], r1[2];  // BF16 RoPE dims 64+8g.. and 96+8g..
  float sc[2];
};

struct Keys {
  // base arrays and sizes held by value: read through a pointer to the kernel arguments they become
  // vector loads that every gather would wait for
  const uint8_t *win_codes, *blk_codes;
  const uint16_t *win_rope, *blk_rope;
  const float *win_scale, *blk_scale;
  uint32_t ring;
  const int32_t* list;
  size_t win_row, blk_row;  // b * ring, b * max_blocks
  uint32_t win_base;        // ring slot of the first window position
  int64_t j_max;            // last visible block (0 when none)
  int n_win, n_list;
  bool use_list;
  // Entry of key slot `slot` (< n_win + n_list): window position t - n_win + 1 + slot, or the
  // compressed block list[slot - n_win] (dense: slot - n_win). Branch-free, so the loads that
  // follow stay in straight-line code and the compiler can wait for them one chunk at a time.
  __device__ __forceinline__ size_t entry(int slot, bool* in_win) const {
    *in_win = slot < n_win;
    const int li = *in_win ? 0 : slot - n_win;
    int64_t j = use_list ? (int64_t)list[li] : (int64_t)li;
    j = j < 0 ? 0 : (j > j_max ? j_max : j);  // list entries are valid by construction; never read outside
    uint32_t ws = win_base + (uint32_t)slot;
    ws = ws >= ring ? ws - ring : ws;
    return *in_win ? win_row + ws : blk_row + (size_t)j;
  }
  // lane (r, g): key r of the chunk's two tiles; slots at or beyond `end` read slot 0 (masked later)
  __device__ __forceinline__ void load(int chunk_slot, int end, int r, int g, Raw& R) const {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      int slot = chunk_slot + tt * 16 + r;
      slot = slot < end ? slot : 0;
      bool w;
      const size_t e = entry(slot, &w);
      const uint8_t* codes = (w ? win_codes : blk_codes) + e * kNope;
      const uint16_t* rope = (w ? win_rope : blk_rope) + e * kRope;
      const float* scl = (w ? win_scale : blk_scale) + e;
      R.c0[tt] = ldg<u32x2>(codes + 8 * g);
      R.c1[tt] = ldg<u32x2>(codes + 32 + 8 * g);
      R.r0[tt] = ldg<u32x4>(rope + 8 * g);
      R.r1[tt] = ldg<u32x4>(rope + 32 + 8 * g);
      R.sc[tt] = ldg<float>(scl);
    }
  }
};

// One 32-key chunk of one wave: S^T = K . Q^T for the two 16-key tiles, the online softmax of head r,
// the keys into the wave's LDS buffer, O^T += V^T . P^T. Lane (r, g): head r; keys 4g+v of each tile.
// Logits stay unscaled (S = q.x); the 1/sqrt(128) and log2(e) factors go into one multiply before
// exp2. The running max m is raised only when a chunk's max exceeds it by more than kLazy (log2
// units), and only then is O rescaled (once per wave, for the heads that moved): the softmax does
// not depend on the reference point, and P stays below 2^kLazy. Slots at or beyond `end` are empty.
__device__ __forceinline__ void attend_chunk(const Raw& cur, int chunk_slot, int end, const bf16x8 (&qb)[4], float* scl,
                                             uint16_t* kd, const int (&voff)[2], int r, int g, float& m_run,
                                             float& l_run, v4f (&O)[8]) {
  constexpr float kC = kLog2eRsqrtD;
  constexpr float kLazy = 8.0f;
  u32x4 kn0[2], kn1[2];
  float Sv[2][4];
  v4f sc4[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    kn0[tt] = fp8x8_to_bf16(cur.c0[tt]);
    kn1[tt] = fp8x8_to_bf16(cur.c1[tt]);
    v4f an = {0.0f, 0.0f, 0.0f, 0.0f}, ar = {0.0f, 0.0f, 0.0f, 0.0f};
    an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kn0[tt]), qb[0], an, 0, 0, 0);
    an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kn1[tt]), qb[1], an, 0, 0, 0);
    ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.r0[tt]), qb[2], ar, 0, 0, 0);
    ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.r1[tt]), qb[3], ar, 0, 0, 0);
    if (g == 0) scl[tt * 16 + r] = cur.sc[tt];
    sc4[tt] = *reinterpret_cast<const v4f*>(scl + tt * 16 + 4 * g);
    const int slot0 = chunk_slot + tt * 16 + 4 * g;
#pragma unroll
    for (int v = 0; v < 4; ++v) Sv[tt][v] = (slot0 + v < end) ? an[v] * sc4[tt][v] + ar[v] : -INFINITY;
  }
  // online softmax of head r (its keys are spread over the 4 lane groups)
  float mx = max3_raw(max3_raw(Sv[0][0], Sv[0][1], Sv[0][2]), max3_raw(Sv[0][3], Sv[1][0], Sv[1][1]),
                      max_raw(Sv[1][2], Sv[1][3]));
  mx = pair_max32(pair_max16(mx));
  const bool raise = mx * kC > m_run * kC + kLazy;  // also true for the first finite max (m_run = -inf)
  if (__builtin_amdgcn_read_exec() & __ballot(raise)) {
    const float m_new = raise ? mx : m_run;
    const float alpha = raise ? __builtin_amdgcn_exp2f((m_run - m_new) * kC) : 1.0f;  // 0 from -inf
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[dt] *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
  float rs = 0.0f;
  u32x4 pr, pn;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float p0 = __builtin_amdgcn_exp2f((Sv[0][v] - m_use) * kC);
    const float p1 = __builtin_amdgcn_exp2f((Sv[1][v] - m_use) * kC);
    rs = v == 0 ? p0 + p1 : rs + (p0 + p1);  // the first pair starts the sum (no add of +0)
    pr[v] = pack_bf16(p0, p1);
    pn[v] = pack_bf16(p0 * sc4[0][v], p1 * sc4[1][v]);
  }
  rs = pair_sum32(pair_sum16(rs));
  l_run += rs;

  // the chunk's keys into this wave's LDS buffer, key-major: lane (r, g) holds dims 32G + 8g .. +7 of key r
  // of both tiles (LDS operations of one wave complete in order, so the reads below see these writes)
  {
    const u32x4 grp[4][2] = {{kn0[0], kn0[1]}, {kn1[0], kn1[1]}, {cur.r0[0], cur.r0[1]}, {cur.r1[0], cur.r1[1]}};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int G = 0; G < 4; ++G)
        *reinterpret_cast<u32x4*>(kd + (tt * 16 + r) * kKdStride + 32 * G + 8 * g) = grp[G][tt];
  }
  // O^T += V^T . P^T : dim tiles 0..3 (nope, P * scale), 4..7 (RoPE, P)
  const bf16x8 bn = __builtin_bit_cast(bf16x8, pn), br = __builtin_bit_cast(bf16x8, pr);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kd + voff[0] + dt * 16));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kd + voff[1] + dt * 16));
    const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
    const u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
    O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), dt < 4 ? bn : br, O[dt], 0, 0,
                                                     0);
  }
}

// NR chunks of one wave: every gather issued first, then the chunks in order (straight-line code).
template <int NR>
__device__ __forceinline__ void attend_round(const Keys K, int slot0, int end, const bf16x8 (&qb)[4], float* scl,
                                             uint16_t* kd, const int (&voff)[2], int r, int g, float& m_run,
                                             float& l_run, v4f (&O)[8]) {
  Raw buf[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) K.load(slot0 + u * kChunk, end, r, g, buf[u]);
#pragma unroll
  for (int u = 0; u < NR; ++u)
    attend_chunk(buf[u], slot0 + u * kChunk, end, qb, scl, kd, voff, r, g, m_run, l_run, O);
}

// The last split's merge of a (query, group): every split's (m, l, o slice) of this thread's head h and
// dims d0..d0+3, loaded at once and unconditionally (a load behind a branch would make the compiler wait
// for all outstanding loads there: one memory round trip per split), NS >= splits slots, the ones past
// the last split duplicates of it that weigh 0. The partials were written with agent-scope stores by
// workgroups on other XCDs, so they are read with agent-scope loads.
template <int NS>
__device__ __forceinline__ void merge_splits(const AttendPartial* all, int splits, int h, int d0, float& M, float& L,
                                             float (&acc)[4]) {
  constexpr float kC = kLog2eRsqrtD;
  auto ld = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  float mv[NS], lv[NS], ov[NS][4];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int sp = min(u, splits - 1);
    mv[u] = ld(&all[sp].m[h]);
    lv[u] = ld(&all[sp].l[h]);
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[u][i] = ld(&all[sp].o[h][d0 + i]);
  }
  M = -INFINITY;
#pragma unroll
  for (int u = 0; u < NS; ++u) M = fmaxf(M, mv[u]);  // duplicates of the last split change nothing
  L = 0.0f;
  acc[0] = acc[1] = acc[2] = acc[3] = 0.0f;
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    // an empty split (m = -inf, l = 0, o = 0) weighs 0, and so does a duplicate
    const float f = u < splits ? __builtin_amdgcn_exp2f((mv[u] - M) * kC) : 0.0f;
    L += lv[u] * f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += ov[u][i] * f;
  }
}

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

  // rotated query as the B operand of S^T = K . Q^T (RoPE dims 64..127: ks = 2, 3)
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v = qraw[ks];
    if (ks >= 2) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int pi = 16 * (ks - 2) + 4 * g + u;
        const float c = S.cos_t[pi], s = S.sin_t[pi];
        const float x0 = bf16_to_f32((uint16_t)(v[u] & 0xFFFFu));
        const float x1 = bf16_to_f32((uint16_t)(v[u] >> 16));
        v[u] = (uint32_t)f32_to_bf16(x0 * c - x1 * s) | ((uint32_t)f32_to_bf16(x0 * s + x1 * c) << 16);
      }
    }
    qb[ks] = __builtin_bit_cast(bf16x8, v);
  }

  float m_run = -INFINITY, l_run = 0.0f;
  v4f O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  uint16_t* kd = S.u.b.kd[wave];
  float* scl = &S.u.b.scl[wave][0][0];
  // V^T operand rows of this lane for the two transposing reads h: MFMA K index 8g + 4h + u (u = r / 4)
  // is key 16 ((4h+u) % 2) + 4g + (4h+u) / 2; the lane addresses that key's dims 4 (r % 4) .. +3 of
  // each 16-dim tile
  int voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kk = 4 * h + (r >> 2);
    voff[h] = (16 * (kk & 1) + 4 * g + (kk >> 1)) * kKdStride + 4 * (r & 3);
  }

  // wave w: key slots [s_begin + w * per, + per) of the split, in rounds of up to kRound chunks
  const int per = ((per_split + kWaves * 16 - 1) / (kWaves * 16)) * 16;
  const int w_begin = s_begin + wave * per;
  const int w_end = min(w_begin + per, s_end);
  const int w_chunks = (per + kChunk - 1) / kChunk;  // the same for every wave
  for (int c = 0; c < w_chunks; c += kRound) {
    const int slot0 = w_begin + c * kChunk;
    switch (min(kRound, w_chunks - c)) {
      case 1: attend_round<1>(K, slot0, w_end, qb, scl, kd, voff, r, g, m_run, l_run, O); break;
      case 2: attend_round<2>(K, slot0, w_end, qb, scl, kd, voff, r, g, m_run, l_run, O); break;
      case 3: attend_round<3>(K, slot0, w_end, qb, scl, kd, voff, r, g, m_run, l_run, O); break;
      case 4: attend_round<4>(K, slot0, w_end, qb, scl, kd, voff, r, g, m_run, l_run, O); break;
      default: attend_round<kRound>(K, slot0, w_end, qb, scl, kd, voff, r, g, m_run, l_run, O); break;
    }
  }

  // ---- merge the 8 wave states: lane (r, g) holds head r, dims dt*16 + 4g + v
  __syncthreads();
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<v4f*>(&S.u.c.o[wave][r][dt * 16 + 4 * g]) = O[dt];
  if (g == 0) {
    S.u.c.m[wave][r] = m_run;
    S.u.c.l[wave][r] = l_run;
  }
  __syncthreads();
  {
    const int h = tid >> 5, d0 = (tid & 31) * 4;
    // wave states in raw logit units (q . x): weight 2^((m_w - M) log2(e) / sqrt(128))
    constexpr float kC = kLog2eRsqrtD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, S.u.c.m[w][h]);
    float L = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = S.u.c.m[w][h];
      if (mw == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f((mw - M) * kC);
      L += S.u.c.l[w][h] * f;
      const v4f ov = *reinterpret_cast<const v4f*>(&S.u.c.o[w][h][d0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += ov[i] * f;
    }
    if (splits > 1) {
      // This split's partial; the last split of the (query, group) to finish merges all of them. The
      // workgroups sit on different XCDs, whose L2s are not coherent with each other: the partials are
      // written and read with agent-scope atomic stores and loads, which go to memory, so no L2
      // writeback or invalidate is needed (an agent-scope release / acquire fence does both, for every
      // dirty line of the L2, at several microseconds). Each thread waits for its own stores to
      // complete before the workgroup counts itself in.
      AttendPartial* mine = args.part + ((size_t)q * hgs + hg) * splits + split;
#pragma unroll
      for (int i = 0; i < 4; ++i) __hip_atomic_store(&mine->o[h][d0 + i], acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d0 == 0) {
        __hip_atomic_store(&mine->m[h], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&mine->l[h], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      uint32_t* cnt = args.cnt + (size_t)q * hgs + hg;
      __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
      __syncthreads();
      if (tid == 0)
        S.last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(splits - 1);
      __syncthreads();
      if (!S.last) return;
      if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
      const AttendPartial* all = args.part + ((size_t)q * hgs + hg) * splits;
      if (splits <= kAttendMaxSplits / 2) merge_splits<kAttendMaxSplits / 2>(all, splits, h, d0, M, L, acc);
      else merge_splits<kAttendMaxSplits>(all, splits, h, d0, M, L, acc);
    }
    const int hh = hg * 16 + h;
    if (hh < a.H) {
      const float inv = 1.0f / L;
      const size_t row = ((size_t)b * a.Tq + tq) * a.H + hh;
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16);
      *reinterpret_cast<uint2*>(a.out + row * kHeadDim + d0) = pk;
      if (a.lse && d0 == 0) a.lse[row] = M * 0.08838834764831845f + __logf(L);  // natural-log units
    }
  }
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
