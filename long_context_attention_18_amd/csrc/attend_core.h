// attend_core.h -- the decode attention's per-wave pieces, shared by attend_kernel (attend.hip) and the
// CSA step launch (indexer.hip): key-slot addressing, the 32-key chunk (QK^T and PV^T on bf16 MFMA with an
// online softmax), the wave and key-split merges.
//
// Figure 3 of "DeepSeek-V4: a million-token context that agents can actually use" (CSA: the selected
// compressed blocks plus a sliding-window branch) and Figure 4 / the HCA paragraph (every compressed block
// plus the window), with one softmax over all of a query's keys:
//   logit = RoPE(q_h, t) . x / sqrt(128),  K = V = the dequantised entry.
// The MFMA operand layouts are described in attend.hip.
#pragma once
#include "attn_common.h"
#include "dev_formats.h"
#include "kernels.h"

namespace lca {
namespace {

constexpr int kWaves = 8;
constexpr int kChunk = 32;     // keys per wave step: two 16-key tiles
constexpr int kKdStride = 136;  // bf16 per key-major LDS row (128 dims + 8 pad)
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The attention's per-wave LDS: each wave's key-major copy of its current chunk (the V^T operand of the
// transposing reads) and its key scales, then, once the keys are done, the wave states for their merge.
struct AttnWaveLds {
  union {
    struct {
      uint16_t kd[kWaves][kChunk * kKdStride];    // per-wave key-major copy of its current chunk
      float scl[kWaves][2][16];                   // per-wave key scales of the chunk's two tiles
    } b;
    struct {
      float o[kWaves][16][kHeadDim + 4];  // row stride 132 floats: conflict-free 16-B accesses
      float m[kWaves][16], l[kWaves][16];
    } c;
  };
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
  const int32_t* list;      // the compressed entries of list slots list0 .. (the whole list: list0 = 0)
  int list0;
  size_t win_row, blk_row;  // b * ring, b * max_blocks
  uint32_t win_base;        // ring slot of the first window position
  int64_t j_max;            // last visible block (0 when none)
  int n_win, n_list;
  bool use_list;
  // Entry of key slot `slot` (< n_win + n_list): window position t - n_win + 1 + slot, or the
  // compressed block of list slot slot - n_win (dense: block slot - n_win). Branch-free, so the loads
  // that follow stay in straight-line code and the compiler can wait for them one chunk at a time.
  // A list held from list0 on is asked only for slots of its own.
  __device__ __forceinline__ size_t entry(int slot, bool* in_win) const {
    *in_win = slot < n_win;
    const int li = *in_win ? list0 : slot - n_win;
    int64_t j = use_list ? (int64_t)list[li - list0] : (int64_t)li;
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
#pragma unroll
    for (int v = 0; v < 4; ++v) Sv[tt][v] = fmaf(an[v], sc4[tt][v], ar[v]);
  }
  if (chunk_slot + kChunk > end) {  // the split's last chunk: slots at or beyond end are empty
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (chunk_slot + tt * 16 + 4 * g + v >= end) Sv[tt][v] = -INFINITY;
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
  const float mC = m_use * kC;
  float rs = 0.0f;
  u32x4 pr, pn;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(Sv[0][v], kC, -mC));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(Sv[1][v], kC, -mC));
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

// NR chunks of one wave (chunk u at slot0 + u stride): every gather issued first, then the chunks in order
// (straight-line code).
template <int NR>
__device__ __forceinline__ void attend_round(const Keys K, int slot0, int stride, int end, const bf16x8 (&qb)[4],
                                             float* scl, uint16_t* kd, const int (&voff)[2], int r, int g,
                                             float& m_run, float& l_run, v4f (&O)[8]) {
  Raw buf[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) K.load(slot0 + u * stride, end, r, g, buf[u]);
#pragma unroll
  for (int u = 0; u < NR; ++u)
    attend_chunk(buf[u], slot0 + u * stride, end, qb, scl, kd, voff, r, g, m_run, l_run, O);
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
  auto ld2 = [](const float* p, float* v) {  // two adjacent floats in one 8-byte load
    const uint64_t w = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v[0] = __uint_as_float((uint32_t)w);
    v[1] = __uint_as_float((uint32_t)(w >> 32));
  };
  float mv[NS], lv[NS], ov[NS][4];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int sp = min(u, splits - 1);
    mv[u] = ld(&all[sp].m[h]);
    lv[u] = ld(&all[sp].l[h]);
    ld2(&all[sp].o[h][d0], &ov[u][0]);
    ld2(&all[sp].o[h][d0 + 2], &ov[u][2]);
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

// The query rows of this lane (head r of the group, dims 32 ks + 8 g ..) as the B operand of S^T = K . Q^T,
// with the position's RoPE rotation applied to the rotated dims 64..127 (ks = 2, 3) from the angles in LDS.
__device__ __forceinline__ void rotate_query(const u32x4 (&qraw)[4], const float* cos_t, const float* sin_t, int g,
                                             bf16x8 (&qb)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v = qraw[ks];
    if (ks >= 2) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int pi = 16 * (ks - 2) + 4 * g + u;
        const float c = cos_t[pi], s = sin_t[pi];
        const float x0 = bf16_to_f32((uint16_t)(v[u] & 0xFFFFu));
        const float x1 = bf16_to_f32((uint16_t)(v[u] >> 16));
        v[u] = (uint32_t)f32_to_bf16(x0 * c - x1 * s) | ((uint32_t)f32_to_bf16(x0 * s + x1 * c) << 16);
      }
    }
    qb[ks] = __builtin_bit_cast(bf16x8, v);
  }
}

// Wave `wave`'s share of a split's key slots [s_begin, s_end): every 8th 32-slot chunk from the wave's
// own, in rounds of up to KR chunks whose gathers are issued together. Starts the running state (m_run,
// l_run, O) of the wave's 16 heads.
template <int KR>
__device__ __forceinline__ void attend_slots(const Keys& K, int s_begin, int s_end, int per_split,
                                             const bf16x8 (&qb)[4], AttnWaveLds& W, int wave, int r, int g,
                                             float& m_run, float& l_run, v4f (&O)[8]) {
  m_run = -INFINITY;
  l_run = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  uint16_t* kd = W.b.kd[wave];
  float* scl = &W.b.scl[wave][0][0];
  // V^T operand rows of this lane for the two transposing reads h: MFMA K index 8g + 4h + u (u = r / 4)
  // is key 16 ((4h+u) % 2) + 4g + (4h+u) / 2; the lane addresses that key's dims 4 (r % 4) .. +3 of
  // each 16-dim tile
  int voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kk = 4 * h + (r >> 2);
    voff[h] = (16 * (kk & 1) + 4 * g + (kk >> 1)) * kKdStride + 4 * (r & 3);
  }
  // the split's 32-slot chunks (the last one partial) dealt to the waves in turn: wave w takes chunks w,
  // w + 8, ..., so no wave holds more than one chunk beyond another's and only the split's last chunk is
  // partial (per-wave ranges rounded each wave's share up to whole chunks)
  (void)per_split;
  constexpr int kStride = kWaves * kChunk;
  const int n_ch = (s_end - s_begin + kChunk - 1) / kChunk;
  const int mine = n_ch > wave ? (n_ch - wave + kWaves - 1) / kWaves : 0;
  for (int c = 0; c < mine; c += KR) {
    const int slot0 = s_begin + (wave + c * kWaves) * kChunk;
    switch (min(KR, mine - c)) {
      case 1: attend_round<1>(K, slot0, kStride, s_end, qb, scl, kd, voff, r, g, m_run, l_run, O); break;
      case 2:
        if constexpr (KR >= 2)
          attend_round<2>(K, slot0, kStride, s_end, qb, scl, kd, voff, r, g, m_run, l_run, O);
        break;
      case 3:
        if constexpr (KR >= 3)
          attend_round<3>(K, slot0, kStride, s_end, qb, scl, kd, voff, r, g, m_run, l_run, O);
        break;
      default:
        if constexpr (KR >= 4)
          attend_round<KR>(K, slot0, kStride, s_end, qb, scl, kd, voff, r, g, m_run, l_run, O);
        break;
    }
  }
}

// The 8 wave states of (query q, head group hg) merged in LDS; with key splits, this split's partial and,
// by the last split of the (query, group) to finish, the merge of all of them; then the output rows (and
// lse). `last`: an LDS word. Every thread calls it; a split that is not the last returns early. poison: the
// split's sum is NaN, and so are the rows it merges into.
__device__ __forceinline__ void attend_finish(const AttendArgs& args, AttnWaveLds& W, int* last, int q, int hg,
                                              int split, float m_run, float l_run, const v4f (&O)[8],
                                              bool poison = false) {
  const AttnArgs& a = args.t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int hgs = (a.H + 15) / 16;
  const int splits = args.splits;
  const int b = q / a.Tq, tq = q % a.Tq;
  // lane (r, g) holds head r, dims dt*16 + 4g + v
  __syncthreads();
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<v4f*>(&W.c.o[wave][r][dt * 16 + 4 * g]) = O[dt];
  if (g == 0) {
    W.c.m[wave][r] = m_run;
    W.c.l[wave][r] = l_run;
  }
  __syncthreads();
  const int h = tid >> 5, d0 = (tid & 31) * 4;
  // wave states in raw logit units (q . x): weight 2^((m_w - M) log2(e) / sqrt(128))
  constexpr float kC = kLog2eRsqrtD;
  // branch-free, so that the LDS reads of all 8 wave states are issued together; a wave without keys
  // (m = -inf, l = 0, o = 0) weighs 0
  float mw[kWaves];
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = W.c.m[w][h];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float f = mw[w] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mw[w] - M) * kC);
    L += W.c.l[w][h] * f;
    const v4f ov = *reinterpret_cast<const v4f*>(&W.c.o[w][h][d0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += ov[i] * f;
  }
  if (poison) L = __builtin_nanf("");
  if (splits > 1) {
    // This split's partial; the last split of the (query, group) to finish merges all of them. The
    // workgroups sit on different XCDs, whose L2s are not coherent with each other: the partials are
    // written and read with agent-scope atomic stores and loads, which go to memory, so no L2
    // writeback or invalidate is needed (an agent-scope release / acquire fence does both, for every
    // dirty line of the L2, at several microseconds). Each thread waits for its own stores to
    // complete before the workgroup counts itself in.
    AttendPartial* mine = args.part + ((size_t)q * hgs + hg) * splits + split;
    uint64_t* op = reinterpret_cast<uint64_t*>(&mine->o[h][d0]);  // (16-byte aligned: d0 % 4 == 0)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __hip_atomic_store(op + i, (uint64_t)__float_as_uint(acc[2 * i]) | ((uint64_t)__float_as_uint(acc[2 * i + 1]) << 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d0 == 0) {
      __hip_atomic_store(&mine->m[h], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&mine->l[h], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    uint32_t* cnt = args.cnt + (size_t)q * hgs + hg;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0)
      *last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(splits - 1);
    __syncthreads();
    if (!*last) return;
    if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
    const AttendPartial* all = args.part + ((size_t)q * hgs + hg) * splits;
    if (splits <= 4) merge_splits<4>(all, splits, h, d0, M, L, acc);
    else if (splits <= 8) merge_splits<8>(all, splits, h, d0, M, L, acc);
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

}  // namespace
}  // namespace lca
