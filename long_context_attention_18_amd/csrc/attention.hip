// attention.hip -- CSA sparse / HCA dense / window-only attention with the sliding-window branch
// under one softmax, for calls with many queries (chunked prefill), on gfx950.
//
// Figure 3 of "DeepSeek-V4: a million-token context that agents can actually use" (CSA: the selected
// compressed blocks plus a sliding-window branch over the recent uncompressed tokens) and Figure 4 /
// the HCA paragraph (every compressed block, densely, plus the same window). Per query t and head h:
//   keys  = {D1 entries: top-k list (CSA) or all j < (t+1)/m (HCA)}
//           + {window entries of positions max(0, t-W+1) .. t}
//   logit = RoPE(q_h, t) . x / sqrt(128),  K = V = the dequantised entry
//   out   = softmax over ALL keys (one normalisation) . x
//
// All query heads share the one KV head. One workgroup per query, one wave per 16 heads. The keys go
// 32 at a time through LDS, gathered and converted once for all heads: every thread brings in 8 dims
// of two keys (key r of the two 16-key tiles) and writes them key-major, the A operand of
// S^T = K.Q^T (keys as the MFMA's M dimension). The S^T accumulator is exactly the B operand of
// O^T = V^T.P^T when MFMA K index 8g + 2v + t is key 4g+v of tile t, so P never leaves registers, and
// the V^T operand comes from the same key-major rows through gfx950's transposing LDS read
// (ds_read_b64_tr_b16: lane 4a + e of a 16-lane group gets element e of the 8-byte rows the group's
// lanes a, a+4, a+8, a+12 address), each lane addressing the key its K index needs. The FP8 codes and
// the BF16 RoPE dims are exact in bf16; the per-entry fp32 scale multiplies the nope logits and is
// folded into P for the nope output dims. The next chunk's gathers are issued before the current chunk
// is computed, into the second of two LDS buffers, one barrier per chunk. Calls with up to 511 queries
// use attend.hip.
#include "attn_common.h"
#include "dev_formats.h"
#include "kernels.h"

namespace lca {

namespace {

constexpr int kMWaves = 4;       // one wave per 16-head group
constexpr int kMThreads = kMWaves * 64;
constexpr int kMChunk = 32;      // keys per step: 16-key tiles, pairs of them one PV K-step
constexpr int kMTiles = kMChunk / 16;
static_assert(kMChunk % 32 == 0 && kMChunk <= 64, "whole PV K-steps; make_entries uses one wave");
// Key-major chunk layout (bf16 offsets): row r of 16-key tile tt at tt * kKdTile + r * kKdStride. In
// 4-byte LDS banks the row stride is 12 (mod 64) and tile 1 starts 32 banks after tile 0, so the 16 rows
// a QK operand read touches (4 banks each) and the four 8-bank row pieces a transposing read gathers per
// 16-lane group (keys 4g, 4g+1 of both tiles) all fall on distinct banks.
constexpr int kKdStride = 152;                 // 76 banks per row: 128 bf16 + 24 pad
constexpr int kKdTile = 16 * kKdStride + 64;   // tile 1 offset: 1248 banks, 32 (mod 64)
constexpr int kKdBuf = (kMTiles - 1) * kKdTile + 16 * kKdStride;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct ManyLds {
  uint16_t kd[2][kKdBuf];                 // key-major chunk (two buffers)
  float scl[2][kMChunk];                  // the keys' FP8 scales (>= 0); -1 marks a slot without a key
  uint32_t kbad[2];                       // per chunk buffer: some slot of the chunk holds no key
  uint32_t ent[2][kMChunk];               // entries of the slots of the chunk after next (~0: no key)
  uint32_t ebad[2];                       // per entry buffer: some slot holds no key
  int32_t list[kMaxTopk];                 // CSA: the query's top-k row
  float cos_t[32], sin_t[32];
};

// The gather of one thread for one chunk: part pp = tid / 16 (dims 8pp .. 8pp+7; pp < 8 the FP8 nope
// codes, pp >= 8 the BF16 RoPE dims), key r = tid % 16 of both tiles.
struct Fetch {
  u32x2 code[kMTiles];
  u32x4 rope[kMTiles];
  float scale[kMTiles];
  bool valid[kMTiles];
  bool bad;  // some slot of the chunk holds no key (the same for every thread)
};

struct Query {
  const uint8_t *blk_codes, *win_codes;
  const uint16_t *blk_rope, *win_rope;
  const float *blk_scale, *win_scale;
  size_t blk_row, win_row;  // b * max_blocks, b * ring
  int32_t N;                // visible blocks
  int32_t n_first, total;   // slots [0, n_first): top-k row or dense blocks; then n_win window positions
  int32_t win_base, ring;   // ring slot of the first window position (t - n_win + 1)
  bool dense;
};

// entry of key slot `slot` (32-bit index arithmetic): slots [0, n_first) the top-k row or the dense
// blocks, then the window positions t - n_win + 1 .. t; branch-free, with an in-bounds entry for slots
// that hold no key
__device__ __forceinline__ void slot_entry(const Query& Q, const int32_t* list, int slot, size_t* e, bool* win,
                                           bool* valid) {
  const bool in_first = slot < Q.n_first;
  const int j = Q.dense ? slot : list[in_first ? slot : 0];
  const bool ok_blk = j >= 0 && j < Q.N;
  const bool live = slot < Q.total;
  int ws = Q.win_base + (slot - Q.n_first);  // < 2 ring for a live window slot: one conditional wrap
  ws = ws >= Q.ring ? ws - Q.ring : ws;
  *valid = live && (!in_first || ok_blk);
  *win = !in_first;
  *e = in_first ? Q.blk_row + (uint32_t)(ok_blk ? j : 0) : Q.win_row + (uint32_t)(live ? ws : 0);
}

// The entries of one chunk's slots, once per chunk (the first kMChunk lanes of wave 0), for the threads that
// gather them: ent[slot] = the entry index in its array (window or compressed: slot >= n_first), ~0
// for a slot without a key; *ebad: whether any slot holds none.
__device__ __forceinline__ void make_entries(const Query& Q, const int32_t* list, int chunk0, uint32_t* ent,
                                             uint32_t* ebad) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < kMChunk) {
    size_t e;
    bool w, ok;
    slot_entry(Q, list, chunk0 + lane, &e, &w, &ok);
    ent[lane] = ok ? (uint32_t)e : 0xFFFFFFFFu;  // entry indices stay below 2^32 (B x rows x 196 B of HBM)
    const uint64_t m = __ballot(!ok);
    if (lane == 0) *ebad = m != 0 ? 1u : 0u;
  }
}

__device__ __forceinline__ void fetch(const Query& Q, const uint32_t* ent, const uint32_t* ebad, int chunk0, int pp,
                                      int r, Fetch& F) {
  F.bad = *ebad != 0u;
#pragma unroll
  for (int tt = 0; tt < kMTiles; ++tt) {
    const uint32_t code = ent[tt * 16 + r];
    const bool ok = code != 0xFFFFFFFFu;
    const bool w = chunk0 + tt * 16 + r >= Q.n_first;
    const size_t e = ok ? (size_t)code : (w ? Q.win_row : Q.blk_row);  // a slot without a key: an in-bounds entry
    F.valid[tt] = ok;
    if (pp < 8) {
      F.code[tt] = ldg<u32x2>((w ? Q.win_codes : Q.blk_codes) + e * kNope + 8 * pp);
      F.scale[tt] = ldg<float>((w ? Q.win_scale : Q.blk_scale) + e);
    } else {
      F.rope[tt] = ldg<u32x4>((w ? Q.win_rope : Q.blk_rope) + e * kRope + 8 * (pp - 8));
    }
  }
}

// the fetched dims into the chunk buffer's key-major rows (a slot without a key as zeros); *kbad: whether
// the chunk needs the masked path
__device__ __forceinline__ void stage(const Fetch& F, int pp, int r, uint16_t* kd, float* scl, uint32_t* kbad) {
#pragma unroll
  for (int tt = 0; tt < kMTiles; ++tt) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 v = pp < 8 ? fp8x8_to_bf16(F.code[tt]) : F.rope[tt];
    if (F.bad && !F.valid[tt]) v = zero;
    *reinterpret_cast<u32x4*>(kd + tt * kKdTile + r * kKdStride + 8 * pp) = v;
  }
  if (pp == 0) {
#pragma unroll
    for (int tt = 0; tt < kMTiles; ++tt) scl[16 * tt + r] = F.valid[tt] ? F.scale[tt] : -1.0f;
  }
  if (threadIdx.x == 0) *kbad = F.bad ? 1u : 0u;
}

__global__ __launch_bounds__(kMThreads) void attn_kernel(AttnArgs a) {
  __shared__ ManyLds S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int q = blockIdx.x;
  const int b = q / a.Tq, tq = q % a.Tq;
  const int64_t t = query_t(a.seq_len, a.seq_T, a.len, a.Tq, b, tq);
  if (t < 0) return;  // ragged batch: no query in this row

  Query Q;
  Q.blk_codes = a.blk_codes;
  Q.win_codes = a.win_codes;
  Q.blk_rope = a.blk_rope;
  Q.win_rope = a.win_rope;
  Q.blk_scale = a.blk_scale;
  Q.win_scale = a.win_scale;
  Q.blk_row = (size_t)b * a.max_blocks;
  Q.win_row = (size_t)b * a.ring;
  Q.N = (int32_t)min((t + 1) / a.m, a.max_blocks);  // 0 for the window-only layer
  Q.dense = a.dense != 0;
  Q.n_first = Q.dense ? Q.N : a.k;
  const int32_t n_win = (int32_t)min((int64_t)a.W, t + 1);
  Q.total = Q.n_first + n_win;
  Q.ring = a.ring;
  Q.win_base = (int32_t)((t - n_win + 1) % a.ring);

  // RoPE angles of position t, the top-k row (CSA), the query rows (head 16 * wave + r, dims 32 ks + 8 g)
  if (tid < 32) {
    float sn, cs;
    rope_angle(t, a.inv_freq[tid], &sn, &cs);
    S.cos_t[tid] = cs;
    S.sin_t[tid] = sn;
  }
  if (!Q.dense) {
    const int32_t* row = a.topk + ((size_t)b * a.Tq + tq) * a.k;
    for (int i = tid; i < a.k; i += kMThreads) S.list[i] = row[i];
  }
  const int head = wave * 16 + r;
  const bool head_ok = head < a.H;
  u32x4 qraw[4];
  {
    const uint16_t* qp = a.q + (((size_t)b * a.Tq + tq) * a.H + (head_ok ? head : 0)) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      qraw[ks] = head_ok ? ldg<u32x4>(qp + ks * 32 + 8 * g) : zero;
    }
  }
  __syncthreads();  // angles and the top-k row in LDS
  make_entries(Q, S.list, 0, S.ent[0], &S.ebad[0]);
  make_entries(Q, S.list, kMChunk, S.ent[1], &S.ebad[1]);
  __syncthreads();

  // chunk 0 into buffer 0
  const int pp = tid >> 4, rr = tid & 15;
  Fetch F;
  fetch(Q, S.ent[0], &S.ebad[0], 0, pp, rr, F);

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
  stage(F, pp, rr, S.kd[0], S.scl[0], &S.kbad[0]);
  __syncthreads();

  constexpr float kC = kLog2eRsqrtD;
  constexpr float kLazy = 8.0f;  // log2 units: O is rescaled only when a head's max rises by more
  float m_run = -INFINITY, l_run = 0.0f;
  v4f O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  const bool active = wave * 16 < a.H;
  const int n_chunks = (Q.total + kMChunk - 1) / kMChunk;
  // V^T operand rows of this lane for the two transposing reads h: MFMA K index 8g + 4h + u (u = r / 4)
  // is key 16 ((4h+u) % 2) + 4g + (4h+u) / 2; the lane addresses that key's dims 4 (r % 4) .. +3 of
  // each 16-dim tile
  int voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kk = 4 * h + (r >> 2);
    voff[h] = (kk & 1) * kKdTile + (4 * g + (kk >> 1)) * kKdStride + 4 * (r & 3);
  }
  for (int c = 0; c < n_chunks; ++c) {
    const int cur = c & 1;
    // the next chunk's gathers first (slots past the end read an in-bounds entry and are masked), then
    // the entries of the chunk after it into the entry buffer the fetch of this chunk read
    fetch(Q, S.ent[(c + 1) & 1], &S.ebad[(c + 1) & 1], (c + 1) * kMChunk, pp, rr, F);
    make_entries(Q, S.list, (c + 2) * kMChunk, S.ent[cur], &S.ebad[cur]);
    if (active) {
      const uint16_t* kd = S.kd[cur];
      const float* scl = S.scl[cur];
      float Sv[kMTiles][4];
      v4f sc4[kMTiles];
#pragma unroll
      for (int tt = 0; tt < kMTiles; ++tt) {
        const uint16_t* krow = kd + tt * kKdTile + r * kKdStride + 8 * g;
        v4f an = {0.0f, 0.0f, 0.0f, 0.0f}, ar = {0.0f, 0.0f, 0.0f, 0.0f};
        an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow)), qb[0], an, 0, 0, 0);
        an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 32)), qb[1], an, 0, 0, 0);
        ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 64)), qb[2], ar, 0, 0, 0);
        ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 96)), qb[3], ar, 0, 0, 0);
        sc4[tt] = *reinterpret_cast<const v4f*>(scl + tt * 16 + 4 * g);
#pragma unroll
        for (int v = 0; v < 4; ++v) Sv[tt][v] = fmaf(an[v], sc4[tt][v], ar[v]);
      }
      if (S.kbad[cur]) {
        // a slot without a key (scale -1, all-zero dims) is masked; an entry whose nope part is all
        // zero has scale 0 and is a key like any other
#pragma unroll
        for (int tt = 0; tt < kMTiles; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v) Sv[tt][v] = sc4[tt][v] >= 0.0f ? Sv[tt][v] : -INFINITY;
      }
      // online softmax of head r (its 32 keys are spread over the 4 lane groups)
      float mx = max3_raw(max3_raw(Sv[0][0], Sv[0][1], Sv[0][2]), max3_raw(Sv[0][3], Sv[1][0], Sv[1][1]),
                          max_raw(Sv[1][2], Sv[1][3]));
#pragma unroll
      for (int tt = 2; tt < kMTiles; tt += 2)
        mx = max3_raw(mx, max3_raw(Sv[tt][0], Sv[tt][1], Sv[tt][2]), max3_raw(Sv[tt][3], Sv[tt + 1][0],
                      max3_raw(Sv[tt + 1][1], Sv[tt + 1][2], Sv[tt + 1][3])));
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
      const float mk = (m_run == -INFINITY) ? 0.0f : m_run * kC;  // exp2 argument S kC - m kC, one fma
      float rs = 0.0f;
#pragma unroll
      for (int ksp = 0; ksp < kMTiles / 2; ++ksp) {
        // P of tiles 2 ksp, 2 ksp + 1: the B operand of one PV K-step
        u32x4 pr, pn;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(Sv[2 * ksp][v], kC, -mk));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(Sv[2 * ksp + 1][v], kC, -mk));
          rs = (ksp == 0 && v == 0) ? p0 + p1 : rs + (p0 + p1);  // the first pair starts the sum (no add of +0)
          pr[v] = pack_bf16(p0, p1);
          pn[v] = pack_bf16(p0 * sc4[2 * ksp][v], p1 * sc4[2 * ksp + 1][v]);
        }
        // O^T += V^T . P^T : dim tiles 0..3 (nope, P * scale), 4..7 (RoPE, P)
        const bf16x8 bn = __builtin_bit_cast(bf16x8, pn), br = __builtin_bit_cast(bf16x8, pr);
        const uint16_t* kv = kd + 2 * ksp * kKdTile;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kv + voff[0] + dt * 16));
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kv + voff[1] + dt * 16));
          const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
          const u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
          O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), dt < 4 ? bn : br, O[dt], 0, 0, 0);
        }
      }
      rs = pair_sum32(pair_sum16(rs));
      l_run += rs;
    }
    // the next chunk into the other buffer (last read in the previous step, before the barrier below)
    if (c + 1 < n_chunks) stage(F, pp, rr, S.kd[cur ^ 1], S.scl[cur ^ 1], &S.kbad[cur ^ 1]);
    __syncthreads();
  }

  // ---- output: lane (r, g) holds head 16 * wave + r, dims dt * 16 + 4g .. +3
  if (active && head_ok) {
    const float inv = 1.0f / l_run;
    const size_t row = ((size_t)b * a.Tq + tq) * a.H + head;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(O[dt][0] * inv) | ((uint32_t)f32_to_bf16(O[dt][1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16(O[dt][2] * inv) | ((uint32_t)f32_to_bf16(O[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(a.out + row * kHeadDim + dt * 16 + 4 * g) = pk;
    }
    if (a.lse && g == 0) a.lse[row] = m_run * 0.08838834764831845f + __logf(l_run);  // natural-log units
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int32_t B, hipStream_t s) {
  const unsigned nq = (unsigned)(B * a.Tq);
  hipLaunchKernelGGL(attn_kernel, dim3(nq), dim3(kMThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lca
