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
// folded into P for the nope output dims. The query is taken times log2(e)/sqrt(128) before its bf16
// rounding and the RoPE half of each logit's MFMA chain starts at minus the head's running maximum, so
// the chunk's values are the exp2 arguments as they come out; each head's softmax denominator is a
// ninth PV MFMA over an all-ones V tile (the same bf16 P as the output's). The next chunk's gathers are issued before the current chunk
// is computed, into the second of two LDS buffers, one barrier per chunk. The window's slots start at the
// first whole 16-key tile after the compressed ones, so a tile reads one array, whose base (the sequence's
// rows) is the same for every lane and takes 32-bit byte offsets; each gathering thread resolves its key's
// entry itself (the top-k row is in LDS). Waves 0-1 gather FP8 codes and scales, waves 2-3 RoPE dims, each
// kind in its own copy of the chunk loop. Calls with up to 511 queries use attend.hip.
#include "attn_common.h"
#include "dev_formats.h"
#include "kernels.h"

namespace lca {

namespace {

constexpr int kMWaves = 4;       // one wave per 16-head group
constexpr int kMThreads = kMWaves * 64;
constexpr int kMChunk = 32;      // keys per step: 16-key tiles, pairs of them one PV K-step
constexpr int kMTiles = kMChunk / 16;
static_assert(kMChunk % 32 == 0 && kMChunk <= 64, "whole PV K-steps");
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
  uint16_t kd[2][kKdBuf];  // key-major chunk (two buffers)
  float scl[2][kMChunk];   // the keys' FP8 scales (>= 0); -1 marks a slot without a key
  uint32_t kbad[2];        // per chunk buffer: some slot of the chunk holds no key
  int32_t list[kMaxTopk];  // CSA: the query's top-k row
  float cos_t[32], sin_t[32];
};

// The gather of one thread for one chunk: part pp = tid / 16 (dims 8pp .. 8pp+7; pp < 8 the FP8 nope
// codes, pp >= 8 the BF16 RoPE dims), key r = tid % 16 of both tiles.
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

struct Fetch {
  u32x4 d[kMTiles];  // the part's dims: FP8 codes in the first two words (pp < 8), else BF16 RoPE dims
  float scale[kMTiles];
  bool valid[kMTiles];
};

// One query's key slots: [0, n_first) the top-k row (CSA) or the visible blocks (HCA), then, from the
// first whole 16-key tile on (win0), the window positions t - n_win + 1 .. t; slots in between hold no
// key. A tile is thus all compressed or all window, and the choice of array is the same for every lane.
struct Query {
  const uint8_t *blk_codes, *win_codes;  // this sequence's rows (offsets below stay under 2^32 bytes)
  const uint16_t *blk_rope, *win_rope;
  const float *blk_scale, *win_scale;
  int32_t N;                // visible blocks
  int32_t n_first;          // top-k slots or visible blocks
  int32_t win0, total;      // first window slot (n_first rounded up to 16), win0 + n_win
  int32_t win_base, ring;   // ring slot of the first window position (t - n_win + 1)
  bool dense;
};

// The gathers of key r of the chunk's two tiles (this thread's part). A slot without a key reads row 0
// of its array (in bounds) and is flagged; its row is zeroed when staged. Branch-free (the array choice is
// uniform), so that the compiler can keep two chunks' loads in flight and wait for the older ones only.
template <bool NOPE>
__device__ __forceinline__ void fetch(const Query& Q, const int32_t* list, int chunk0, int pp, int r, Fetch& F) {
#pragma unroll
  for (int tt = 0; tt < kMTiles; ++tt) {
    const int tile0 = chunk0 + tt * 16;
    const int slot = tile0 + r;
    const bool win = tile0 >= Q.win0;
    int ws = Q.win_base + (slot - Q.win0);  // < 2 ring for a live window slot: one conditional wrap
    ws = ws >= Q.ring ? ws - Q.ring : ws;
    const int jl = list[min(slot, kMaxTopk - 1)];  // (CSA: slot < win0 <= kMaxTopk; unused otherwise)
    const int j = Q.dense ? slot : jl;
    const bool ok = win ? slot < Q.total : (slot < Q.n_first && j >= 0 && j < Q.N);
    const uint32_t e = ok ? (uint32_t)(win ? ws : j) : 0u;
    F.valid[tt] = ok;
    // byte offsets in 32 bits from the sequence's (uniform) row base
    if (NOPE) {
      const u32x2 c = ldg<u32x2>((win ? Q.win_codes : Q.blk_codes) + (e * (uint32_t)kNope + 8u * (uint32_t)pp));
      F.d[tt][0] = c[0];
      F.d[tt][1] = c[1];
      F.scale[tt] = ldg<float>((const uint8_t*)(win ? Q.win_scale : Q.blk_scale) + e * 4u);
    } else {
      F.d[tt] = ldg<u32x4>((const uint8_t*)(win ? Q.win_rope : Q.blk_rope) +
                           (e * (uint32_t)(2 * kRope) + 16u * (uint32_t)(pp - 8)));
    }
  }
}

// the fetched dims into the chunk buffer's key-major rows (a slot without a key as zeros); *kbad: whether
// the chunk needs the masked path (wave 0's part-0 lanes cover all of the chunk's slots)
template <bool NOPE>
__device__ __forceinline__ void stage(const Fetch& F, int pp, int r, int koff, uint16_t* kd, float* scl, uint32_t* kbad) {
  bool bad = false;
#pragma unroll
  for (int tt = 0; tt < kMTiles; ++tt) bad |= !F.valid[tt];
#pragma unroll
  for (int tt = 0; tt < kMTiles; ++tt) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 v = NOPE ? fp8x8_to_bf16((u32x2){F.d[tt][0], F.d[tt][1]}) : F.d[tt];
    if (bad && !F.valid[tt]) v = zero;
    *reinterpret_cast<u32x4*>(kd + tt * kKdTile + koff) = v;
  }
  if (NOPE && pp == 0) {
#pragma unroll
    for (int tt = 0; tt < kMTiles; ++tt) scl[16 * tt + r] = F.valid[tt] ? F.scale[tt] : -1.0f;
  }
  if (NOPE && threadIdx.x < 64) {
    const uint64_t m = __ballot(pp == 0 && bad);
    if (threadIdx.x == 0) *kbad = m != 0 ? 1u : 0u;
  }
}

__global__ __launch_bounds__(kMThreads) void attn_kernel(AttnArgs a) {
  __shared__ ManyLds S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int q = blockIdx.x;
  const int b = q / a.Tq, tq = q % a.Tq;
  const int64_t t = query_t(a.seq_len, a.seq_T, a.seq_cap, a.len, a.Tq, b, tq);
  if (t < 0) return;  // ragged batch: no query in this row

  Query Q;
  const size_t brow = (size_t)b * a.max_blocks, wrow = (size_t)b * a.ring;
  Q.blk_codes = a.blk_codes + brow * kNope;
  Q.win_codes = a.win_codes + wrow * kNope;
  Q.blk_rope = a.blk_rope + brow * kRope;
  Q.win_rope = a.win_rope + wrow * kRope;
  Q.blk_scale = a.blk_scale + brow;
  Q.win_scale = a.win_scale + wrow;
  Q.N = (int32_t)min((t + 1) / a.m, a.max_blocks);  // 0 for the window-only layer
  Q.dense = a.dense != 0;
  Q.n_first = Q.dense ? Q.N : a.k;
  Q.win0 = (Q.n_first + 15) & ~15;
  const int32_t n_win = (int32_t)min((int64_t)a.W, t + 1);
  Q.total = Q.win0 + n_win;
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

  // rotated query as the B operand of S^T = K . Q^T (RoPE dims 64..127: ks = 2, 3), times log2(e)/sqrt(128)
  // before its bf16 rounding: the logits come out of the MFMA in exp2 units
  constexpr float kC = kLog2eRsqrtD;
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v = qraw[ks];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x0 = bf16_to_f32((uint16_t)(v[u] & 0xFFFFu));
      const float x1 = bf16_to_f32((uint16_t)(v[u] >> 16));
      float y0 = x0, y1 = x1;
      if (ks >= 2) {
        const int pi = 16 * (ks - 2) + 4 * g + u;
        const float c = S.cos_t[pi], s = S.sin_t[pi];
        y0 = x0 * c - x1 * s;
        y1 = x0 * s + x1 * c;
      }
      v[u] = (uint32_t)f32_to_bf16(y0 * kC) | ((uint32_t)f32_to_bf16(y1 * kC) << 16);
    }
    qb[ks] = __builtin_bit_cast(bf16x8, v);
  }

  // Running state of head r (log2 units): m_run, the softmax's reference point (-inf until the head has a
  // key); the RoPE half of every logit starts its MFMA chain at -ref (ref = m_run, 0 before the first
  // key), so the chunk's values are already logit - ref, the exp2 argument. O is rescaled only when a
  // chunk's maximum rises above ref by more than kLazy (lim); the row sum l accumulates in a ninth PV
  // MFMA whose V tile is all ones (every lane of head r holds it), from the same bf16 P as O.
  constexpr float kLazy = 8.0f;
  float m_run = -INFINITY, ref = 0.0f, lim = -INFINITY;
  v4f nref = {0.0f, 0.0f, 0.0f, 0.0f};
  v4f O[8], Lsum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, (u32x4){0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
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
  // This thread gathers part pp of key rr of both tiles of a chunk (parts 0-7, the FP8 codes, in waves 0-1;
  // the choice is per wave, so each kind of wave runs its own copy of the loop).
  const int pp = tid >> 4, rr = tid & 15;
  const int koff = rr * kKdStride + 8 * pp;
  auto run = [&](auto nope_tag) {
    constexpr bool NOPE = decltype(nope_tag)::value;
    Fetch F;
    fetch<NOPE>(Q, S.list, 0, pp, rr, F);
    stage<NOPE>(F, pp, rr, koff, S.kd[0], S.scl[0], &S.kbad[0]);
    __syncthreads();
  // Step c (chunk c in buffer cur): the next chunk's gathers first (slots past the end read an in-bounds
  // entry and are masked), then chunk c, then the next chunk into the other buffer.
  auto step = [&](int c, int cur) {
    fetch<NOPE>(Q, S.list, (c + 1) * kMChunk, pp, rr, F);
    if (active) {
      const uint16_t* kd = S.kd[cur];
      const float* scl = S.scl[cur];
      float Sv[kMTiles][4];
      v4f sc4[kMTiles];
#pragma unroll
      for (int tt = 0; tt < kMTiles; ++tt) {
        const uint16_t* krow = kd + tt * kKdTile + r * kKdStride + 8 * g;
        v4f an = {0.0f, 0.0f, 0.0f, 0.0f};
        an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow)), qb[0], an, 0, 0, 0);
        an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 32)), qb[1], an, 0, 0, 0);
        v4f ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 64)), qb[2], nref, 0, 0, 0);
        ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 96)), qb[3], ar, 0, 0, 0);
        sc4[tt] = *reinterpret_cast<const v4f*>(scl + tt * 16 + 4 * g);
#pragma unroll
        for (int v = 0; v < 4; ++v) Sv[tt][v] = fmaf(an[v], sc4[tt][v], ar[v]);  // logit - ref
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
      mx = pair_max32(pair_max16(mx));  // the chunk's largest logit - ref
      const bool raise = mx > lim;      // the first finite maximum, or a rise of more than kLazy
      if (__builtin_amdgcn_read_exec() & __ballot(raise)) {
        const float m_new = raise ? mx + ref : m_run;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 0 from -inf
        const float sh = raise ? mx : 0.0f;                                          // m_new - ref
#pragma unroll
        for (int tt = 0; tt < kMTiles; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v) Sv[tt][v] -= sh;
        Lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) O[dt] *= alpha;
        m_run = m_new;
        ref = m_run == -INFINITY ? 0.0f : m_run;
        lim = m_run == -INFINITY ? -INFINITY : kLazy;
        nref = (v4f){-ref, -ref, -ref, -ref};
      }
#pragma unroll
      for (int ksp = 0; ksp < kMTiles / 2; ++ksp) {
        // P of tiles 2 ksp, 2 ksp + 1: the B operand of one PV K-step
        u32x4 pr, pn;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p0 = __builtin_amdgcn_exp2f(Sv[2 * ksp][v]);
          const float p1 = __builtin_amdgcn_exp2f(Sv[2 * ksp + 1][v]);
          pr[v] = pack_bf16(p0, p1);
          pn[v] = pack_bf16(p0 * sc4[2 * ksp][v], p1 * sc4[2 * ksp + 1][v]);
        }
        // O^T += V^T . P^T : dim tiles 0..3 (nope, P * scale), 4..7 (RoPE, P); the row sums from the ones tile
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
        Lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, br, Lsum, 0, 0, 0);
      }
    }
    // the next chunk into the other buffer (last read in the previous step, before the barrier below)
    if (c + 1 < n_chunks) stage<NOPE>(F, pp, rr, koff, S.kd[cur ^ 1], S.scl[cur ^ 1], &S.kbad[cur ^ 1]);
    __syncthreads();
  };
  for (int c = 0; c < n_chunks; c += 2) {
    step(c, 0);
    if (c + 1 < n_chunks) step(c + 1, 1);
  }
  };
  if (__builtin_amdgcn_readfirstlane(pp) < 8) run(BoolTag<true>{});
  else run(BoolTag<false>{});

  // ---- output: lane (r, g) holds head 16 * wave + r, dims dt * 16 + 4g .. +3
  if (active && head_ok) {
    const float l_run = Lsum[0];
    const float inv = 1.0f / l_run;
    const size_t row = ((size_t)b * a.Tq + tq) * a.H + head;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(O[dt][0] * inv) | ((uint32_t)f32_to_bf16(O[dt][1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16(O[dt][2] * inv) | ((uint32_t)f32_to_bf16(O[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(a.out + row * kHeadDim + dt * 16 + 4 * g) = pk;
    }
    if (a.lse && g == 0) a.lse[row] = m_run * 0.6931471805599453f + __logf(l_run);  // natural-log units
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int32_t B, hipStream_t s) {
  const unsigned nq = (unsigned)(B * a.Tq);
  hipLaunchKernelGGL(attn_kernel, dim3(nq), dim3(kMThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lca
