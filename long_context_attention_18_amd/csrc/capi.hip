// capi.hip -- the extern "C" boundary of liblca.so (declared in include/lca.h).
//
// Host-side only: argument checks, cache carving, workspace layout, and the
// kernel launches. Every check happens before the first launch of a call, so
// a rejected call enqueues nothing.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/lca.h"
#include "kernels.h"

using namespace lca;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool desc_ok(const lca_layer_desc* d) {
  if (!d) return false;
  if (d->kind != LCA_KIND_CSA && d->kind != LCA_KIND_HCA && d->kind != LCA_KIND_SWA) return false;
  if (d->kind != LCA_KIND_SWA && (d->m < 1 || d->m > 128)) return false;
  if (d->n_heads < 1 || d->n_heads > 64) return false;
  if (d->window < 1 || d->window > 4096) return false;
  if (d->kind == LCA_KIND_CSA) {
    if (d->idx_heads < 1 || d->idx_heads > 8) return false;
    if (d->topk < 1 || d->topk > 2048) return false;
  }
  return true;
}

int32_t tail_width(const lca_layer_desc* d) {
  return d->kind == LCA_KIND_CSA ? 384 : (d->kind == LCA_KIND_HCA ? 256 : 0);
}

// tokens per compressed entry; the window-only layer has no compressed stream (no blocks at any m)
int64_t pool_m(const lca_layer_desc* d) { return d->kind == LCA_KIND_SWA ? 1 : d->m; }
int64_t n_blocks_max(const lca_layer_desc* d, int64_t max_ctx) {
  return d->kind == LCA_KIND_SWA ? 0 : max_ctx / d->m;
}

struct Layout {
  size_t blk_codes, blk_scale, blk_rope, idx_codes, idx_scale, win_codes, win_scale, win_rope, tail, inv_freq, total;
};

Layout layout(const lca_layer_desc* d, int32_t B, int64_t max_ctx, int32_t ring) {
  Layout L{};
  const size_t nb = (size_t)B * (size_t)n_blocks_max(d, max_ctx);
  const size_t nw = (size_t)B * (size_t)ring;
  size_t off = 0;
  L.blk_codes = off; off = align_up(off + nb * 64);
  L.blk_scale = off; off = align_up(off + nb * 4);
  L.blk_rope = off; off = align_up(off + nb * 128);
  if (d->kind == LCA_KIND_CSA) {
    L.idx_codes = off; off = align_up(off + nb * 32);
    L.idx_scale = off; off = align_up(off + nb * 2);
  }
  L.win_codes = off; off = align_up(off + nw * 64);
  L.win_scale = off; off = align_up(off + nw * 4);
  L.win_rope = off; off = align_up(off + nw * 128);
  L.tail = off; off = align_up(off + (size_t)B * pool_m(d) * tail_width(d) * 2);
  L.inv_freq = off; off = align_up(off + 32 * sizeof(double));
  L.total = off;
  return L;
}

bool sizes_ok(const lca_layer_desc* d, int32_t B, int64_t max_ctx, int32_t ring) {
  if (B < 1 || B > 65535) return false;
  if (max_ctx < pool_m(d) || max_ctx > ((int64_t)1 << 32)) return false;
  if (n_blocks_max(d, max_ctx) > kMaxBlocks) return false;  // scan segments per query fit the selection's LDS
  if (ring < d->window || ring > (1 << 24)) return false;
  return true;
}

// Workspace: the one-launch attention's (query, head group) counters first (fixed size and place: they
// must be zero between calls), then, for CSA, one block per query (histogram, scan segment counts,
// score keys, candidates), then the attention's split partials. The counters' and the per-query
// blocks' places do not depend on a call's Tq, so what must be zero between calls stays put.
struct WsLayout {
  size_t cnt, qbase, qstride, off_seg, off_keys, off_cand, off_sync, off_list, off_rec, part, total;
  int32_t G2;
};

WsLayout ws_layout(const lca_layer_desc* d, int32_t B, int32_t max_tq, int64_t max_ctx) {
  WsLayout W{};
  const int64_t max_blocks = n_blocks_max(d, max_ctx);
  const size_t nq = (size_t)B * (size_t)max_tq;
  // the attention's (query, group) counters, then its key splits' partials, then the per-query blocks: no
  // offset depends on the call's Tq, so calls with different query counts share one workspace (the
  // per-query state a call leaves zero stays where the next call looks for it)
  W.cnt = 0;
  W.part = align_up(kAttendCounterBytes);
  size_t off = align_up(W.part + (size_t)kAttendMaxWGs * sizeof(AttendPartial));
  W.qbase = off;
  W.G2 = (int32_t)((max_blocks + kScanPerWG - 1) / kScanPerWG);
  if (d->kind == LCA_KIND_CSA) {
    size_t q = align_up((size_t)kHistBins * 4);
    // segment counts: kScanPerWG blocks per scan segment, kTileSeg per query-tile segment, kScoreChunk per
    // in-launch-threshold segment
    const int64_t tile_blocks = max_blocks < kTileMaxBlocks ? max_blocks : kTileMaxBlocks;
    const int64_t n_seg = std::max<int64_t>({(int64_t)W.G2, (tile_blocks + kTileSeg - 1) / kTileSeg,
                                             (max_blocks + kScoreChunk - 1) / kScoreChunk});
    W.off_seg = q; q = align_up(q + (size_t)n_seg * 4);
    W.off_keys = q; q = align_up(q + (size_t)max_blocks * 4);
    W.off_cand = q; q = align_up(q + (size_t)max_blocks * 8);
    W.off_sync = q; q = align_up(q + kSyncBytes);             // the in-launch threshold's counter, ready word
    W.off_list = q; q = align_up(q + (size_t)kMaxTopk * 4);   // its top-k list, read by the attention
    W.off_rec = q; q = align_up(q + ((size_t)kRecHdrSlots + (size_t)n_seg * kRecMaxWords) * 8);  // its records
    W.qstride = q;
    off += nq * q;
  }
  // (partials exist only with splits, and then (query, group, split) triples number <= kAttendMaxWGs)
  W.total = align_up(off);
  return W;
}

// Key splits of the one-launch attention: none for up to 768 keys, else about one 32-key chunk per
// wave (8 waves per workgroup), within kAttendMaxWGs workgroups per call. n_keys: the most keys a query of the call attends.
int32_t attend_splits(int32_t nq, int32_t H, int64_t n_keys) {
  const int64_t groups = (H + 15) / 16;
  const int64_t chunks = (n_keys + 31) / 32;
  // up to 3 chunks per wave the partials and the merge cost more than the split saves (and without splits
  // a wave's chunks beyond kRound take a second round of gathers, which costs more than the merge)
  if (chunks <= kAttendNoSplitChunks * 8) return 1;
  int64_t s = (chunks + 7) / 8;
  const int64_t cap = kAttendMaxWGs / (nq * groups);
  if (s > cap) s = cap;
  return (int32_t)(s < 1 ? 1 : (s > kAttendMaxSplits ? kAttendMaxSplits : s));
}

void attend_workspace(AttendArgs* args, const lca_cache* c, int32_t Tq, void* ws_dev, size_t ws_bytes) {
  args->splits = 1;
  if (!ws_dev) return;
  WsLayout W = ws_layout(&c->desc, c->batch, Tq, c->max_ctx);
  if (ws_bytes < W.total) return;
  const int64_t N_last = c->max_blocks > 0 ? c->len / c->desc.m : 0;  // visible blocks of the last query (the most)
  const int64_t n_list = c->desc.kind == LCA_KIND_CSA ? (N_last < c->desc.topk ? N_last : c->desc.topk) : N_last;
  const int64_t n_win = c->len < c->desc.window ? c->len : c->desc.window;
  args->splits = attend_splits(c->batch * Tq, c->desc.n_heads, n_list + n_win);
  args->part = (AttendPartial*)((char*)ws_dev + W.part);
  args->cnt = (uint32_t*)((char*)ws_dev + W.cnt);
}

lca_status launch_status(hipError_t e) { return e == hipSuccess ? LCA_OK : LCA_ERR_LAUNCH; }

bool cache_ok(const lca_cache* c) {
  if (!c || !desc_ok(&c->desc) || !c->win_codes_dev || !c->win_scale_dev || !c->win_rope_dev) return false;
  if (c->desc.kind == LCA_KIND_SWA) return c->max_blocks == 0 && c->desc.m == 1;
  return c->blk_codes_dev && c->tail_dev;
}

IngestArgs ingest_args(lca_cache* c, const uint16_t* kv, const uint16_t* gate, const uint16_t* ik,
                       const uint16_t* ig, int32_t T) {
  IngestArgs a{};
  a.kv = kv;
  a.gate = gate;
  a.ik = ik;
  a.ig = ig;
  a.blk_codes = c->blk_codes_dev;
  a.blk_scale = c->blk_scale_dev;
  a.blk_rope = c->blk_rope_dev;
  a.idx_codes = c->idx_codes_dev;
  a.idx_scale = c->idx_scale_dev;
  a.win_codes = c->win_codes_dev;
  a.win_scale = c->win_scale_dev;
  a.win_rope = c->win_rope_dev;
  a.tail = c->tail_dev;
  a.len = c->len;
  a.max_blocks = c->max_blocks;
  a.T = T;
  a.m = c->desc.m;
  a.ring = c->ring;
  a.tail_width = c->tail_width;
  a.B = c->batch;
  a.inv_freq = c->rope_inv_freq_dev;
  return a;
}

lca_status compress_impl(lca_cache* c, bool csa, const uint16_t* kv, const uint16_t* gate, const uint16_t* ik,
                         const uint16_t* ig, const float* bias, const float* idx_bias, int32_t T, void* stream) {
  if (!cache_ok(c) || !kv || !gate || !bias) return LCA_ERR_NULL;
  if (csa ? c->desc.kind != LCA_KIND_CSA : c->desc.kind != LCA_KIND_HCA) return LCA_ERR_UNSUPPORTED;
  if (csa && (!ik || !ig || !idx_bias || !c->idx_codes_dev || !c->idx_scale_dev)) return LCA_ERR_NULL;
  if (T < 1) return LCA_ERR_SHAPE;
  if (c->pending != 0 || c->ragged) return LCA_ERR_ORDER;
  if (c->len + T > c->max_ctx) return LCA_ERR_CAPACITY;
  IngestArgs a = ingest_args(c, kv, gate, ik, ig, T);
  a.bias = bias;
  a.idx_bias = idx_bias;
  const int64_t m = c->desc.m;
  a.first = c->len / m;
  const int64_t n_blocks = (c->len + T) / m - c->len / m;
  hipError_t e = launch_compress(a, csa, n_blocks, (hipStream_t)stream);
  if (e != hipSuccess) return LCA_ERR_LAUNCH;
  c->pending = T;
  return LCA_OK;
}

}  // namespace

extern "C" {

const char* lca_status_str(lca_status s) {
  switch (s) {
    case LCA_OK: return "ok";
    case LCA_ERR_NULL: return "null pointer";
    case LCA_ERR_SHAPE: return "size out of range";
    case LCA_ERR_UNSUPPORTED: return "unsupported descriptor";
    case LCA_ERR_CAPACITY: return "cache or window state too small";
    case LCA_ERR_ORDER: return "compress / append out of order";
    case LCA_ERR_WORKSPACE: return "workspace missing or too small";
    case LCA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t lca_cache_bytes(const lca_layer_desc* desc, int32_t batch, int64_t max_ctx, int32_t ring) {
  if (!desc_ok(desc) || !sizes_ok(desc, batch, max_ctx, ring)) return 0;
  return layout(desc, batch, max_ctx, ring).total;
}

lca_status lca_cache_bind(const lca_layer_desc* desc, lca_cache* cache, void* base_dev, size_t bytes, int32_t batch,
                          int64_t max_ctx, int32_t ring, void* stream) {
  if (!desc || !cache || !base_dev) return LCA_ERR_NULL;
  if (!desc_ok(desc)) return LCA_ERR_UNSUPPORTED;
  if (!sizes_ok(desc, batch, max_ctx, ring)) return LCA_ERR_SHAPE;
  if (((uintptr_t)base_dev) % kAlign != 0) return LCA_ERR_SHAPE;
  Layout L = layout(desc, batch, max_ctx, ring);
  if (bytes < L.total) return LCA_ERR_CAPACITY;
  std::memset(cache, 0, sizeof(*cache));
  cache->desc = *desc;
  if (desc->kind != LCA_KIND_CSA) {
    cache->desc.idx_heads = 0;
    cache->desc.topk = 0;
  }
  const bool swa = desc->kind == LCA_KIND_SWA;
  if (swa) cache->desc.m = 1;
  cache->batch = batch;
  cache->ring = ring;
  cache->max_ctx = max_ctx;
  cache->max_blocks = n_blocks_max(desc, max_ctx);
  char* base = (char*)base_dev;
  if (!swa) {
    cache->blk_codes_dev = (uint8_t*)(base + L.blk_codes);
    cache->blk_scale_dev = (float*)(base + L.blk_scale);
    cache->blk_rope_dev = (uint16_t*)(base + L.blk_rope);
    cache->tail_dev = (uint16_t*)(base + L.tail);
  }
  if (desc->kind == LCA_KIND_CSA) {
    cache->idx_codes_dev = (uint8_t*)(base + L.idx_codes);
    cache->idx_scale_dev = (uint8_t*)(base + L.idx_scale);
  }
  cache->win_codes_dev = (uint8_t*)(base + L.win_codes);
  cache->win_scale_dev = (float*)(base + L.win_scale);
  cache->win_rope_dev = (uint16_t*)(base + L.win_rope);
  cache->tail_width = tail_width(desc);
  for (int i = 0; i < 32; ++i) cache->rope_inv_freq[i] = std::pow(10000.0, -(double)(2 * i) / 64.0);
  cache->rope_inv_freq_dev = (double*)(base + L.inv_freq);
  if (launch_fill_zero(base_dev, L.total, (hipStream_t)stream) != hipSuccess) return LCA_ERR_LAUNCH;
  // the kernels read the frequencies from this device copy (kept out of every launch's arguments)
  return launch_status(hipMemcpyAsync(cache->rope_inv_freq_dev, cache->rope_inv_freq, 32 * sizeof(double),
                                      hipMemcpyHostToDevice, (hipStream_t)stream));
}

size_t lca_workspace_scores_offset(const lca_layer_desc* desc, int32_t batch, int32_t query, int64_t max_ctx) {
  if (!desc_ok(desc) || desc->kind != LCA_KIND_CSA || batch < 1 || query < 0 || max_ctx < desc->m) return 0;
  WsLayout W = ws_layout(desc, batch, 1, max_ctx);
  return W.qbase + (size_t)query * W.qstride + W.off_keys;
}

size_t lca_workspace_bytes(const lca_layer_desc* desc, int32_t batch, int32_t max_tq, int64_t max_ctx) {
  if (!desc_ok(desc) || batch < 1 || max_tq < 1 || max_ctx < pool_m(desc)) return 0;
  return ws_layout(desc, batch, max_tq, max_ctx).total;
}

lca_status lca_workspace_init(void* ws_dev, size_t bytes, void* stream) {
  if (!ws_dev) return LCA_ERR_NULL;
  if (((uintptr_t)ws_dev) % kAlign != 0 || bytes % 16 != 0) return LCA_ERR_SHAPE;
  return launch_status(launch_fill_zero(ws_dev, bytes, (hipStream_t)stream));
}

lca_status lca_csa_compress(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                            const uint16_t* ik_dev, const uint16_t* ig_dev, const float* bias_dev,
                            const float* idx_bias_dev, int32_t T, void* stream) {
  return compress_impl(cache, true, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, T, stream);
}

lca_status lca_hca_compress(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                            const float* bias_dev, int32_t T, void* stream) {
  return compress_impl(cache, false, kv_dev, gate_dev, nullptr, nullptr, bias_dev, nullptr, T, stream);
}

lca_status lca_swa_tail_append(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                               const uint16_t* ik_dev, const uint16_t* ig_dev, int32_t T, void* stream) {
  if (!cache_ok(cache) || !kv_dev) return LCA_ERR_NULL;
  const bool csa = cache->desc.kind == LCA_KIND_CSA, swa = cache->desc.kind == LCA_KIND_SWA;
  if (!swa && !gate_dev) return LCA_ERR_NULL;
  if (csa && (!ik_dev || !ig_dev)) return LCA_ERR_NULL;
  if (T < 1) return LCA_ERR_SHAPE;
  if (cache->ragged || cache->pending != (swa ? 0 : T)) return LCA_ERR_ORDER;  // the window-only layer has no compressor
  if (cache->len + T > cache->max_ctx) return LCA_ERR_CAPACITY;
  IngestArgs a = ingest_args(cache, kv_dev, gate_dev, csa ? ik_dev : nullptr, csa ? ig_dev : nullptr, T);
  const int64_t end = cache->len + T;
  const int64_t win_first = (end - cache->ring > cache->len) ? end - cache->ring : cache->len;
  a.first = win_first;
  a.n_win = (int32_t)(end - win_first);
  int64_t tail_first = (end / cache->desc.m) * cache->desc.m;
  if (tail_first < cache->len) tail_first = cache->len;
  const int32_t n_tail = swa ? 0 : (int32_t)(end - tail_first);
  hipError_t e = launch_append(a, csa, n_tail, (hipStream_t)stream);
  if (e != hipSuccess) return LCA_ERR_LAUNCH;
  cache->len = end;
  cache->pending = 0;
  return LCA_OK;
}

}  // extern "C"

namespace {

// compute units of the current device, read once per device
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

lca_status score_args(lca_cache* cache, const uint16_t* qI_dev, const float* w_dev, bool need_q, int32_t Tq,
                      int32_t* topk_dev, bool need_topk, void* ws_dev, size_t ws_bytes, ScoreArgs* out) {
  if (!cache_ok(cache)) return LCA_ERR_NULL;
  if (need_q && (!qI_dev || !w_dev)) return LCA_ERR_NULL;
  if (need_topk && !topk_dev) return LCA_ERR_NULL;
  if (cache->desc.kind != LCA_KIND_CSA || !cache->idx_codes_dev) return LCA_ERR_UNSUPPORTED;
  if (Tq < 1 || Tq > cache->len) return LCA_ERR_SHAPE;
  if ((int64_t)cache->batch * Tq > kMaxGridY) return LCA_ERR_SHAPE;  // queries index grid.y
  if (cache->pending != 0 || cache->ragged) return LCA_ERR_ORDER;
  if (!ws_dev) return LCA_ERR_WORKSPACE;
  WsLayout W = ws_layout(&cache->desc, cache->batch, Tq, cache->max_ctx);
  if (ws_bytes < W.total) return LCA_ERR_WORKSPACE;
  ScoreArgs a{};
  char* ws = (char*)ws_dev;
  a.qI = qI_dev;
  a.w = w_dev;
  a.idx_codes = cache->idx_codes_dev;
  a.idx_scale = cache->idx_scale_dev;
  a.qbase = (uint8_t*)(ws + W.qbase);
  a.qstride = W.qstride;
  a.off_seg = W.off_seg;
  a.off_keys = W.off_keys;
  a.off_cand = W.off_cand;
  a.off_sync = W.off_sync;
  a.off_list = W.off_list;
  a.off_rec = W.off_rec;
  a.topk = topk_dev;
  a.len = cache->len;
  a.max_blocks = cache->max_blocks;
  a.Tq = Tq;
  a.HI = cache->desc.idx_heads;
  a.k = cache->desc.topk;
  a.m = cache->desc.m;
  a.G2 = W.G2;
  {
    // score workgroups of the last query: one per chunk, or, with many queries, one per kMultiChunks
    const int64_t g1 = (a.len / a.m + kScoreChunk - 1) / kScoreChunk;  // score chunks of the last query
    int64_t wgs = g1;
    a.chunk_step = 0;
    const int64_t nq = (int64_t)cache->batch * Tq;
    // query tiles: many queries, each seeing at most kTileMaxBlocks blocks (the last query sees the most)
    a.tiles = nq >= kTileMinQueries && a.len / a.m <= kTileMaxBlocks ? 1 : 0;
    if (!a.tiles && nq >= kMultiMinQueries) {
      wgs = (g1 + kMultiChunks - 1) / kMultiChunks;
      wgs = wgs < 1 ? 1 : wgs;
      a.chunk_step = (int32_t)wgs;
    } else if (!a.tiles && g1 >= 2) {
      // One workgroup per chunk runs as a single wave of workgroups when nq * g1 fits the compute units.
      // When only the last, at most half-full chunk column pushes it past that, workgroup 0 of each
      // query scores the last chunk after its own: a short second chunk instead of a second wave of
      // whole workgroups after the first has drained.
      const int64_t cap = (int64_t)kScoreWGsPerCU * device_cus();
      const int64_t tail = a.len / a.m - (g1 - 1) * kScoreChunk;
      if (nq * g1 > cap && nq * (g1 - 1) <= cap && tail <= kScoreChunk / 2) {
        wgs = g1 - 1;
        a.fold_tail = 1;
      }
    }
    // each workgroup counts at least cmin keys (twice its share of k) into the query's histogram
    const int64_t w = wgs > 0 ? wgs : 1;
    const int64_t cm = 2 * (((int64_t)a.k + w - 1) / w);
    a.cmin = (int32_t)(cm < 16 ? 16 : (cm > kCandCap ? kCandCap : cm));
  }
  *out = a;
  return LCA_OK;
}

// The in-launch threshold and selection for a decode-sized call's score launch: one score workgroup per
// chunk, every one of them counted in at its query's counter. Each workgroup's record carries its
// candidates down to where cmin = twice its share of k plus 16 still fit, which covers the query's winners
// unless a chunk holds far more than its share (then the last workgroup takes them from the key rows:
// exact, slower). Records of 32 to 256 words, as cmin needs; the last workgroup reads all of them at once
// (at most kPrefMaxLoads words per thread).
// The one-launch step (csa_step_kernel) takes a call whose attention splits hold at most kStepListMax
// slots each; LCA_STEP_UNFUSED in the environment keeps the two-launch path (the same results).
bool step_fusable(const lca_cache* before, const lca_cache* after, const AttendArgs& args) {
  if (std::getenv("LCA_STEP_UNFUSED")) return false;
  if (args.splits > 1 && (!args.part || !args.cnt)) return false;
  const int64_t N_last = after->len / after->desc.m;
  const int64_t n_list = N_last < after->desc.topk ? N_last : after->desc.topk;
  const int64_t n_win = after->len < after->desc.window ? after->len : after->desc.window;
  const int64_t per_split = (n_list + n_win + args.splits * 16 - 1) / (args.splits * 16) * 16;
  (void)before;
  return per_split <= kStepListMax;
}

// A new nonzero token for every step launch (its lists' ready words compare against it)
uint32_t next_step_token() {
  static std::atomic<uint32_t> counter{0};
  uint32_t t = counter.fetch_add(1u, std::memory_order_relaxed) + 1u;
  if (t == 0u) t = counter.fetch_add(1u, std::memory_order_relaxed) + 1u;
  return t;
}

bool use_coop(ScoreArgs* a, int64_t nq) {
  if (a->tiles || a->chunk_step != 0) return false;
  const int64_t nb = a->len / a->m;  // the most blocks a query of the call sees
  const int64_t g1 = std::max<int64_t>(1, (nb + kScoreChunk - 1) / kScoreChunk);
  const int64_t cols = a->fold_tail ? g1 - 1 : g1;
  (void)nq;  // no workgroup waits for another: any number of them works
  if (g1 > kMaxSegs) return false;
  const int64_t cmin = 2 * ((a->k + cols - 1) / cols) + 16;
  int64_t R = kRecMinWords;
  while (R < cmin && R < kRecMaxWords) R *= 2;
  if (R < cmin || g1 > kRecHdrSlots || g1 * R > (int64_t)kPrefMaxLoads * kScoreThreads) return false;
  a->coop = 1;
  a->n_cols = (int32_t)cols;
  a->pref_slots = (int32_t)R;
  a->cmin = (int32_t)cmin;
  return true;
}

}  // namespace

extern "C" {

lca_status lca_csa_index_score(lca_cache* cache, const uint16_t* qI_dev, const float* w_dev, int32_t Tq,
                               void* ws_dev, size_t ws_bytes, void* stream) {
  ScoreArgs a;
  lca_status st = score_args(cache, qI_dev, w_dev, true, Tq, nullptr, false, ws_dev, ws_bytes, &a);
  if (st != LCA_OK) return st;
  a.write_keys = 1;  // this call leaves every visible block's key in the workspace
  return launch_status(launch_index_score(a, cache->batch, (hipStream_t)stream));
}

lca_status lca_csa_topk_select(lca_cache* cache, int32_t Tq, int32_t* topk_dev, void* ws_dev, size_t ws_bytes,
                               void* stream) {
  ScoreArgs a;
  lca_status st = score_args(cache, nullptr, nullptr, false, Tq, topk_dev, true, ws_dev, ws_bytes, &a);
  if (st != LCA_OK) return st;
  return launch_status(launch_topk_select(a, cache->batch, (hipStream_t)stream));
}

lca_status lca_csa_indexer_topk(lca_cache* cache, const uint16_t* qI_dev, const float* w_dev, int32_t Tq,
                                int32_t* topk_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  ScoreArgs a;
  lca_status st = score_args(cache, qI_dev, w_dev, true, Tq, topk_dev, true, ws_dev, ws_bytes, &a);
  if (st != LCA_OK) return st;
  if (use_coop(&a, (int64_t)cache->batch * Tq)) {  // scores, bound, candidates and selection in one launch
    ScanArgs sa{};
    sa.a = a;
    return launch_status(launch_index_select(sa, cache->batch, (hipStream_t)stream));
  }
  a.tile_select = a.tiles;  // query tiles select in the score launch itself
  hipError_t e = launch_index_score(a, cache->batch, (hipStream_t)stream);
  if (e != hipSuccess) return LCA_ERR_LAUNCH;
  return launch_status(launch_topk_select(a, cache->batch, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// kind: the layer kind the entry point serves; dense = every visible block (HCA) or none (SWA: no blocks)
lca_status attn_args(lca_cache* cache, int32_t kind, const uint16_t* q_dev, const int32_t* topk_dev, int32_t Tq,
                     uint16_t* out_dev, float* lse_dev, AttnArgs* out) {
  if (!cache_ok(cache) || !q_dev || !out_dev) return LCA_ERR_NULL;
  if (cache->desc.kind != kind) return LCA_ERR_UNSUPPORTED;
  const bool dense = kind != LCA_KIND_CSA;
  if (Tq < 1 || Tq > cache->len) return LCA_ERR_SHAPE;
  if (cache->pending != 0 || cache->ragged) return LCA_ERR_ORDER;
  if ((int64_t)Tq + cache->desc.window - 1 > cache->ring) return LCA_ERR_CAPACITY;
  AttnArgs a{};
  a.q = q_dev;
  a.topk = dense ? nullptr : topk_dev;
  // SWA: max_blocks = 0, so no query sees a block; the block arrays alias the window's, never read
  const bool swa = kind == LCA_KIND_SWA;
  a.blk_codes = swa ? cache->win_codes_dev : cache->blk_codes_dev;
  a.blk_scale = swa ? cache->win_scale_dev : cache->blk_scale_dev;
  a.blk_rope = swa ? cache->win_rope_dev : cache->blk_rope_dev;
  a.win_codes = cache->win_codes_dev;
  a.win_scale = cache->win_scale_dev;
  a.win_rope = cache->win_rope_dev;
  a.out = out_dev;
  a.lse = lse_dev;
  a.len = cache->len;
  a.max_blocks = cache->max_blocks;
  a.Tq = Tq;
  a.H = cache->desc.n_heads;
  a.k = dense ? 0 : cache->desc.topk;
  a.m = cache->desc.m;
  a.W = cache->desc.window;
  a.ring = cache->ring;
  a.dense = dense ? 1 : 0;
  a.inv_freq = cache->rope_inv_freq_dev;
  *out = a;
  return LCA_OK;
}

// Few queries: a workgroup per (query, 16 heads) over all keys (attend.hip). Many queries: a
// workgroup per query and all heads (attention.hip).
lca_status attention_impl(lca_cache* cache, int32_t kind, const uint16_t* q_dev, const int32_t* topk_dev,
                          int32_t Tq, uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes,
                          void* stream) {
  const bool dense = kind != LCA_KIND_CSA;
  if (!dense && !topk_dev) return LCA_ERR_NULL;
  AttnArgs a;
  lca_status st = attn_args(cache, kind, q_dev, topk_dev, Tq, out_dev, lse_dev, &a);
  if (st != LCA_OK) return st;
  const int32_t nq = cache->batch * Tq;
  hipStream_t s = (hipStream_t)stream;
  if (nq <= kAttendMaxQueries) {
    AttendArgs args{};
    args.t = a;
    attend_workspace(&args, cache, Tq, ws_dev, ws_bytes);
    return launch_status(launch_attend(args, cache->batch, dense ? kAttendDense : kAttendList, s));
  }
  return launch_status(launch_attention(a, cache->batch, s));
}

// One decode step of a dense layer (HCA: compress when blocks complete, then attention with the append
// in the same launch; window-only: the append in the attention launch). Every check before any launch.
lca_status dense_step_impl(lca_cache* cache, int32_t kind, const uint16_t* kv_dev, const uint16_t* gate_dev,
                           const float* bias_dev, int32_t T, const uint16_t* q_dev, uint16_t* out_dev,
                           float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  const bool hca = kind == LCA_KIND_HCA;
  if (!cache_ok(cache) || !kv_dev || !q_dev || !out_dev || (hca && (!gate_dev || !bias_dev))) return LCA_ERR_NULL;
  if (cache->desc.kind != kind) return LCA_ERR_UNSUPPORTED;
  if (T < 1 || (int64_t)cache->batch * T > kAttendMaxQueries) return LCA_ERR_SHAPE;
  if (cache->pending != 0 || cache->ragged) return LCA_ERR_ORDER;
  if (cache->len + T > cache->max_ctx) return LCA_ERR_CAPACITY;
  lca_cache after = *cache;  // the cache once the T tokens are in: what the queries see
  after.len = cache->len + T;
  AttendArgs args{};
  lca_status st = attn_args(&after, kind, q_dev, nullptr, T, out_dev, lse_dev, &args.t);
  if (st != LCA_OK) return st;
  attend_workspace(&args, &after, T, ws_dev, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  const int64_t m = cache->desc.m;
  const int64_t end = cache->len + T;
  if (hca) {
    const int64_t n_blocks = end / m - cache->len / m;
    if (n_blocks > 0) {
      IngestArgs ca = ingest_args(cache, kv_dev, gate_dev, nullptr, nullptr, T);
      ca.bias = bias_dev;
      ca.first = cache->len / m;
      if (launch_compress(ca, false, n_blocks, s) != hipSuccess) return LCA_ERR_LAUNCH;
    }
  }
  IngestArgs app = ingest_args(cache, kv_dev, gate_dev, nullptr, nullptr, T);
  const int64_t win_first = (end - cache->ring > cache->len) ? end - cache->ring : cache->len;
  app.first = win_first;
  app.n_win = (int32_t)(end - win_first);
  int32_t n_tail = 0;
  if (hca) {
    int64_t tail_first = (end / m) * m;
    if (tail_first < cache->len) tail_first = cache->len;
    n_tail = (int32_t)(end - tail_first);
  }
  args.app = app;
  args.app_units = app.n_win + n_tail;
  if (launch_attend(args, cache->batch, kAttendDense, s) != hipSuccess) return LCA_ERR_LAUNCH;
  cache->len = end;
  cache->pending = 0;
  return LCA_OK;
}

lca_status topk_attn_impl(lca_cache* cache, const uint16_t* qI_dev, const float* w_dev, bool score,
                          const uint16_t* q_dev, int32_t Tq, int32_t* topk_dev, uint16_t* out_dev, float* lse_dev,
                          void* ws_dev, size_t ws_bytes, void* stream) {
  AttendArgs args{};
  lca_status st = score_args(cache, qI_dev, w_dev, score, Tq, topk_dev, false, ws_dev, ws_bytes, &args.s);
  if (st != LCA_OK) return st;
  st = attn_args(cache, LCA_KIND_CSA, q_dev, nullptr, Tq, out_dev, lse_dev, &args.t);
  if (st != LCA_OK) return st;
  attend_workspace(&args, cache, Tq, ws_dev, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (score && use_coop(&args.s, (int64_t)cache->batch * Tq)) {
    // one launch for scores, bound, candidates and each query's selection; the attention reads the lists
    ScanArgs sa{};
    sa.a = args.s;
    if (launch_index_select(sa, cache->batch, s) != hipSuccess) return LCA_ERR_LAUNCH;
    return launch_status(launch_attend(args, cache->batch, kAttendListWs, s));
  }
  if (score) {
    hipError_t e = launch_index_score(args.s, cache->batch, s);
    if (e != hipSuccess) return LCA_ERR_LAUNCH;
  }
  hipError_t e = launch_topk_select(args.s, cache->batch, s, false);
  if (e != hipSuccess) return LCA_ERR_LAUNCH;
  return launch_status(launch_attend(args, cache->batch, kAttendSelect, s));
}

}  // namespace

extern "C" {

lca_status lca_csa_sparse_attn(lca_cache* cache, const uint16_t* q_dev, const int32_t* topk_dev, int32_t Tq,
                               uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return attention_impl(cache, LCA_KIND_CSA, q_dev, topk_dev, Tq, out_dev, lse_dev, ws_dev, ws_bytes, stream);
}

lca_status lca_hca_dense_attn(lca_cache* cache, const uint16_t* q_dev, int32_t Tq, uint16_t* out_dev,
                              float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return attention_impl(cache, LCA_KIND_HCA, q_dev, nullptr, Tq, out_dev, lse_dev, ws_dev, ws_bytes, stream);
}

lca_status lca_swa_attn(lca_cache* cache, const uint16_t* q_dev, int32_t Tq, uint16_t* out_dev, float* lse_dev,
                        void* ws_dev, size_t ws_bytes, void* stream) {
  return attention_impl(cache, LCA_KIND_SWA, q_dev, nullptr, Tq, out_dev, lse_dev, ws_dev, ws_bytes, stream);
}

lca_status lca_hca_step(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev, const float* bias_dev,
                        int32_t T, const uint16_t* q_dev, uint16_t* out_dev, float* lse_dev, void* ws_dev,
                        size_t ws_bytes, void* stream) {
  return dense_step_impl(cache, LCA_KIND_HCA, kv_dev, gate_dev, bias_dev, T, q_dev, out_dev, lse_dev, ws_dev,
                         ws_bytes, stream);
}

lca_status lca_swa_step(lca_cache* cache, const uint16_t* kv_dev, int32_t T, const uint16_t* q_dev,
                        uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return dense_step_impl(cache, LCA_KIND_SWA, kv_dev, nullptr, nullptr, T, q_dev, out_dev, lse_dev, ws_dev,
                         ws_bytes, stream);
}

lca_status lca_csa_topk_attn(lca_cache* cache, const uint16_t* q_dev, int32_t Tq, int32_t* topk_dev,
                             uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return topk_attn_impl(cache, nullptr, nullptr, false, q_dev, Tq, topk_dev, out_dev, lse_dev, ws_dev, ws_bytes,
                        stream);
}

}  // extern "C"

namespace {

// The shape checks of a CSA decode step (every one before any launch).
lca_status csa_step_check(const lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                          const uint16_t* ik_dev, const uint16_t* ig_dev, const float* bias_dev,
                          const float* idx_bias_dev, int32_t T) {
  if (!cache_ok(cache) || !kv_dev || !gate_dev || !ik_dev || !ig_dev || !bias_dev || !idx_bias_dev)
    return LCA_ERR_NULL;
  if (cache->desc.kind != LCA_KIND_CSA || !cache->idx_codes_dev) return LCA_ERR_UNSUPPORTED;
  if (T < 1 || (int64_t)cache->batch * T > kAttendMaxQueries) return LCA_ERR_SHAPE;
  if (cache->pending != 0 || cache->ragged) return LCA_ERR_ORDER;
  if (cache->len + T > cache->max_ctx) return LCA_ERR_CAPACITY;
  return LCA_OK;
}

lca_status csa_step_impl(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev, const uint16_t* ik_dev,
                         const uint16_t* ig_dev, const float* bias_dev, const float* idx_bias_dev, int32_t T,
                         const uint16_t* qI_dev, const float* w_dev, const uint16_t* q_dev, int32_t* topk_dev,
                         uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream,
                         void* const* ev, int32_t* plan = nullptr) {
  // every check first, so a rejected call leaves the cache as it was
  lca_status st = csa_step_check(cache, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, T);
  if (st != LCA_OK) return st;
  lca_cache after = *cache;  // the cache once the T tokens are in: what the query kernels see
  after.len = cache->len + T;
  AttendArgs args{};
  st = score_args(&after, qI_dev, w_dev, true, T, topk_dev, false, ws_dev, ws_bytes, &args.s);
  if (st != LCA_OK) return st;
  st = attn_args(&after, LCA_KIND_CSA, q_dev, nullptr, T, out_dev, lse_dev, &args.t);
  if (st != LCA_OK) return st;
  attend_workspace(&args, &after, T, ws_dev, ws_bytes);
  const bool coop = use_coop(&args.s, (int64_t)cache->batch * T);
  const bool one_launch = coop && step_fusable(cache, &after, args);
  if (plan) {  // the launches the step takes after the compress, nothing launched
    *plan = one_launch ? 1 : coop ? 2 : 3;
    return LCA_OK;
  }
  hipStream_t s = (hipStream_t)stream;
  // the timed variant's events: step start, indexer start, indexer end, attention end
  auto mark = [&](int i) { return !ev || !ev[i] || hipEventRecord((hipEvent_t)ev[i], s) == hipSuccess; };
  const int64_t m = cache->desc.m;
  if (!mark(0)) return LCA_ERR_LAUNCH;
  // compress the blocks the T tokens complete (their keys are scored below)
  const int64_t n_blocks = (cache->len + T) / m - cache->len / m;
  if (n_blocks > 0) {
    IngestArgs ca = ingest_args(cache, kv_dev, gate_dev, ik_dev, ig_dev, T);
    ca.bias = bias_dev;
    ca.idx_bias = idx_bias_dev;
    ca.first = cache->len / m;
    if (launch_compress(ca, true, n_blocks, s) != hipSuccess) return LCA_ERR_LAUNCH;
  }
  // the append (window entries, tail): a row of the score launch (in-launch threshold) or of the
  // candidate-scan launch; the attention after them reads the new window entries
  IngestArgs app = ingest_args(cache, kv_dev, gate_dev, ik_dev, ig_dev, T);
  const int64_t end = cache->len + T;
  const int64_t win_first = (end - cache->ring > cache->len) ? end - cache->ring : cache->len;
  app.first = win_first;
  app.n_win = (int32_t)(end - win_first);
  int64_t tail_first = (end / m) * m;
  if (tail_first < cache->len) tail_first = cache->len;
  const int32_t units = app.n_win + (int32_t)(end - tail_first);
  if (coop) {
    if (one_launch) {
      // one launch: the score workgroups (scores, records, the selection by the last of each query), then
      // the attention workgroups over the lists (and the append)
      StepArgs sa{};
      sa.idx.a = args.s;
      sa.att = args;
      sa.att.app = app;
      sa.att.app_units = units;
      sa.token = next_step_token();
      sa.n_queries = cache->batch * T;
      sa.n_idx = (sa.n_queries * args.s.n_cols + 7) / 8 * 8;
      sa.n_att = sa.n_queries * ((after.desc.n_heads + 15) / 16) * args.splits;
      if (!mark(1)) return LCA_ERR_LAUNCH;
      if (launch_csa_step(sa, s) != hipSuccess) return LCA_ERR_LAUNCH;
      if (!mark(2) || !mark(3)) return LCA_ERR_LAUNCH;
      cache->len = end;
      cache->pending = 0;
      return LCA_OK;
    }
    // two launches: scores + bound + candidates + selection (+ the append), then the attention
    ScanArgs sa{};
    sa.a = args.s;
    sa.app = app;
    sa.app_units = units;
    if (!mark(1)) return LCA_ERR_LAUNCH;
    if (launch_index_select(sa, cache->batch, s) != hipSuccess) return LCA_ERR_LAUNCH;
    if (!mark(2)) return LCA_ERR_LAUNCH;
    if (launch_attend(args, cache->batch, kAttendListWs, s) != hipSuccess) return LCA_ERR_LAUNCH;
    if (!mark(3)) return LCA_ERR_LAUNCH;
    cache->len = end;
    cache->pending = 0;
    return LCA_OK;
  }
  if (!mark(1)) return LCA_ERR_LAUNCH;
  if (launch_index_score(args.s, cache->batch, s) != hipSuccess) return LCA_ERR_LAUNCH;
  if (launch_topk_select(args.s, cache->batch, s, false, &app, units) != hipSuccess) return LCA_ERR_LAUNCH;
  if (!mark(2)) return LCA_ERR_LAUNCH;
  if (launch_attend(args, cache->batch, kAttendSelect, s) != hipSuccess) return LCA_ERR_LAUNCH;
  if (!mark(3)) return LCA_ERR_LAUNCH;
  cache->len = end;
  cache->pending = 0;
  return LCA_OK;
}

// ---- the CSA decode step without a caller workspace: for callers that cannot allocate (code under HIP
// graph capture, tight serving loops). Its workspace is this file-scope device array, one per GPU the
// library runs on, held until the process ends. Host code never uses the array's name as an address
// (on the host it is only a stand-in for the symbol): the device address comes from hipGetSymbolAddress,
// once per device, and every kernel gets that pointer.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

struct StaticScratch {
  std::mutex mu;
  void* ptr = nullptr;        // the device's address of `scratch`
  uint64_t layout_key = 0;    // workspace layout of the last call on the device (0: none yet)
};
StaticScratch g_scratch[64];

// The device address of `scratch` on the current device, zeroed at its first use; a call whose workspace
// layout differs from the previous call's re-zeroes the bytes it uses (the histograms and counters it
// needs zero sit where the last layout kept other data). Both fills are kernels on `stream`.
lca_status static_scratch(const lca_cache* cache, int32_t T, hipStream_t stream, void** out) {
  const WsLayout W = ws_layout(&cache->desc, cache->batch, T, cache->max_ctx);
  if (W.total > kStaticScratchBytes) return LCA_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return LCA_ERR_LAUNCH;
  StaticScratch& S = g_scratch[dev];
  std::lock_guard<std::mutex> lock(S.mu);
  if (!S.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LCA_ERR_LAUNCH;
    if (launch_fill_zero(p, kStaticScratchBytes, stream) != hipSuccess) return LCA_ERR_LAUNCH;
    S.ptr = p;
  }
  const uint64_t key = ((uint64_t)W.qstride << 20) ^ ((uint64_t)W.total << 1) ^ 1u;
  if (S.layout_key != key) {
    if (launch_fill_zero(S.ptr, W.total, stream) != hipSuccess) return LCA_ERR_LAUNCH;
    S.layout_key = key;
  }
  *out = S.ptr;
  return LCA_OK;
}

}  // namespace

extern "C" {

lca_status lca_csa_step(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev, const uint16_t* ik_dev,
                        const uint16_t* ig_dev, const float* bias_dev, const float* idx_bias_dev, int32_t T,
                        const uint16_t* qI_dev, const float* w_dev, const uint16_t* q_dev, int32_t* topk_dev,
                        uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return csa_step_impl(cache, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, T, qI_dev, w_dev, q_dev,
                       topk_dev, out_dev, lse_dev, ws_dev, ws_bytes, stream, nullptr);
}

lca_status lca_csa_step_launches(const lca_cache* cache, int32_t T, void* ws_dev, size_t ws_bytes,
                                 int32_t* launches) {
  if (!cache || !launches) return LCA_ERR_NULL;
  // the step's own checks and plan, on a copy of the cache, with stand-in inputs that nothing reads
  static uint16_t in16[1];
  static float in32[1];
  static int32_t topk[1];
  lca_cache c = *cache;
  return csa_step_impl(&c, in16, in16, in16, in16, in32, in32, T, in16, in32, in16, topk, in16, nullptr, ws_dev,
                       ws_bytes, nullptr, nullptr, launches);
}

lca_status lca_csa_step_timed(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                              const uint16_t* ik_dev, const uint16_t* ig_dev, const float* bias_dev,
                              const float* idx_bias_dev, int32_t T, const uint16_t* qI_dev, const float* w_dev,
                              const uint16_t* q_dev, int32_t* topk_dev, uint16_t* out_dev, float* lse_dev,
                              void* ws_dev, size_t ws_bytes, void* stream, void* const* events) {
  if (!events) return LCA_ERR_NULL;
  return csa_step_impl(cache, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, T, qI_dev, w_dev, q_dev,
                       topk_dev, out_dev, lse_dev, ws_dev, ws_bytes, stream, events);
}

lca_status lca_csa_step_noalloc(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                                const uint16_t* ik_dev, const uint16_t* ig_dev, const float* bias_dev,
                                const float* idx_bias_dev, int32_t T, const uint16_t* qI_dev, const float* w_dev,
                                const uint16_t* q_dev, int32_t* topk_dev, uint16_t* out_dev, float* lse_dev,
                                void* stream) {
  // the step's own checks first: a rejected call touches neither the cache nor the scratch
  lca_status st = csa_step_check(cache, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, T);
  if (st != LCA_OK) return st;
  if (!qI_dev || !w_dev) return LCA_ERR_NULL;
  void* ws = nullptr;
  lca_cache after = *cache;
  after.len = cache->len + T;
  st = static_scratch(&after, T, (hipStream_t)stream, &ws);
  if (st != LCA_OK) return st;
  return csa_step_impl(cache, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, T, qI_dev, w_dev, q_dev,
                       topk_dev, out_dev, lse_dev, ws, kStaticScratchBytes, stream, nullptr);
}

lca_status lca_csa_attend(lca_cache* cache, const uint16_t* qI_dev, const float* w_dev, const uint16_t* q_dev,
                          int32_t Tq, int32_t* topk_dev, uint16_t* out_dev, float* lse_dev, void* ws_dev,
                          size_t ws_bytes, void* stream) {
  return topk_attn_impl(cache, qI_dev, w_dev, true, q_dev, Tq, topk_dev, out_dev, lse_dev, ws_dev, ws_bytes,
                        stream);
}

}  // extern "C"

// ---------------------------------------------------------------- persistence
namespace {

constexpr int kSections = 9;

void snapshot_layout(int32_t kind, int32_t m, int32_t tw, int64_t len, int64_t n_win, lca_snapshot_info* I,
                     size_t* sizes = nullptr) {
  std::memset(I, 0, sizeof(*I));
  I->magic = LCA_SNAPSHOT_MAGIC;
  I->version = LCA_SNAPSHOT_VERSION;
  I->kind = kind;
  I->m = m;
  I->tail_width = tw;
  I->len = len;
  I->n_blocks = kind == LCA_KIND_SWA ? 0 : len / m;
  I->n_win = n_win;
  I->n_tail = kind == LCA_KIND_SWA ? 0 : len % m;
  const size_t nb = (size_t)I->n_blocks, nw = (size_t)n_win, nt = (size_t)I->n_tail;
  const bool csa = kind == LCA_KIND_CSA;
  const size_t sz[kSections] = {nb * 64, nb * 4, nb * 128, csa ? nb * 32 : 0, csa ? nb * 2 : 0,
                                nw * 64, nw * 4, nw * 128, nt * (size_t)tw * 2};
  size_t off = LCA_SNAPSHOT_HEADER;
  for (int i = 0; i < kSections; ++i) {
    I->off[i] = off;
    off = align_up(off + sz[i]);
    if (sizes) sizes[i] = sz[i];
  }
  I->off[kSections] = off;
  I->bytes = off;
}

void add_run(CopyArgs& a, const void* src, void* dst, uint64_t bytes, uint64_t src_stride, uint64_t dst_stride) {
  if (bytes == 0) return;
  if (a.n_runs >= kMaxCopyRuns) {  // at most 21 runs by construction; the launcher refuses an overflow
    a.n_runs = kMaxCopyRuns + 1;
    return;
  }
  CopyRun& r = a.run[a.n_runs++];
  r.src = (const uint8_t*)src;
  r.dst = (uint8_t*)dst;
  r.bytes = bytes;
  r.src_stride = src_stride;
  r.dst_stride = dst_stride;
}

// positions p0 .. p0+n-1 (n <= R) of a ring of R slots: at most two runs of consecutive slots
int ring_runs(int64_t p0, int64_t n, int32_t R, int64_t pos[2], int64_t cnt[2]) {
  if (n <= 0) return 0;
  const int64_t first = std::min<int64_t>(n, R - p0 % R);
  pos[0] = p0;
  cnt[0] = first;
  if (first == n) return 1;
  pos[1] = p0 + first;
  cnt[1] = n - first;
  return 2;
}

// The runs between sequence b0 of the cache and a snapshot buffer laid out as I. to_snapshot: cache ->
// buffer; else buffer -> cache, repeated for every grid row (cache strides, the same buffer). Window
// positions len-nw .. len-1 (nw <= ring) sit at buffer index pos - (len - I.n_win).
void state_runs(const lca_cache* c, int32_t b0, const lca_snapshot_info& I, int64_t nw, uint8_t* buf,
                bool to_snapshot, CopyArgs& a) {
  const size_t mb = (size_t)c->max_blocks, R = (size_t)c->ring, nb = (size_t)I.n_blocks;
  const size_t tw2 = (size_t)c->tail_width * 2;
  auto pair = [&](void* cache_p, uint64_t off, uint64_t bytes, uint64_t stride) {
    if (to_snapshot) add_run(a, cache_p, buf + off, bytes, 0, 0);
    else add_run(a, buf + off, cache_p, bytes, 0, stride);
  };
  if (c->desc.kind != LCA_KIND_SWA) {
    pair(c->blk_codes_dev + (size_t)b0 * mb * 64, I.off[0], nb * 64, mb * 64);
    pair(c->blk_scale_dev + (size_t)b0 * mb, I.off[1], nb * 4, mb * 4);
    pair(c->blk_rope_dev + (size_t)b0 * mb * 64, I.off[2], nb * 128, mb * 128);
    pair(c->tail_dev + (size_t)b0 * c->desc.m * c->tail_width, I.off[8], (size_t)I.n_tail * tw2,
         (size_t)c->desc.m * tw2);
  }
  if (c->desc.kind == LCA_KIND_CSA) {
    pair(c->idx_codes_dev + (size_t)b0 * mb * 32, I.off[3], nb * 32, mb * 32);
    pair(c->idx_scale_dev + (size_t)b0 * mb * 2, I.off[4], nb * 2, mb * 2);
  }
  int64_t pos[2], cnt[2];
  const int n = ring_runs(I.len - nw, nw, c->ring, pos, cnt);
  for (int i = 0; i < n; ++i) {
    const size_t slot = (size_t)b0 * R + (size_t)(pos[i] % c->ring);
    const uint64_t idx = (uint64_t)(pos[i] - (I.len - I.n_win));
    pair(c->win_codes_dev + slot * 64, I.off[5] + idx * 64, (uint64_t)cnt[i] * 64, R * 64);
    pair(c->win_scale_dev + slot, I.off[6] + idx * 4, (uint64_t)cnt[i] * 4, R * 4);
    pair(c->win_rope_dev + slot * 64, I.off[7] + idx * 128, (uint64_t)cnt[i] * 128, R * 128);
  }
}

}  // namespace

extern "C" {

lca_status lca_snapshot_layout(const lca_cache* cache, lca_snapshot_info* info) {
  if (!cache_ok(cache) || !info) return LCA_ERR_NULL;
  if (cache->pending != 0 || cache->ragged) return LCA_ERR_ORDER;
  snapshot_layout(cache->desc.kind, cache->desc.m, cache->tail_width, cache->len,
                  std::min<int64_t>(cache->len, cache->ring), info);
  return LCA_OK;
}

}  // extern "C"

namespace {

lca_status snapshot_impl(const lca_cache* cache, int32_t seq, int64_t len, void* dst_dev, size_t bytes,
                         lca_snapshot_info* info, void* stream) {
  if (seq < 0 || seq >= cache->batch) return LCA_ERR_SHAPE;
  if (((uintptr_t)dst_dev) % kAlign != 0) return LCA_ERR_SHAPE;
  if (cache->pending != 0) return LCA_ERR_ORDER;
  if (len < 0 || len > cache->max_ctx) return LCA_ERR_SHAPE;
  lca_snapshot_info I;
  size_t sz[kSections];
  snapshot_layout(cache->desc.kind, cache->desc.m, cache->tail_width, len, std::min<int64_t>(len, cache->ring), &I,
                  sz);
  if (bytes < I.bytes) return LCA_ERR_CAPACITY;
  CopyArgs a{};
  state_runs(cache, seq, I, I.n_win, (uint8_t*)dst_dev, true, a);
  // zeros in the alignment gaps, so a snapshot's bytes depend on the state alone
  for (int i = 0; i < kSections; ++i)
    add_run(a, nullptr, (uint8_t*)dst_dev + I.off[i] + sz[i], I.off[i + 1] - I.off[i] - sz[i], 0, 0);
  static_assert(sizeof(lca_snapshot_info) <= sizeof(a.header), "header words hold the info");
  std::memcpy(a.header, &I, sizeof(I));
  a.header_dst = (uint8_t*)dst_dev;
  if (launch_copy_runs(a, 1, (hipStream_t)stream) != hipSuccess) return LCA_ERR_LAUNCH;
  *info = I;
  return LCA_OK;
}

}  // namespace

extern "C" {

lca_status lca_cache_snapshot(const lca_cache* cache, int32_t seq, void* dst_dev, size_t bytes,
                              lca_snapshot_info* info, void* stream) {
  if (!cache_ok(cache) || !dst_dev || !info) return LCA_ERR_NULL;
  if (cache->ragged) return LCA_ERR_ORDER;
  return snapshot_impl(cache, seq, cache->len, dst_dev, bytes, info, stream);
}

lca_status lca_ragged_snapshot(const lca_cache* cache, int32_t seq, int64_t len, void* dst_dev, size_t bytes,
                               lca_snapshot_info* info, void* stream) {
  if (!cache_ok(cache) || !info) return LCA_ERR_NULL;
  if (!dst_dev) {  // layout only
    if (len < 0 || len > cache->max_ctx) return LCA_ERR_SHAPE;
    snapshot_layout(cache->desc.kind, cache->desc.m, cache->tail_width, len, std::min<int64_t>(len, cache->ring),
                    info);
    return LCA_OK;
  }
  return snapshot_impl(cache, seq, len, dst_dev, bytes, info, stream);
}

lca_status lca_cache_restore(lca_cache* cache, int32_t seq, const void* src_dev, size_t bytes,
                             const lca_snapshot_info* info, void* stream) {
  if (!cache_ok(cache) || !src_dev || !info) return LCA_ERR_NULL;
  if (info->magic != LCA_SNAPSHOT_MAGIC || info->version != LCA_SNAPSHOT_VERSION) return LCA_ERR_UNSUPPORTED;
  if (info->kind != cache->desc.kind || info->m != cache->desc.m || info->tail_width != cache->tail_width)
    return LCA_ERR_UNSUPPORTED;
  if (seq < -1 || seq >= cache->batch) return LCA_ERR_SHAPE;
  if (((uintptr_t)src_dev) % kAlign != 0) return LCA_ERR_SHAPE;
  if (cache->pending != 0) return LCA_ERR_ORDER;
  if (info->len < 0 || info->n_win < 0 || info->n_win > info->len) return LCA_ERR_SHAPE;
  if (info->len > cache->max_ctx) return LCA_ERR_CAPACITY;
  // the window attention reads must all be in the snapshot
  if (info->n_win < std::min<int64_t>(info->len, cache->desc.window)) return LCA_ERR_SHAPE;
  lca_snapshot_info E;
  snapshot_layout(info->kind, info->m, info->tail_width, info->len, info->n_win, &E);
  if (E.n_blocks != info->n_blocks || E.n_tail != info->n_tail || E.bytes != info->bytes ||
      std::memcmp(E.off, info->off, sizeof(E.off)) != 0)
    return LCA_ERR_SHAPE;
  if (bytes < info->bytes) return LCA_ERR_CAPACITY;
  // every sequence of a uniform cache holds the same number of tokens
  if (!cache->ragged && seq >= 0 && cache->batch > 1 && cache->len != info->len) return LCA_ERR_SHAPE;
  CopyArgs a{};
  const int64_t nw = std::min<int64_t>(info->n_win, cache->ring);
  state_runs(cache, seq < 0 ? 0 : seq, E, nw, (uint8_t*)const_cast<void*>(src_dev), false, a);
  if (launch_copy_runs(a, seq < 0 ? cache->batch : 1, (hipStream_t)stream) != hipSuccess) return LCA_ERR_LAUNCH;
  if (!cache->ragged) cache->len = info->len;
  return LCA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- ragged batches
namespace {

// The per-sequence arrays of a ragged call, checked on the host; max_end = the most tokens any
// sequence holds after the call (sizes the launches, whose workgroups beyond a sequence's own
// work return at once).
struct Ragged {
  const int64_t* len_dev;
  const int32_t* T_dev;
  int32_t T_max;
  int64_t max_end;
  int64_t blocks;  // most blocks one sequence completes
  int32_t units;   // most append units (window entries + tail rows) of one sequence
  int64_t cap;     // > 0: the kernels' capacity guard (lengths on the device, see ragged_T)
};

lca_status ragged_check(lca_cache* c, int32_t T_max, const int64_t* len_h, const int32_t* T_h,
                        const int64_t* len_d, const int32_t* T_d, Ragged* r) {
  if (!cache_ok(c) || !len_h || !T_h || !len_d || !T_d) return LCA_ERR_NULL;
  if (T_max < 1 || T_max > (1 << 24)) return LCA_ERR_SHAPE;
  if (c->pending != 0) return LCA_ERR_ORDER;
  if (!c->ragged && c->len != 0) return LCA_ERR_ORDER;  // a cache turns ragged while empty
  const int64_t m = c->desc.m;
  *r = Ragged{len_d, T_d, T_max, 0, 0, 0, 0};
  for (int32_t b = 0; b < c->batch; ++b) {
    const int64_t len = len_h[b];
    const int32_t T = T_h[b];
    if (len < 0 || T < 0 || T > T_max) return LCA_ERR_SHAPE;
    if (len + T > c->max_ctx) return LCA_ERR_CAPACITY;
    const int64_t end = len + T;
    r->max_end = std::max(r->max_end, end);
    if (c->desc.kind != LCA_KIND_SWA) r->blocks = std::max(r->blocks, end / m - len / m);
    const int64_t win_first = std::max(len, end - (int64_t)c->ring);
    const int64_t tail_first = std::max(len, c->desc.kind == LCA_KIND_SWA ? end : (end / m) * m);
    r->units = std::max<int32_t>(r->units, (int32_t)((end - win_first) + (end - tail_first)));
  }
  return LCA_OK;
}

lca_status ragged_ingest_impl(lca_cache* c, const Ragged& r, const uint16_t* kv, const uint16_t* gate,
                              const uint16_t* ik, const uint16_t* ig, const float* bias, const float* idx_bias,
                              bool with_append, IngestArgs* app_out, hipStream_t s) {
  const int32_t kind = c->desc.kind;
  if (!kv) return LCA_ERR_NULL;
  if (kind != LCA_KIND_SWA && (!gate || !bias)) return LCA_ERR_NULL;
  if (kind == LCA_KIND_CSA && (!ik || !ig || !idx_bias)) return LCA_ERR_NULL;
  const bool csa = kind == LCA_KIND_CSA;
  IngestArgs a = ingest_args(c, kv, gate, csa ? ik : nullptr, csa ? ig : nullptr, r.T_max);
  a.len = 0;
  a.seq_len = r.len_dev;
  a.seq_T = r.T_dev;
  a.seq_cap = r.cap;
  a.bias = bias;
  a.idx_bias = csa ? idx_bias : nullptr;
  if (r.blocks > 0 && launch_compress(a, csa, r.blocks, s) != hipSuccess) return LCA_ERR_LAUNCH;
  a.first = 0;
  a.n_win = 0;  // per sequence in the kernel
  if (app_out) *app_out = a;
  if (with_append && launch_append(a, csa, r.units, s) != hipSuccess) return LCA_ERR_LAUNCH;
  return LCA_OK;
}

// A ragged step's launches (lca_ragged_step; lca_ragged_step_graph when adv_len is set: the attention
// launch then advances the lengths on the device).
lca_status ragged_step_impl(lca_cache* cache, const Ragged& r, int64_t* adv_len, const uint16_t* kv_dev,
                            const uint16_t* gate_dev, const uint16_t* ik_dev, const uint16_t* ig_dev,
                            const float* bias_dev, const float* idx_bias_dev, const uint16_t* qI_dev,
                            const float* w_dev, const uint16_t* q_dev, int32_t* topk_dev, uint16_t* out_dev,
                            float* lse_dev, void* ws_dev, size_t ws_bytes, hipStream_t s) {
  const int32_t T_max = r.T_max;
  if ((int64_t)cache->batch * T_max > kAttendMaxQueries) return LCA_ERR_SHAPE;
  if (!kv_dev || !q_dev || !out_dev) return LCA_ERR_NULL;
  const int32_t kind = cache->desc.kind;
  // the queries' view: the cache after the call, sized by the longest sequence (the argument builders
  // check shapes against it; the kernels take each sequence's own length from len_dev / T_dev)
  lca_cache after = *cache;
  after.ragged = 0;
  after.len = std::max<int64_t>(r.max_end, T_max);
  AttendArgs args{};
  lca_status st;
  if (kind == LCA_KIND_CSA) {
    st = score_args(&after, qI_dev, w_dev, true, T_max, topk_dev, false, ws_dev, ws_bytes, &args.s);
    if (st != LCA_OK) return st;
    args.s.seq_len = r.len_dev;
    args.s.seq_T = r.T_dev;
    args.s.seq_cap = r.cap;
  }
  st = attn_args(&after, kind, q_dev, nullptr, T_max, out_dev, lse_dev, &args.t);
  if (st != LCA_OK) return st;
  args.t.seq_len = r.len_dev;
  args.t.seq_T = r.T_dev;
  args.t.seq_cap = r.cap;
  attend_workspace(&args, &after, T_max, ws_dev, ws_bytes);
  if (adv_len) {
    args.adv_len = adv_len;
    args.adv_cnt = (uint32_t*)ws_dev + kAdvCounter;
  }
  if (kind == LCA_KIND_CSA) {
    // compress; then as lca_csa_step: scores + selection with the append in the same launch, then the
    // attention -- or score, candidate scan with the append, selection + attention
    IngestArgs app;
    st = ragged_ingest_impl(cache, r, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, false, &app, s);
    if (st != LCA_OK) return st;
    cache->ragged = 1;
    if (use_coop(&args.s, (int64_t)cache->batch * T_max)) {
      ScanArgs sa{};
      sa.a = args.s;
      sa.app = app;
      sa.app_units = r.units;
      if (launch_index_select(sa, cache->batch, s) != hipSuccess) return LCA_ERR_LAUNCH;
      return launch_status(launch_attend(args, cache->batch, kAttendListWs, s));
    }
    if (launch_index_score(args.s, cache->batch, s) != hipSuccess) return LCA_ERR_LAUNCH;
    if (launch_topk_select(args.s, cache->batch, s, false, &app, r.units) != hipSuccess) return LCA_ERR_LAUNCH;
    return launch_status(launch_attend(args, cache->batch, kAttendSelect, s));
  }
  st = ragged_ingest_impl(cache, r, kv_dev, gate_dev, nullptr, nullptr, bias_dev, nullptr, true, nullptr, s);
  if (st != LCA_OK) return st;
  cache->ragged = 1;
  return launch_status(launch_attend(args, cache->batch, kAttendDense, s));
}

}  // namespace

extern "C" {

lca_status lca_ragged_ingest(lca_cache* cache, int32_t T_max, const int64_t* len_host, const int32_t* T_host,
                             const int64_t* len_dev, const int32_t* T_dev, const uint16_t* kv_dev,
                             const uint16_t* gate_dev, const uint16_t* ik_dev, const uint16_t* ig_dev,
                             const float* bias_dev, const float* idx_bias_dev, void* stream) {
  Ragged r;
  lca_status st = ragged_check(cache, T_max, len_host, T_host, len_dev, T_dev, &r);
  if (st != LCA_OK) return st;
  st = ragged_ingest_impl(cache, r, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, true, nullptr,
                          (hipStream_t)stream);
  if (st == LCA_OK) cache->ragged = 1;
  return st;
}

lca_status lca_ragged_step(lca_cache* cache, int32_t T_max, const int64_t* len_host, const int32_t* T_host,
                           const int64_t* len_dev, const int32_t* T_dev, const uint16_t* kv_dev,
                           const uint16_t* gate_dev, const uint16_t* ik_dev, const uint16_t* ig_dev,
                           const float* bias_dev, const float* idx_bias_dev, const uint16_t* qI_dev,
                           const float* w_dev, const uint16_t* q_dev, int32_t* topk_dev, uint16_t* out_dev,
                           float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  Ragged r;
  lca_status st = ragged_check(cache, T_max, len_host, T_host, len_dev, T_dev, &r);
  if (st != LCA_OK) return st;
  return ragged_step_impl(cache, r, nullptr, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, qI_dev, w_dev,
                          q_dev, topk_dev, out_dev, lse_dev, ws_dev, ws_bytes, (hipStream_t)stream);
}

lca_status lca_ragged_step_graph(lca_cache* cache, int32_t T_max, int64_t cap_len, int64_t* len_dev,
                                 const int32_t* T_dev, const uint16_t* kv_dev, const uint16_t* gate_dev,
                                 const uint16_t* ik_dev, const uint16_t* ig_dev, const float* bias_dev,
                                 const float* idx_bias_dev, const uint16_t* qI_dev, const float* w_dev,
                                 const uint16_t* q_dev, int32_t* topk_dev, uint16_t* out_dev, float* lse_dev,
                                 void* ws_dev, size_t ws_bytes, void* stream) {
  if (!cache_ok(cache) || !len_dev || !T_dev) return LCA_ERR_NULL;
  if (T_max < 1 || T_max > (1 << 24)) return LCA_ERR_SHAPE;
  if (cap_len < T_max || cap_len > cache->max_ctx) return LCA_ERR_CAPACITY;
  if (cache->pending != 0) return LCA_ERR_ORDER;
  if (!cache->ragged && cache->len != 0) return LCA_ERR_ORDER;  // a cache turns ragged while empty
  if (!ws_dev) return LCA_ERR_WORKSPACE;  // the advance counter lives there
  if (ws_bytes < lca_workspace_bytes(&cache->desc, cache->batch, T_max, cache->max_ctx)) return LCA_ERR_WORKSPACE;
  // the launches of any step of T_max tokens per sequence that ends at or below cap_len: grids for cap_len,
  // the compress launch always (at most ceil(T_max / m) blocks per sequence), the largest append
  const int64_t m = cache->desc.m;
  Ragged r{len_dev, T_dev, T_max, cap_len, 0, 0, cap_len};
  if (cache->desc.kind != LCA_KIND_SWA) r.blocks = (T_max + m - 1) / m;
  const int64_t win = std::min<int64_t>(T_max, cache->ring);
  const int64_t tail = cache->desc.kind == LCA_KIND_SWA ? 0 : std::min<int64_t>(T_max, m - 1);
  r.units = (int32_t)(win + tail);
  return ragged_step_impl(cache, r, len_dev, kv_dev, gate_dev, ik_dev, ig_dev, bias_dev, idx_bias_dev, qI_dev, w_dev,
                          q_dev, topk_dev, out_dev, lse_dev, ws_dev, ws_bytes, (hipStream_t)stream);
}

}  // extern "C"
