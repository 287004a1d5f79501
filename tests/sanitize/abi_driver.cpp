// Drives every entry point of include/lca.h through its host-side checks and launch planning, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against the real host code (csrc/capi.hip) and
// stand-ins for the kernel launches and the HIP runtime (launch_stubs.hip, hip_stubs.cpp): valid calls
// of all three layer kinds (ingest, indexer, attention, the one-call steps, snapshot / restore, ragged
// batches, the no-allocation step) return LCA_OK with the expected launches; invalid ones return their
// error codes and change nothing. Cache and workspace memory are host buffers (no launch touches them);
// the other device pointers are never dereferenced.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/lca.h"

extern "C" int stub_launches(const char* name);
extern "C" void stub_reset();

static int g_fail = 0;
#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                               \
    }                                                                         \
  } while (0)

namespace {
const uint16_t* U16 = reinterpret_cast<const uint16_t*>(0x10000);
const float* F32 = reinterpret_cast<const float*>(0x20000);
uint16_t* O16 = reinterpret_cast<uint16_t*>(0x30000);
float* OF32 = reinterpret_cast<float*>(0x40000);
int32_t* TOPK = reinterpret_cast<int32_t*>(0x50000);

lca_layer_desc desc(int kind, int m, int heads, int window, int hi, int k) {
  lca_layer_desc d;
  d.kind = kind;
  d.m = m;
  d.n_heads = heads;
  d.window = window;
  d.idx_heads = hi;
  d.topk = k;
  return d;
}

struct Bound {
  std::vector<uint8_t> mem, ws;
  lca_cache c;
  size_t ws_bytes = 0;
  void* wsp() { return ws.data(); }
};

bool bind(Bound& b, const lca_layer_desc& d, int32_t B, int64_t max_ctx, int32_t ring, int32_t max_tq) {
  const size_t n = lca_cache_bytes(&d, B, max_ctx, ring);
  if (!n) return false;
  b.mem.assign(n + 256, 0);
  void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(b.mem.data()) + 255) & ~uintptr_t(255));
  if (lca_cache_bind(&d, &b.c, base, n, B, max_ctx, ring, nullptr) != LCA_OK) return false;
  b.ws_bytes = lca_workspace_bytes(&d, B, max_tq, max_ctx);
  b.ws.assign(b.ws_bytes ? b.ws_bytes : 1, 0);
  return b.ws_bytes == 0 || lca_workspace_init(b.ws.data(), b.ws_bytes, nullptr) == LCA_OK;
}

// T tokens in: compress (CSA / HCA) then append
int ingest(Bound& b, int32_t T) {
  lca_cache* c = &b.c;
  int st = LCA_OK;
  if (c->desc.kind == LCA_KIND_CSA) st = lca_csa_compress(c, U16, U16, U16, U16, F32, F32, T, nullptr);
  if (c->desc.kind == LCA_KIND_HCA) st = lca_hca_compress(c, U16, U16, F32, T, nullptr);
  if (st != LCA_OK) return st;
  const bool csa = c->desc.kind == LCA_KIND_CSA, swa = c->desc.kind == LCA_KIND_SWA;
  return lca_swa_tail_append(c, U16, swa ? nullptr : U16, csa ? U16 : nullptr, csa ? U16 : nullptr, T, nullptr);
}

// k = 256: the decode calls take the one-launch indexer (every query's chunks fit its records); k = 1024
// at 8.5K blocks: the three-launch path (score, candidate scan, selection in the attention launch)
void csa_paths(int k) {
  const bool one_launch = k == 256;
  const lca_layer_desc d = desc(LCA_KIND_CSA, 4, 64, 128, 8, k);
  Bound b;
  EXPECT(bind(b, d, 4, 40000, 128, 4));
  lca_cache* c = &b.c;
  EXPECT(c->max_blocks == 10000 && c->len == 0 && c->idx_codes_dev != nullptr);
  EXPECT(ingest(b, 4096) == LCA_OK && c->len == 4096);
  EXPECT(ingest(b, 30000) == LCA_OK && c->len == 34096);
  // order: append without compress, compress twice
  EXPECT(lca_swa_tail_append(c, U16, U16, U16, U16, 1, nullptr) == LCA_ERR_ORDER);
  EXPECT(lca_csa_compress(c, U16, U16, U16, U16, F32, F32, 1, nullptr) == LCA_OK);
  EXPECT(lca_csa_compress(c, U16, U16, U16, U16, F32, F32, 1, nullptr) == LCA_ERR_ORDER);
  EXPECT(lca_swa_tail_append(c, U16, U16, U16, U16, 1, nullptr) == LCA_OK && c->len == 34097);
  // indexer and attention, every call form
  stub_reset();
  EXPECT(lca_csa_indexer_topk(c, U16, F32, 1, TOPK, b.wsp(), b.ws_bytes, nullptr) == LCA_OK);
  EXPECT(stub_launches("index_select") == (one_launch ? 1 : 0));
  EXPECT(stub_launches("index_score") == (one_launch ? 0 : 1));
  EXPECT(lca_csa_index_score(c, U16, F32, 1, b.wsp(), b.ws_bytes, nullptr) == LCA_OK);
  EXPECT(lca_csa_topk_select(c, 1, TOPK, b.wsp(), b.ws_bytes, nullptr) == LCA_OK);
  EXPECT(lca_csa_sparse_attn(c, U16, TOPK, 1, O16, OF32, b.wsp(), b.ws_bytes, nullptr) == LCA_OK);
  EXPECT(lca_csa_sparse_attn(c, U16, TOPK, 1, O16, nullptr, nullptr, 0, nullptr) == LCA_OK);  // no workspace
  EXPECT(lca_csa_attend(c, U16, F32, U16, 1, TOPK, O16, OF32, b.wsp(), b.ws_bytes, nullptr) == LCA_OK);
  EXPECT(lca_csa_topk_attn(c, U16, 1, TOPK, O16, OF32, b.wsp(), b.ws_bytes, nullptr) == LCA_OK);
  // the one-call step across a block boundary; the timed and the no-allocation variants
  for (int i = 0; i < 6; ++i) {
    stub_reset();
    const bool completes = (c->len + 1) % 4 == 0;
    EXPECT(lca_csa_step(c, U16, U16, U16, U16, F32, F32, 1, U16, F32, U16, TOPK, O16, nullptr, b.wsp(), b.ws_bytes,
                        nullptr) == LCA_OK);
    EXPECT(stub_launches("compress") == (completes ? 1 : 0));
    // one launch for the indexer and the attention, or the indexer's launch(es) and the attention's
    EXPECT(one_launch ? stub_launches("csa_step") == 1 && stub_launches("index_select") == 0 &&
                            stub_launches("attend") == 0
                      : stub_launches("csa_step") == 0 && stub_launches("attend") == 1);
    EXPECT(stub_launches("topk_select") == (one_launch ? 0 : 1));
  }
  // the launch plan agrees with the launches
  int32_t plan = 0;
  EXPECT(lca_csa_step_launches(c, 1, b.wsp(), b.ws_bytes, &plan) == LCA_OK && plan == (one_launch ? 1 : 3));
  EXPECT(lca_csa_step_launches(c, 1, nullptr, 0, &plan) == LCA_ERR_WORKSPACE);
  // the two-launch path on request
  setenv("LCA_STEP_UNFUSED", "1", 1);
  EXPECT(lca_csa_step_launches(c, 1, b.wsp(), b.ws_bytes, &plan) == LCA_OK && plan == (one_launch ? 2 : 3));
  for (int i = 0; i < 2; ++i) {
    stub_reset();
    EXPECT(lca_csa_step(c, U16, U16, U16, U16, F32, F32, 1, U16, F32, U16, TOPK, O16, nullptr, b.wsp(), b.ws_bytes,
                        nullptr) == LCA_OK);
    EXPECT(stub_launches("csa_step") == 0 && stub_launches("attend") == 1);
    EXPECT(stub_launches("index_select") == (one_launch ? 1 : 0));
  }
  unsetenv("LCA_STEP_UNFUSED");
  void* ev[4] = {reinterpret_cast<void*>(1), nullptr, reinterpret_cast<void*>(2), reinterpret_cast<void*>(3)};
  const int64_t len0 = c->len;
  EXPECT(lca_csa_step_timed(c, U16, U16, U16, U16, F32, F32, 1, U16, F32, U16, TOPK, O16, nullptr, b.wsp(),
                            b.ws_bytes, nullptr, ev) == LCA_OK && c->len == len0 + 1);
  EXPECT(lca_csa_step_timed(c, U16, U16, U16, U16, F32, F32, 1, U16, F32, U16, TOPK, O16, nullptr, b.wsp(),
                            b.ws_bytes, nullptr, nullptr) == LCA_ERR_NULL && c->len == len0 + 1);
  for (int i = 0; i < 3; ++i)
    EXPECT(lca_csa_step_noalloc(c, U16, U16, U16, U16, F32, F32, 1, U16, F32, U16, TOPK, O16, OF32, nullptr) ==
           LCA_OK);
  // T > 1: the ring (128) holds no T + window - 1 = 130 slots; a workspace sized for 4 queries per
  // sequence, not 5; B * T beyond 511
  EXPECT(lca_csa_step(c, U16, U16, U16, U16, F32, F32, 3, U16, F32, U16, TOPK, O16, OF32, b.wsp(), b.ws_bytes,
                      nullptr) == LCA_ERR_CAPACITY);
  EXPECT(lca_csa_step(c, U16, U16, U16, U16, F32, F32, 5, U16, F32, U16, TOPK, O16, OF32, b.wsp(), b.ws_bytes,
                      nullptr) == LCA_ERR_WORKSPACE);
  EXPECT(lca_csa_step(c, U16, U16, U16, U16, F32, F32, 128, U16, F32, U16, TOPK, O16, OF32, b.wsp(), b.ws_bytes,
                      nullptr) == LCA_ERR_SHAPE);
  // capacity, nulls, a short workspace, a wrong kind
  const int64_t len1 = c->len;
  EXPECT(lca_csa_compress(c, U16, U16, U16, U16, F32, F32, 100000, nullptr) == LCA_ERR_CAPACITY);
  EXPECT(lca_csa_step(c, nullptr, U16, U16, U16, F32, F32, 1, U16, F32, U16, TOPK, O16, OF32, b.wsp(), b.ws_bytes,
                      nullptr) == LCA_ERR_NULL);
  EXPECT(lca_csa_indexer_topk(c, U16, F32, 1, TOPK, b.wsp(), 100, nullptr) == LCA_ERR_WORKSPACE);
  EXPECT(lca_hca_dense_attn(c, U16, 1, O16, OF32, b.wsp(), b.ws_bytes, nullptr) != LCA_OK);
  EXPECT(c->len == len1 && c->pending == 0);
  // snapshot of one sequence, restored into another
  lca_snapshot_info info;
  EXPECT(lca_snapshot_layout(c, &info) == LCA_OK && info.len == c->len && info.bytes > 0);
  std::vector<uint8_t> snap(info.bytes + 256);
  void* sp = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(snap.data()) + 255) & ~uintptr_t(255));
  EXPECT(lca_cache_snapshot(c, 1, sp, info.bytes, &info, nullptr) == LCA_OK);
  EXPECT(lca_cache_restore(c, 2, sp, info.bytes, &info, nullptr) == LCA_OK);
  EXPECT(lca_cache_snapshot(c, 4, sp, info.bytes, &info, nullptr) == LCA_ERR_SHAPE);
  EXPECT(lca_cache_snapshot(c, 0, sp, info.bytes - 1, &info, nullptr) != LCA_OK);
  lca_snapshot_info bad = info;
  bad.m = 5;
  EXPECT(lca_cache_restore(c, 0, sp, info.bytes, &bad, nullptr) != LCA_OK);
  // many-query calls (chunked-prefill shapes): the query-tile indexer and the many-query attention
  Bound p;
  const lca_layer_desc dp = desc(LCA_KIND_CSA, 4, 64, 128, 8, 512);
  EXPECT(bind(p, dp, 1, 40000, 4096 + 127, 4096));
  EXPECT(ingest(p, 36000) == LCA_OK);
  EXPECT(lca_csa_indexer_topk(&p.c, U16, F32, 4096, TOPK, p.wsp(), p.ws_bytes, nullptr) == LCA_OK);
  EXPECT(lca_csa_sparse_attn(&p.c, U16, TOPK, 4096, O16, OF32, p.wsp(), p.ws_bytes, nullptr) == LCA_OK);
  EXPECT(lca_csa_index_score(&p.c, U16, F32, 600, p.wsp(), p.ws_bytes, nullptr) == LCA_OK);
  EXPECT(lca_csa_topk_select(&p.c, 600, TOPK, p.wsp(), p.ws_bytes, nullptr) == LCA_OK);
}

void dense_paths() {
  const lca_layer_desc h = desc(LCA_KIND_HCA, 128, 64, 128, 0, 0);
  Bound b;
  EXPECT(bind(b, h, 8, 70000, 128, 1));
  lca_cache* c = &b.c;
  EXPECT(ingest(b, 65536) == LCA_OK && c->len == 65536);
  EXPECT(lca_hca_dense_attn(c, U16, 1, O16, OF32, b.wsp(), b.ws_bytes, nullptr) == LCA_OK);
  EXPECT(lca_hca_dense_attn(c, U16, 1, O16, OF32, nullptr, 0, nullptr) == LCA_OK);
  for (int i = 0; i < 130; ++i)
    EXPECT(lca_hca_step(c, U16, U16, F32, 1, U16, O16, nullptr, b.wsp(), b.ws_bytes, nullptr) == LCA_OK);
  EXPECT(c->len == 65536 + 130);
  EXPECT(lca_csa_indexer_topk(c, U16, F32, 1, TOPK, b.wsp(), b.ws_bytes, nullptr) == LCA_ERR_UNSUPPORTED);
  const lca_layer_desc s = desc(LCA_KIND_SWA, 1, 16, 1024, 0, 0);
  Bound w;
  EXPECT(bind(w, s, 2, 5000, 1026, 3));
  EXPECT(ingest(w, 1500) == LCA_OK);
  EXPECT(lca_swa_attn(&w.c, U16, 1, O16, OF32, w.wsp(), w.ws_bytes, nullptr) == LCA_OK);
  for (int T : {1, 3, 1})
    EXPECT(lca_swa_step(&w.c, U16, T, U16, O16, OF32, w.wsp(), w.ws_bytes, nullptr) == LCA_OK);
  EXPECT(lca_swa_step(&w.c, U16, 4, U16, O16, OF32, w.wsp(), w.ws_bytes, nullptr) == LCA_ERR_CAPACITY);
  lca_snapshot_info info;
  EXPECT(lca_snapshot_layout(&w.c, &info) == LCA_OK && info.n_blocks == 0);
}

void ragged_paths() {
  const lca_layer_desc d = desc(LCA_KIND_CSA, 4, 16, 128, 4, 64);
  Bound b;
  EXPECT(bind(b, d, 3, 20000, 131, 4));
  lca_cache* c = &b.c;
  const int64_t len0[3] = {0, 0, 0};
  const int32_t T0[3] = {3000, 17, 9000};
  const int64_t* LD = reinterpret_cast<const int64_t*>(0x60000);
  const int32_t* TD = reinterpret_cast<const int32_t*>(0x70000);
  EXPECT(lca_ragged_ingest(c, 9000, len0, T0, LD, TD, U16, U16, U16, U16, F32, F32, nullptr) == LCA_OK);
  EXPECT(c->ragged == 1);
  const int64_t len1[3] = {3000, 17, 9000};
  const int32_t T1[3] = {1, 0, 4};
  EXPECT(lca_ragged_step(c, 4, len1, T1, LD, TD, U16, U16, U16, U16, F32, F32, U16, F32, U16, TOPK, O16, OF32,
                         b.wsp(), b.ws_bytes, nullptr) == LCA_OK);
  const int32_t Tbad[3] = {1, 0, 5};
  EXPECT(lca_ragged_step(c, 4, len1, Tbad, LD, TD, U16, U16, U16, U16, F32, F32, U16, F32, U16, TOPK, O16, OF32,
                         b.wsp(), b.ws_bytes, nullptr) == LCA_ERR_SHAPE);
  // uniform calls refuse a ragged cache
  EXPECT(lca_csa_step(c, U16, U16, U16, U16, F32, F32, 1, U16, F32, U16, TOPK, O16, OF32, b.wsp(), b.ws_bytes,
                      nullptr) == LCA_ERR_ORDER);
  // the capture-friendly step: lengths on the device only; a second ragged cache, empty
  Bound g;
  EXPECT(bind(g, d, 3, 20000, 131, 1));
  int64_t* LDG = reinterpret_cast<int64_t*>(0x80000);
  for (int i = 0; i < 3; ++i) {
    stub_reset();
    EXPECT(lca_ragged_step_graph(&g.c, 1, 12000, LDG, TD, U16, U16, U16, U16, F32, F32, U16, F32, U16, TOPK, O16,
                                 OF32, g.wsp(), g.ws_bytes, nullptr) == LCA_OK);
    EXPECT(stub_launches("compress") == 1 && stub_launches("attend") == 1);
    EXPECT(stub_launches("index_select") + stub_launches("index_score") == 1);
  }
  EXPECT(g.c.ragged == 1);
  EXPECT(lca_ragged_step_graph(&g.c, 1, 30000, LDG, TD, U16, U16, U16, U16, F32, F32, U16, F32, U16, TOPK, O16, OF32,
                               g.wsp(), g.ws_bytes, nullptr) == LCA_ERR_CAPACITY);
  EXPECT(lca_ragged_step_graph(&g.c, 1, 12000, LDG, TD, U16, U16, U16, U16, F32, F32, U16, F32, U16, TOPK, O16, OF32,
                               nullptr, 0, nullptr) == LCA_ERR_WORKSPACE);
  EXPECT(lca_ragged_step_graph(&g.c, 1, 12000, nullptr, TD, U16, U16, U16, U16, F32, F32, U16, F32, U16, TOPK, O16,
                               OF32, g.wsp(), g.ws_bytes, nullptr) == LCA_ERR_NULL);
  EXPECT(lca_ragged_step_graph(&b.c, 512, 12000, LDG, TD, U16, U16, U16, U16, F32, F32, U16, F32, U16, TOPK, O16,
                               OF32, b.wsp(), b.ws_bytes, nullptr) != LCA_OK);  // B * T beyond 511
  lca_snapshot_info info;
  std::vector<uint8_t> snap(1 << 22);
  void* sp = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(snap.data()) + 255) & ~uintptr_t(255));
  EXPECT(lca_ragged_snapshot(c, 2, 9004, sp, (1 << 22) - 256, &info, nullptr) == LCA_OK && info.len == 9004);
}

void descriptors() {
  EXPECT(lca_cache_bytes(nullptr, 1, 100, 128) == 0);
  const lca_layer_desc bad[] = {desc(7, 4, 64, 128, 8, 1024),       desc(LCA_KIND_CSA, 0, 64, 128, 8, 1024),
                                desc(LCA_KIND_CSA, 4, 65, 128, 8, 1024), desc(LCA_KIND_CSA, 4, 64, 0, 8, 1024),
                                desc(LCA_KIND_CSA, 4, 64, 128, 9, 1024), desc(LCA_KIND_CSA, 4, 64, 128, 8, 4096),
                                desc(LCA_KIND_HCA, 129, 64, 128, 0, 0),  desc(LCA_KIND_SWA, 1, 16, 5000, 0, 0)};
  for (const auto& d : bad) EXPECT(lca_cache_bytes(&d, 1, 1000, 128) == 0);
  const lca_layer_desc ok = desc(LCA_KIND_CSA, 4, 64, 128, 8, 1024);
  EXPECT(lca_cache_bytes(&ok, 0, 1000, 128) == 0);
  EXPECT(lca_cache_bytes(&ok, 1, 1000, 100) == 0);  // ring < window
  EXPECT(lca_cache_bytes(&ok, 4, (int64_t)1 << 20, 128) > 0);
  EXPECT(lca_cache_bytes(&ok, 1 << 30, (int64_t)1 << 40, 128) == 0);  // beyond any size_t it could hold
  EXPECT(lca_workspace_bytes(&ok, 4, 1, (int64_t)1 << 20) > 0);
  lca_cache c;
  std::vector<uint8_t> small(1024);
  EXPECT(lca_cache_bind(&ok, &c, small.data(), small.size(), 1, 1000, 128, nullptr) != LCA_OK);
  EXPECT(lca_csa_step(nullptr, U16, U16, U16, U16, F32, F32, 1, U16, F32, U16, TOPK, O16, OF32, nullptr, 0,
                      nullptr) == LCA_ERR_NULL);
  for (int s = 1; s >= -8; --s) EXPECT(lca_status_str(s) != nullptr);
}
}  // namespace

int main() {
  descriptors();
  csa_paths(256);
  csa_paths(1024);
  dense_paths();
  ragged_paths();
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi driver: all checks passed\n");
  return 0;
}
