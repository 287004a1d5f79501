// Host-only stand-ins for the kernel launches of the HIP library, for the CPU sanitizer build of the
// host side of the C ABI (csrc/capi.hip): each records the call and checks the launch arguments the
// host code computed (sizes, counts), then returns success without touching any device pointer.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../long_context_attention_18_amd/csrc/kernels.h"

namespace {
int g_count[16];
const char* g_names[16] = {"copy_runs", "compress", "append", "fill_zero", "index_score", "topk_select",
                           "index_select", "attend", "attention", "csa_step"};

void need(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "launch stub: bad argument: %s\n", what);
    std::abort();
  }
}
}  // namespace

extern "C" int stub_launches(const char* name) {
  for (int i = 0; i < 10; ++i)
    if (!std::strcmp(name, g_names[i])) return g_count[i];
  return -1;
}
extern "C" void stub_reset() { std::memset(g_count, 0, sizeof(g_count)); }

namespace lca {
hipError_t launch_copy_runs(CopyArgs& a, int32_t n_dst, hipStream_t) {
  need(a.n_runs >= 0 && a.n_runs <= kMaxCopyRuns && n_dst >= 1, "copy runs");
  ++g_count[0];
  return hipSuccess;
}
hipError_t launch_compress(const IngestArgs& a, bool, int64_t n_blocks, hipStream_t) {
  need(n_blocks >= 0 && a.B >= 1 && a.m >= 1, "compress");  // 0: no block completes (no launch)
  if (n_blocks == 0) return hipSuccess;
  ++g_count[1];
  return hipSuccess;
}
hipError_t launch_append(const IngestArgs& a, bool, int32_t n_tail, hipStream_t) {
  need(a.B >= 1 && n_tail >= 0, "append");
  ++g_count[2];
  return hipSuccess;
}
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t) {
  need(p != nullptr && bytes % 16 == 0, "fill");
  ++g_count[3];
  return hipSuccess;
}
hipError_t launch_index_score(const ScoreArgs& a, int32_t B, hipStream_t) {
  need(B >= 1 && a.Tq >= 1 && a.k >= 1, "index score");
  ++g_count[4];
  return hipSuccess;
}
hipError_t launch_topk_select(const ScoreArgs& a, int32_t B, hipStream_t, bool, const IngestArgs*, int32_t units) {
  need(B >= 1 && a.Tq >= 1 && units >= 0, "topk select");
  ++g_count[5];
  return hipSuccess;
}
hipError_t launch_index_select(const ScanArgs& args, int32_t B, hipStream_t) {
  const ScoreArgs& a = args.a;
  need(B >= 1 && a.coop == 1 && a.n_cols >= 1, "index select");
  need(a.pref_slots >= kRecMinWords && a.pref_slots <= kRecMaxWords && (a.pref_slots & (a.pref_slots - 1)) == 0,
       "record words");
  need((int64_t)(a.n_cols + (a.fold_tail ? 1 : 0)) * a.pref_slots <= (int64_t)kPrefMaxLoads * kScoreThreads,
       "records per query");
  need(a.cmin <= a.pref_slots, "candidates per record");
  ++g_count[6];
  return hipSuccess;
}
hipError_t launch_csa_step(const StepArgs& sa, hipStream_t) {
  const ScoreArgs& a = sa.idx.a;
  need(sa.token != 0u && sa.n_queries >= 1 && a.coop == 1 && a.n_cols >= 1 && sa.idx.app_units == 0, "step");
  need(sa.n_idx % 8 == 0 && sa.n_idx >= sa.n_queries * a.n_cols && sa.n_idx < sa.n_queries * a.n_cols + 8,
       "step score workgroups");
  const int hgs = (sa.att.t.H + 15) / 16;
  need(sa.att.splits >= 1 && sa.n_att == sa.n_queries * hgs * sa.att.splits, "step attention workgroups");
  need(sa.att.splits == 1 || (sa.att.part && sa.att.cnt && sa.n_att <= kAttendMaxWGs), "step partials");
  need((int64_t)(a.n_cols + (a.fold_tail ? 1 : 0)) * a.pref_slots <= (int64_t)kPrefMaxLoads * kScoreThreads,
       "step records per query");
  need(sa.att.app_units >= 0 && sa.att.t.Tq == a.Tq, "step append");
  ++g_count[9];
  return hipSuccess;
}
hipError_t launch_attend(const AttendArgs& args, int32_t B, int mode, hipStream_t) {
  need(B >= 1 && mode >= kAttendList && mode <= kAttendListWs, "attend");
  (void)args;
  ++g_count[7];
  return hipSuccess;
}
hipError_t launch_attention(const AttnArgs& a, int32_t B, hipStream_t) {
  need(B >= 1 && a.Tq >= 1, "attention");
  ++g_count[8];
  return hipSuccess;
}
}  // namespace lca
