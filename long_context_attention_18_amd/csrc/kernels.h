// kernels.h -- internal launch interface between the C ABI (capi.hip) and
// the gfx950 kernels. Not installed; the public interface is include/lca.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lca {

constexpr int kHeadDim = 128;
constexpr int kNope = 64;
constexpr int kRope = 64;
constexpr int kIdxDim = 64;

// ---- indexer / top-k tiling --------------------------------------------
constexpr int kScoreWaves = 8;                        // waves per score workgroup
constexpr int kScoreIters = 8;                        // 32-block tiles per wave
constexpr int kScoreChunk = kScoreWaves * kScoreIters * 32;  // blocks per workgroup (2048)
constexpr int kScoreThreads = kScoreWaves * 64;
// Calls with at least kMultiMinQueries queries (chunked prefill) score kMultiChunks chunks per workgroup
constexpr int kMultiMinQueries = 512;
constexpr int kMultiChunks = 8;
// score workgroups one compute unit holds at once (8 waves of at most 128 VGPRs, the kernel's launch bound)
constexpr int kScoreWGsPerCU = 2;
// Calls with at least kTileMinQueries queries, each seeing at most kTileMaxBlocks blocks, score in query
// tiles: kTileQueries queries of one sequence per workgroup of kTileWaves waves (indexer.hip)
constexpr int kTileMinQueries = 2048;
constexpr int kTileQueries = 8;
constexpr int kTileWaves = 8;
constexpr int64_t kTileMaxBlocks = 65535;
constexpr int kTileSeg = 256;  // blocks per candidate segment of the query tiles (one wave writes a segment)
constexpr int kTileBoundCap = 760;  // keys of a query's threshold bin the query tiles' selection holds in LDS
constexpr int kTilePrefWords = 258;  // segment offsets (at most 257), even so the digit bins stay 8-byte aligned
static_assert(kTileQueries == kTileWaves, "the tiles' selection runs one wave per query");
static_assert((kTileMaxBlocks + kTileSeg - 1) / kTileSeg + 1 <= kTilePrefWords, "segment offsets fit");
constexpr int kHistBins = 4096;                       // top 12 bits of the ordered score key
static_assert(2 * kTileBoundCap + kTilePrefWords + 256 <= kHistBins / 2,
              "a query's selection scratch fits its histogram words");
constexpr int kScanPerWG = 8192;                      // keys per candidate-scan workgroup
constexpr int kCandCap = 8192;                        // candidates the select kernel holds in LDS
constexpr int64_t kMaxBlocks = 2048LL * kScoreChunk;  // compressed blocks per sequence the indexer serves
constexpr int kMaxSegs = (int)(kMaxBlocks / kScanPerWG);  // candidate-scan segments per query (512)
static_assert((kTileMaxBlocks + kTileSeg - 1) / kTileSeg <= kMaxSegs, "query-tile segments fit the selection");

// ---- attention tiling ----------------------------------------------------
constexpr int kAttnKeys = 64;                         // keys staged per iteration (many-query kernel)
constexpr int kAttendMaxQueries = 511;                // up to this many queries per call: attend.hip
constexpr int kPrefMaxLoads = 17;  // segment slots one thread of the selecting score workgroup loads at once
static_assert(kTileMinQueries > kAttendMaxQueries, "decode-step calls (with their append) never use query tiles");
constexpr int64_t kMaxGridY = 65535;                  // launch limit of grid.y (indexer grids: one row per query)

struct IngestArgs {
  const uint16_t* kv;      // [B][T][128]
  const uint16_t* gate;    // [B][T][128]
  const uint16_t* ik;      // [B][T][64]   (CSA) or null
  const uint16_t* ig;      // [B][T][64]   (CSA) or null
  const float* bias;       // [m][128]
  const float* idx_bias;   // [m][64]     (CSA) or null
  uint8_t* blk_codes;      // [B][max_blocks][64]
  float* blk_scale;        // [B][max_blocks]
  uint16_t* blk_rope;      // [B][max_blocks][64]
  uint8_t* idx_codes;      // [B][max_blocks][32]
  uint8_t* idx_scale;      // [B][max_blocks][2]
  uint8_t* win_codes;      // [B][R][64]
  float* win_scale;        // [B][R]
  uint16_t* win_rope;      // [B][R][64]
  uint16_t* tail;          // [B][m][tail_width]
  int64_t len;             // tokens already appended before this call
  int64_t max_blocks;
  int64_t first;           // first block (compress) / first window token (append)
  int32_t T;
  int32_t m;
  int32_t ring;
  int32_t tail_width;
  int32_t n_win;           // append: window tokens written
  int32_t B;
  const double* inv_freq;  // [32], device copy of the cache's RoPE frequencies
  // ragged batches: sequence b holds seq_len[b] tokens before the call and adds seq_T[b] <= T of them
  // (rows 0..seq_T[b]-1 of its inputs); null: every sequence holds len and adds T. seq_cap > 0: a
  // sequence that would hold more than seq_cap tokens adds none (ragged_T)
  const int64_t* seq_len;
  const int32_t* seq_T;
  int64_t seq_cap;
};

// The indexer's workspace is one block per query (so its place does not depend on how many queries
// a call has): [histogram kHistBins u32][seg_cnt u32 per candidate segment][keys max_blocks u32]
// [candidates max_blocks u64], each part 256-byte aligned, qstride bytes per query.
struct ScoreArgs {
  const uint16_t* qI;      // [B][Tq][HI][64]
  const float* w;          // [B][Tq][HI]
  const uint8_t* idx_codes;
  const uint8_t* idx_scale;
  uint8_t* qbase;          // ws: per-query blocks
  uint64_t qstride;
  uint64_t off_seg, off_keys, off_cand;
  int32_t* topk;           // [B][Tq][k]
  int64_t len;
  int64_t max_blocks;
  int32_t Tq;
  int32_t HI;
  int32_t k;
  int32_t m;
  int32_t G2;              // scan segments per query
  int32_t cmin;            // keys each score workgroup counts into the histogram at least (twice its share of k)
  int32_t chunk_step;      // 0: a score workgroup per 2048-block chunk; else one per chunk_step chunks of a query
  int32_t fold_tail;       // 1: the grid leaves out the last chunk of each query, which workgroup 0 scores
                           //    after its own (decode grids that a short last chunk would push past the CUs)
  int32_t tiles;           // 1: query tiles (the score launch also writes the candidates; no scan)
  int32_t write_keys;      // tiles: also write every visible block's key (the separate score call's contract)
  int32_t tile_select;     // tiles: the score launch also selects the top-k lists into topk (combined call)
  // In-launch threshold and selection (decode-sized calls, indexer.hip): every score workgroup also writes
  // a record (its bin counts and candidates) and counts itself in; the last of a query to arrive selects
  // the query's top-k into its workspace list (and topk when not null)
  int32_t coop;
  int32_t n_cols;          // coop: score workgroup columns (chunks; the folded last chunk is not a column)
  int32_t pref_slots;      // coop: 64-bit words per record (64, 128 or 256)
  uint64_t off_sync, off_list, off_rec;
  // ragged batches (see IngestArgs): the queries of sequence b are its seq_T[b] new tokens, positions
  // seq_len[b] + i for rows i < seq_T[b]; null: positions len - Tq + i
  const int64_t* seq_len;
  const int32_t* seq_T;
  int64_t seq_cap;
};

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and row broadcasts (GFX9
// data-parallel primitives: one VALU add each, no LDS round trip): lanes shifted in from outside a
// 16-lane row contribute 0, and rows 1-3 then take the running totals of the rows before them.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Tokens sequence b adds in a ragged call: seq_T[b], or none when that would take it beyond seq_cap
// (cap > 0: the capacity a call sized its launches for without reading the lengths on the host)
__device__ __forceinline__ int32_t ragged_T(const int64_t* seq_len, const int32_t* seq_T, int64_t cap, int b) {
  const int32_t T = seq_T[b];
  return (cap > 0 && seq_len[b] + T > cap) ? 0 : T;
}

// Position of query row tq of sequence b, or -1 when the row holds no query (ragged batches)
__device__ __forceinline__ int64_t query_t(const int64_t* seq_len, const int32_t* seq_T, int64_t cap, int64_t len,
                                           int32_t Tq, int b, int tq) {
  if (seq_len) return tq < ragged_T(seq_len, seq_T, cap, b) ? seq_len[b] + tq : -1;
  return len - Tq + tq;
}

__device__ __forceinline__ uint32_t* q_hist(const ScoreArgs& a, int q) { return (uint32_t*)(a.qbase + (size_t)q * a.qstride); }
__device__ __forceinline__ uint32_t* q_seg(const ScoreArgs& a, int q) { return (uint32_t*)(a.qbase + (size_t)q * a.qstride + a.off_seg); }
__device__ __forceinline__ uint32_t* q_keys(const ScoreArgs& a, int q) { return (uint32_t*)(a.qbase + (size_t)q * a.qstride + a.off_keys); }
__device__ __forceinline__ uint64_t* q_cand(const ScoreArgs& a, int q) { return (uint64_t*)(a.qbase + (size_t)q * a.qstride + a.off_cand); }
// coop: the query's counter of score workgroups that arrived (word 0; zero between calls) and, for the
// one-launch step, its list-ready word (word kSyncReady: the launch's token once the list is out). The two
// sit in different 128-byte lines: the attention workgroups poll the ready word while the score
// workgroups count themselves in, and polls of the counter's line slow those atomics down.
__device__ __forceinline__ uint32_t* q_sync(const ScoreArgs& a, int q) { return (uint32_t*)(a.qbase + (size_t)q * a.qstride + a.off_sync); }
constexpr int kSyncReady = 32;
constexpr int kSyncBytes = 256;
// coop: per query, kRecHdrSlots record headers (one 64-bit word per score chunk: the chunk's largest key
// << 32 | its floor bin << 16 | its candidate count), then one record of pref_slots words per score chunk
// (its candidates, key << 32 | ~block, in block order, zero-padded)
constexpr int kRecHdrSlots = kMaxSegs;
constexpr int kRecMinWords = 32;
constexpr int kRecMaxWords = 256;
__device__ __forceinline__ uint64_t* q_rec(const ScoreArgs& a, int q) { return (uint64_t*)(a.qbase + (size_t)q * a.qstride + a.off_rec); }
// coop: the query's top-k list (k int32, ascending, -1 padded), read by the attention launch
__device__ __forceinline__ int32_t* q_list(const ScoreArgs& a, int q) { return (int32_t*)(a.qbase + (size_t)q * a.qstride + a.off_list); }

struct AttnArgs {
  const uint16_t* q;       // [B][Tq][H][128]
  const int32_t* topk;     // [B][Tq][k] (CSA) or null (HCA)
  const uint8_t* blk_codes;
  const float* blk_scale;
  const uint16_t* blk_rope;
  const uint8_t* win_codes;
  const float* win_scale;
  const uint16_t* win_rope;
  uint16_t* out;           // [B][Tq][H][128]
  float* lse;              // [B][Tq][H] or null
  int64_t len;
  int64_t max_blocks;
  int32_t Tq;
  int32_t H;
  int32_t k;               // CSA: top-k slots; HCA: 0
  int32_t m;
  int32_t W;
  int32_t ring;
  int32_t dense;           // 1 = HCA (every visible block), 0 = CSA (topk list)
  const double* inv_freq;  // [32], device copy of the cache's RoPE frequencies
  const int64_t* seq_len;  // ragged batches, as in ScoreArgs
  const int32_t* seq_T;
  int64_t seq_cap;
};

// One-launch attention for a few queries (attend.hip): the query's compressed entries come from the
// caller's top-k list (LIST), the list the in-launch selection left in the workspace (LIST_WS: always
// valid; a query that sees at most k blocks attends to all of them without reading a list), every visible
// block (DENSE), or the top-k selection run in the same workgroup over the scan's candidates (SELECT).
constexpr int kMaxTopk = 2048;
constexpr int kAttendList = 0, kAttendDense = 1, kAttendSelect = 2, kAttendListWs = 3;
// Key splits of the one-launch attention: a (query, 16-head group) may be spread over up to
// kAttendMaxSplits workgroups (about one 32-key chunk per wave), each over its share of the keys; each writes a partial (running max,
// sum and unnormalised O of its 16 heads) with agent-scope stores that complete before it counts itself
// in on a per-(query, group) counter, and the last to count in merges them.
constexpr int kAttendMaxSplits = 16;
constexpr int kAttendNoSplitChunks = 3;  // 32-key chunks per wave up to which a (query, head group) is not split
constexpr int kAttendMaxWGs = 256;  // with splits, a call stays within one workgroup per CU (LDS allows one)
struct AttendPartial {
  float m[16], l[16];
  float o[16][kHeadDim];
};
constexpr size_t kAttendCounterBytes = 8192;  // (query, group) counters: 511 queries x 4 groups x 4 B, padded
constexpr int kAdvCounter = (int)(kAttendCounterBytes / 4) - 1;  // the length-advance counter: the last slot
static_assert(511 * 4 <= kAdvCounter, "advance counter overlaps the (query, group) counters");
struct AttendArgs {
  ScoreArgs s;  // selection inputs (kAttendSelect)
  AttnArgs t;
  AttendPartial* part;  // [B*Tq][groups][splits] (splits > 1)
  uint32_t* cnt;        // [B*Tq][groups], zero between calls (splits > 1)
  int32_t splits;
  // kAttendDense with app_units > 0: the launch also appends the step's tokens (window entries by the
  // split-0 workgroups that read the window, tail copies by head group 0 of split 0), before attending
  IngestArgs app;
  int32_t app_units;
  // a step whose lengths live on the device (capture-friendly ragged step): the last workgroup of the
  // launch to have read its length (adv_cnt, zero between calls) adds ragged_T to every seq_len
  int64_t* adv_len;
  uint32_t* adv_cnt;
};


// Contiguous runs copied between a cache and a snapshot buffer (persist.hip): run i moves `bytes`
// from src + y * src_stride to dst + y * dst_stride for every grid row y < n_dst (src = null: writes
// zeros); the launcher sets `unit` (16, 4 or 1 bytes) from the addresses' alignment. Workgroup (0, 0)
// also writes the kCopyHeaderWords header words to header_dst when it is not null.
constexpr int kMaxCopyRuns = 24;
constexpr int kCopyHeaderWords = 64;
struct CopyRun {
  const uint8_t* src;
  uint8_t* dst;
  uint64_t bytes;
  uint64_t src_stride, dst_stride;
  int32_t unit;
};
struct CopyArgs {
  CopyRun run[kMaxCopyRuns];
  int32_t n_runs;
  uint8_t* header_dst;
  uint32_t header[kCopyHeaderWords];
};
hipError_t launch_copy_runs(CopyArgs& a, int32_t n_dst, hipStream_t s);

hipError_t launch_compress(const IngestArgs& a, bool csa, int64_t n_blocks, hipStream_t s);
hipError_t launch_append(const IngestArgs& a, bool csa, int32_t n_tail, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_index_score(const ScoreArgs& a, int32_t B, hipStream_t s);
struct ScanArgs {
  ScoreArgs a;
  IngestArgs app;     // a decode step's append, done by the scan launch (app_units > 0)
  int32_t app_units;  // window entries + tail copies per sequence
};
hipError_t launch_topk_select(const ScoreArgs& a, int32_t B, hipStream_t s, bool with_select = true,
                              const IngestArgs* app = nullptr, int32_t app_units = 0);
// The in-launch-threshold score launch (ScoreArgs.coop): scores, bound, candidates and the selection of
// every query; with app_units > 0 one more row of workgroups writes the step's append.
hipError_t launch_index_select(const ScanArgs& args, int32_t B, hipStream_t s);
// The CSA decode step in one launch (csa_step_kernel, indexer.hip): the one-launch indexer's score
// workgroups, then the attention workgroups over the lists they leave (list mode, the step's append
// written by the attention). Each query's last score workgroup stores `token` into the second word of
// the query's sync slot once its list is complete; a new token every launch, so the word needs no reset.
constexpr int kStepListMax = 512;                 // list slots one attention split holds in LDS
constexpr uint64_t kStepWaitTicks = 50000000ull;  // 0.5 s of the 100 MHz clock: the list wait's bound
struct StepArgs {
  ScanArgs idx;       // idx.a: the scores and selection (coop); no append row
  AttendArgs att;     // the attention (list mode) and the append
  uint32_t token;     // nonzero
  int32_t n_queries;  // B * Tq
  int32_t n_idx;      // n_queries * n_cols, rounded up to a multiple of 8
  int32_t n_att;      // n_queries * head groups * splits
};
static_assert(sizeof(StepArgs) <= 4096, "kernel arguments beyond 4 KiB");
hipError_t launch_csa_step(const StepArgs& sa, hipStream_t s);
hipError_t launch_attend(const AttendArgs& args, int32_t B, int mode, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int32_t B, hipStream_t s);

}  // namespace lca
