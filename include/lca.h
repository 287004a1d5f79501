/*
 * lca.h -- C ABI of liblca.so: hybrid compressed long-context attention
 * (CSA / HCA compressed KV cache + sliding window) on AMD gfx950 (MI355X).
 *
 * The method is the one the pages describe in "DeepSeek-V4: a million-token
 * context that agents can actually use" (molayo1419.me rendering of the
 * Hugging Face blog): CSA paragraph and Figure 3 (KV entries compressed 4x by
 * softmax-gated pooling with a learned positional bias; an FP4 lightning
 * indexer, a ReLU-scored multi-head dot product, picks the top-k compressed
 * blocks per query; a sliding-window branch covers the recent uncompressed
 * tokens), HCA paragraph and Figure 4 (128x compression, no selection, dense
 * attention over the compressed stream plus the same window), and the
 * storage paragraph (FP8 KV entries, BF16 RoPE dims, FP4 indexer). The cache
 * layout -- a compressed cache, a separate sliding-window state and a
 * separately managed uncompressed tail -- follows the KV-cache section of
 * velog.io "DeepSeek V4 논문 정리".
 *
 * Conventions for every entry point:
 *  - All pointers named *_dev are device pointers; the caller owns every
 *    byte (allocate, keep alive until the stream is done, free). The library
 *    never allocates, frees or synchronises.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *    the call returns at once. Kernel faults surface at the caller's next
 *    synchronisation.
 *  - Arguments are checked on the host before anything is launched; a bad
 *    argument returns a negative status and launches nothing.
 *  - BF16 tensors are passed as uint16_t bit patterns; every tensor is dense
 *    row-major with the shape written next to it; B = batch of the cache.
 *  - Every sequence of a cache holds the same number of tokens (`len`),
 *    except through the ragged calls (lca_ragged_*), where the caller
 *    passes each sequence's length with every call.
 *  - A cache (and a workspace) is not thread-safe; distinct caches are
 *    independent.
 *
 * Entry (196 bytes, one per compressed block and one per window token):
 *   64 "nope" dims as FP8 E4M3FN codes + one fp32 scale, 64 RoPE dims BF16.
 * Indexer key (34 bytes, CSA): 64 dims as FP4 E2M1 (two per byte, element
 *   2i in the low nibble) + two E8M0 scale bytes (one per 32 dims).
 */
#ifndef LCA_H
#define LCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lca_status;
#define LCA_OK 0
#define LCA_ERR_NULL (-1)        /* a required pointer is NULL */
#define LCA_ERR_SHAPE (-2)       /* a size is out of range or inconsistent */
#define LCA_ERR_UNSUPPORTED (-3) /* a descriptor value this library does not implement */
#define LCA_ERR_CAPACITY (-4)    /* the cache or the window state is too small for the call */
#define LCA_ERR_ORDER (-5)       /* compress / append called out of order */
#define LCA_ERR_WORKSPACE (-6)   /* workspace missing or smaller than lca_workspace_bytes() */
#define LCA_ERR_LAUNCH (-7)      /* the HIP runtime rejected a launch */

#define LCA_KIND_CSA 0
#define LCA_KIND_HCA 1
/* Window-only layer: the sliding window and nothing else (the layer
 * interleave paragraph: the final MTP block of V4-Pro's stack runs only the
 * sliding window). Its cache holds the window state alone. */
#define LCA_KIND_SWA 2

#define LCA_HEAD_DIM 128 /* shared KV head: 64 nope + 64 RoPE dims */
#define LCA_NOPE_DIM 64
#define LCA_ROPE_DIM 64
#define LCA_IDX_DIM 64   /* lightning-indexer head dim */

/* One attention layer. Supported: kind CSA, HCA or SWA; 1 <= n_heads <= 64;
 * 1 <= window <= 4096; CSA and HCA: 1 <= m <= 128; CSA: 1 <= idx_heads <= 8
 * and 1 <= topk <= 2048 (both ignored for HCA and SWA; m ignored for SWA:
 * the bound cache stores m = 1, idx_heads = topk = 0). */
typedef struct lca_layer_desc {
  int32_t kind;      /* LCA_KIND_CSA, LCA_KIND_HCA or LCA_KIND_SWA */
  int32_t m;         /* tokens pooled into one entry (CSA 4, HCA 128 on the pages) */
  int32_t n_heads;   /* query heads, dim 128, all sharing the one KV head */
  int32_t window;    /* W: sliding-window length in tokens, the query included */
  int32_t idx_heads; /* CSA: lightning-indexer query heads, dim 64 */
  int32_t topk;      /* CSA: compressed blocks kept per query */
} lca_layer_desc;

/* A bound cache. Fill it with lca_cache_bind(); the library updates `len`
 * and `pending`; every other field is read-only for the caller. */
typedef struct lca_cache {
  lca_layer_desc desc;
  int32_t batch;      /* B */
  int32_t ring;       /* R: window-state slots per sequence (token s lives in slot s mod R) */
  int64_t max_ctx;    /* token capacity per sequence */
  int64_t max_blocks; /* max_ctx / m (0 for SWA) */
  int64_t len;        /* tokens appended so far (same for every sequence) */
  int64_t pending;    /* tokens compressed but not yet appended (0 or T) */
  /* compressed cache (D1): [B][max_blocks][64] u8, [B][max_blocks] f32, [B][max_blocks][64] bf16;
   * NULL for SWA */
  uint8_t* blk_codes_dev;
  float* blk_scale_dev;
  uint16_t* blk_rope_dev;
  /* CSA indexer keys (D3): [B][max_blocks][32] u8 (FP4 pairs), [B][max_blocks][2] u8 (E8M0); NULL for HCA */
  uint8_t* idx_codes_dev;
  uint8_t* idx_scale_dev;
  /* sliding-window state (D2): [B][R][64] u8, [B][R] f32, [B][R][64] bf16 */
  uint8_t* win_codes_dev;
  float* win_scale_dev;
  uint16_t* win_rope_dev;
  /* uncompressed tail: [B][m][tail_width] bf16, token p in slot p mod m;
   * tail_width = 128 (kv) + 128 (gate) [+ 64 (ik) + 64 (ig) for CSA]; NULL and 0 for SWA */
  uint16_t* tail_dev;
  int32_t tail_width;
  int32_t ragged;     /* 1 once a ragged call (lca_ragged_*) used the cache: it then tracks no len */
  /* RoPE frequencies 10000^(-2i/64), i < 32, computed on the host at bind */
  double rope_inv_freq[32];
  /* their device copy (256 B at the end of the cache memory), what the kernels read */
  double* rope_inv_freq_dev;
} lca_cache;

/* Bytes of device memory lca_cache_bind() carves for one layer:
 * D1 (196 B/block) + D3 (34 B/block, CSA) + D2 (196 B/slot) + tail + the
 * 256-B RoPE frequency table, each array 256-byte aligned. max_blocks = max_ctx / m; SWA: D2 and the
 * table only. Returns 0 for an invalid descriptor or size. */
size_t lca_cache_bytes(const lca_layer_desc* desc, int32_t batch, int64_t max_ctx, int32_t ring);

/* Carve `base_dev` (>= lca_cache_bytes() bytes, 256-byte aligned) into the
 * arrays above, zero them on `stream`, set len = pending = 0 and fill the
 * RoPE frequencies (host array, and its device copy, written on `stream`). ring >= window; to let Tq queries attend in one call
 * (chunked prefill), ring >= Tq + window - 1. */
lca_status lca_cache_bind(const lca_layer_desc* desc, lca_cache* cache, void* base_dev, size_t bytes,
                          int32_t batch, int64_t max_ctx, int32_t ring, void* stream);

/* Scratch one call of lca_csa_indexer_topk / lca_csa_attend /
 * lca_csa_sparse_attn / lca_hca_dense_attn needs for up to max_tq queries per sequence at up to
 * max_ctx tokens. It holds counters of the attention's key splits and, for
 * CSA, a 16 KiB histogram per query, all of which must be zero when a call
 * starts: zero the workspace once with lca_workspace_init() before its first
 * use; every completed call leaves them zero again (an lca_csa_index_score
 * without its selection excepted, see below). Everything else in it is
 * rewritten by each call. A workspace may be shared by caches of the same or
 * smaller shape; calls sharing one workspace must not overlap in time.
 * lca_csa_sparse_attn and lca_hca_dense_attn also accept ws_dev = NULL (they
 * then use fewer, longer workgroups for few queries). */
size_t lca_workspace_bytes(const lca_layer_desc* desc, int32_t batch, int32_t max_tq, int64_t max_ctx);
lca_status lca_workspace_init(void* ws_dev, size_t bytes, void* stream);

/* Where the indexer leaves its scores (CSA): after lca_csa_index_score (or
 * lca_csa_indexer_topk / lca_csa_attend with B*Tq < 2048 or more than 65535
 * visible blocks) on a cache of this shape, the workspace holds at this byte
 * offset the row of max_ctx/m uint32 keys of query `query` (= b*Tq + i),
 * valid for its visible blocks j < (t+1)/m: key = bits(score) ^ (score < 0 ?
 * 0xFFFFFFFF : 0x80000000), so keys order like the scores. Written only when
 * some query of the call sees more than topk blocks. (The combined calls with
 * more queries score in query tiles and keep only the selection's
 * candidates.) Returns 0 for HCA or invalid arguments. */
size_t lca_workspace_scores_offset(const lca_layer_desc* desc, int32_t batch, int32_t query, int64_t max_ctx);

/* CSA compressor (CSA paragraph and Figure 3: every m = 4 tokens pooled into
 * one entry by softmax-gated pooling with a learned positional bias).
 * Consumes the tail plus T new tokens at positions len .. len+T-1 and writes
 * the D1 entry and the D3 indexer key of every block that these tokens
 * complete. Per block j and channel c:
 *   a_i = softmax_i(gate[jm+i][c] + bias[i][c]),  y_c = sum_i a_i * key_i[c]
 * where key_i is the token's kv with dims 64..127 RoPE-rotated at the
 * token's own position; the indexer key pools ik with ig and idx_bias the
 * same way (no RoPE) and is stored as MX-FP4.
 *   kv_dev, gate_dev: [B][T][128] bf16; ik_dev, ig_dev: [B][T][64] bf16;
 *   bias_dev: [m][128] f32; idx_bias_dev: [m][64] f32.
 * Must be followed by lca_swa_tail_append() with the same tokens before the
 * next compress (LCA_ERR_ORDER otherwise); len + T <= max_ctx. */
lca_status lca_csa_compress(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                            const uint16_t* ik_dev, const uint16_t* ig_dev, const float* bias_dev,
                            const float* idx_bias_dev, int32_t T, void* stream);

/* HCA compressor (HCA paragraph and Figure 4: the same pooling at m = 128,
 * no indexer key). Arguments as lca_csa_compress without ik/ig/idx_bias. */
lca_status lca_hca_compress(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                            const float* bias_dev, int32_t T, void* stream);

/* Sliding-window state and uncompressed tail (Figure 3's sliding-window
 * branch; the KV-cache section's separate window state and separately
 * managed tail). Writes the window entry of each of the T tokens (its kv,
 * dims 64..127 RoPE-rotated at its position, FP8/BF16-encoded with its own
 * scale) into slot s mod R (only the last R tokens of a long call survive),
 * keeps the BF16 inputs of the tokens of the not yet complete block in the
 * tail, and advances len by T. Same input layout as the compressor; ik/ig
 * are NULL for HCA. Requires the preceding compress of exactly these T
 * tokens. SWA: no compressor and no tail; only kv is read (gate, ik, ig may
 * be NULL) and no compress precedes. */
lca_status lca_swa_tail_append(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                               const uint16_t* ik_dev, const uint16_t* ig_dev, int32_t T, void* stream);

/* CSA lightning indexer + per-query top-k (CSA paragraph: FP4, ReLU-scored
 * multi-head dot product; the top-k compressed blocks per query). The
 * queries are the last Tq appended tokens, positions len-Tq .. len-1; query
 * t sees blocks j < (t+1)/m (the block's last token at or before t). Per
 * visible block:
 *   s_h = fp32( <MXFP4(qI_h), key_j> ),  score_j = sum_h w_h * max(s_h, 0)
 * (a chain of fmaf over h = 0..idx_heads-1 from +0). topk_dev receives the
 * min(k, visible) blocks with the largest (score, -j), in ascending j,
 * padded with -1.
 *   qI_dev: [B][Tq][idx_heads][64] bf16; w_dev: [B][Tq][idx_heads] f32;
 *   topk_dev: [B][Tq][k] int32. B * Tq <= 65535 (else LCA_ERR_SHAPE). */
lca_status lca_csa_indexer_topk(lca_cache* cache, const uint16_t* qI_dev, const float* w_dev, int32_t Tq,
                                int32_t* topk_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* The two method steps of lca_csa_indexer_topk as separate calls (same
 * arguments; the scores travel in the workspace, so both calls must get the
 * same cache state, Tq and workspace, in this order, with nothing else using
 * the workspace in between; an lca_csa_index_score without its
 * lca_csa_topk_select leaves the workspace histograms counting it: the next
 * selection is then slower, still exact, and clears them):
 *  lca_csa_index_score: the lightning-indexer scores of every visible block
 *    of the Tq queries (an HBM stream over the FP4 keys; with B*Tq >= 2048
 *    queries that each see at most 65535 blocks, query tiles of 8 that also
 *    leave the selection's candidates);
 *  lca_csa_topk_select: the per-query top-k of those scores into topk_dev. */
lca_status lca_csa_index_score(lca_cache* cache, const uint16_t* qI_dev, const float* w_dev, int32_t Tq,
                               void* ws_dev, size_t ws_bytes, void* stream);
lca_status lca_csa_topk_select(lca_cache* cache, int32_t Tq, int32_t* topk_dev, void* ws_dev, size_t ws_bytes,
                               void* stream);

/* CSA sparse attention (Figure 3): per query t and head h, one softmax over
 * the multiset {D1 entries selected by topk} + {window entries of positions
 * max(0, t-W+1) .. t}; K = V = the dequantised 128-dim entry; logits
 * RoPE(q_h, t) . x / sqrt(128). Entries of -1 in topk are skipped.
 *   q_dev: [B][Tq][n_heads][128] bf16 (not rotated); topk_dev: [B][Tq][k];
 *   out_dev: [B][Tq][n_heads][128] bf16; lse_dev: [B][Tq][n_heads] f32
 *   (natural-log log-sum-exp of the logits) or NULL. */
lca_status lca_csa_sparse_attn(lca_cache* cache, const uint16_t* q_dev, const int32_t* topk_dev, int32_t Tq,
                               uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* HCA dense attention (HCA paragraph and Figure 4): as lca_csa_sparse_attn
 * over every visible D1 entry j < (t+1)/m plus the window. */
lca_status lca_hca_dense_attn(lca_cache* cache, const uint16_t* q_dev, int32_t Tq, uint16_t* out_dev,
                              float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* Window-only attention of an SWA cache (layer interleave paragraph: the
 * final MTP block runs only the sliding window): per query t and head h, one
 * softmax over the window entries of positions max(0, t-W+1) .. t; logits,
 * K = V and outputs as lca_csa_sparse_attn. ws_dev may be NULL (W <= 768
 * never splits a query's keys). */
lca_status lca_swa_attn(lca_cache* cache, const uint16_t* q_dev, int32_t Tq, uint16_t* out_dev, float* lse_dev,
                        void* ws_dev, size_t ws_bytes, void* stream);

/* One decode step of an HCA layer in one call: the T new tokens of every
 * sequence go in (lca_hca_compress for the blocks they complete, then the
 * window entries and tail copies of lca_swa_tail_append) and their T
 * queries attend (lca_hca_dense_attn): the same cache bytes and outputs as
 * those calls. One launch, two when a block completes: the append runs in
 * the attention launch (each workgroup that reads the window writes the new
 * entries itself before reading them back). For decode-sized calls:
 * B * T <= 511 (else LCA_ERR_SHAPE); ring >= T + window - 1. Arguments as
 * the three calls; lse_dev and ws_dev may be NULL. Checks everything before
 * launching: a rejected call leaves the cache unchanged. */
lca_status lca_hca_step(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev, const float* bias_dev,
                        int32_t T, const uint16_t* q_dev, uint16_t* out_dev, float* lse_dev, void* ws_dev,
                        size_t ws_bytes, void* stream);

/* One decode step of a window-only layer (the final MTP block): the T new
 * tokens' window entries (lca_swa_tail_append) and their queries' window
 * attention (lca_swa_attn) in one launch; the same results as the two
 * calls. Limits and checks as lca_hca_step. */
lca_status lca_swa_step(lca_cache* cache, const uint16_t* kv_dev, int32_t T, const uint16_t* q_dev,
                        uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* The CSA query path with the selection and the attention in one launch
 * (CSA paragraph: top-k compressed blocks per query; Figure 3: their
 * attention joined with the sliding-window branch under one softmax).
 * Results are those of lca_csa_indexer_topk followed by lca_csa_sparse_attn
 * on the same arguments: the same top-k lists bit for bit, attention outputs
 * equal up to fp32 summation order.
 *  lca_csa_attend: indexer scores, top-k and attention of the Tq queries
 *    (three kernels: score, candidate scan, selection + attention).
 *  lca_csa_topk_attn: the same after a separate lca_csa_index_score with the
 *    same cache state, Tq and workspace.
 * topk_dev ([B][Tq][k] int32) may be NULL when the lists are not wanted.
 * Every workgroup of the last kernel selects its query's list itself (one
 * per 16 heads): meant for decode-sized Tq; large Tq (chunked prefill) is
 * cheaper through the separate calls. Workspace and histogram rules as for
 * lca_csa_indexer_topk; ring >= Tq + window - 1. */
lca_status lca_csa_attend(lca_cache* cache, const uint16_t* qI_dev, const float* w_dev, const uint16_t* q_dev,
                          int32_t Tq, int32_t* topk_dev, uint16_t* out_dev, float* lse_dev, void* ws_dev,
                          size_t ws_bytes, void* stream);
lca_status lca_csa_topk_attn(lca_cache* cache, const uint16_t* q_dev, int32_t Tq, int32_t* topk_dev,
                             uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* One decode step of a CSA layer in one call: the T new tokens of every
 * sequence go in (lca_csa_compress + lca_swa_tail_append: the blocks they
 * complete are pooled into D1/D3, their window entries and tail copies are
 * written) and their T queries attend (lca_csa_attend): same results, bit for
 * bit in the cache and the top-k lists. One launch (two when a block
 * completes: compress first): workgroups that score every visible block (a
 * workgroup per 2048 blocks of each query, each keeping its best candidates),
 * the last of each query to finish selecting its top-k, and after them in the
 * same grid the attention workgroups, each of which waits for its query's
 * list (the append rides with them). With the environment variable
 * LCA_STEP_UNFUSED set, or when a query's key split would exceed 512 keys,
 * the indexer and the attention take a launch each (the same results, bit for
 * bit). (Queries seeing more than 1M blocks, or k too large for a query's
 * chunks, take three: score, candidate scan with the append, selection +
 * attention.) For decode-sized calls: B * T <= 511
 * (else LCA_ERR_SHAPE); ring >= T + window - 1. Inputs as for the compressor
 * and lca_csa_attend; topk_dev and lse_dev may be NULL. Checks everything
 * before launching: a rejected call leaves the cache unchanged. */
lca_status lca_csa_step(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev, const uint16_t* ik_dev,
                        const uint16_t* ig_dev, const float* bias_dev, const float* idx_bias_dev, int32_t T,
                        const uint16_t* qI_dev, const float* w_dev, const uint16_t* q_dev, int32_t* topk_dev,
                        uint16_t* out_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* lca_csa_step with timing marks, for measuring the step's kernels one by
 * one: the same launches and results, plus hipEventRecord on `stream` of
 * events[0] before the compress launch (when a block completes), events[1]
 * before the indexer launch, events[2] after it (after the candidate scan
 * on the three-launch path) and events[3] after the attention (on the
 * one-launch path events[2] and events[3] both follow the step's launch). events is a
 * host array of 4 hipEvent_t (entries may be NULL: not recorded), owned by
 * the caller; events == NULL is LCA_ERR_NULL. The marks sit between the
 * launches, so they separate kernels that would otherwise follow each other
 * directly. */
lca_status lca_csa_step_timed(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                              const uint16_t* ik_dev, const uint16_t* ig_dev, const float* bias_dev,
                              const float* idx_bias_dev, int32_t T, const uint16_t* qI_dev, const float* w_dev,
                              const uint16_t* q_dev, int32_t* topk_dev, uint16_t* out_dev, float* lse_dev,
                              void* ws_dev, size_t ws_bytes, void* stream, void* const* events);

/* The kernel launches lca_csa_step would make for T tokens per sequence on
 * this cache and workspace, after the compress launch of a step whose
 * tokens complete a block: 1 (the indexer and the attention in one launch),
 * 2 (the indexer's launch, then the attention's) or 3 (score, candidate scan
 * with the append, selection + attention), in *launches. Launches nothing
 * and changes nothing; the same checks as lca_csa_step on the cache, T and
 * the workspace (its status when they fail). For tools that time or
 * profile the step's kernels. */
lca_status lca_csa_step_launches(const lca_cache* cache, int32_t T, void* ws_dev, size_t ws_bytes,
                                 int32_t* launches);

/* lca_csa_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same launches and results as lca_csa_step (bit for bit), with the
 * workspace taken from a 32 MiB device array inside the library instead of
 * the caller's: one array per GPU the library runs on, held until the
 * process ends. The call allocates nothing; the caller still passes every
 * input and output. Its first call on a device (and any call whose
 * workspace layout -- batch, T, max_ctx, layer -- differs from the previous
 * call's on that device) first clears the bytes it uses with a fill kernel
 * on `stream`. Limits: lca_workspace_bytes(desc, B, T, max_ctx) must not
 * exceed 32 MiB (else LCA_ERR_WORKSPACE, nothing launched): a 1M-token
 * context at B = 4 and T = 1 fits. Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. qI_dev and w_dev are
 * required. */
lca_status lca_csa_step_noalloc(lca_cache* cache, const uint16_t* kv_dev, const uint16_t* gate_dev,
                                const uint16_t* ik_dev, const uint16_t* ig_dev, const float* bias_dev,
                                const float* idx_bias_dev, int32_t T, const uint16_t* qI_dev, const float* w_dev,
                                const uint16_t* q_dev, int32_t* topk_dev, uint16_t* out_dev, float* lse_dev,
                                void* stream);

/* ---- persistence: snapshot and restore of one sequence's state ----------
 * The KV-cache section of velog.io "DeepSeek V4 논문 정리" keeps compressed KV
 * on disk for requests that share a prefix. A snapshot is a contiguous
 * buffer holding one sequence's whole state at its current length: its
 * compressed entries (D1), indexer keys (D3, CSA), window entries in
 * position order and uncompressed tail rows, behind a 256-byte header that
 * starts with a copy of lca_snapshot_info. The buffer is device memory; the
 * caller moves it to host memory or disk and back as plain bytes. Restoring
 * it into a cache gives that cache exactly the state (bit for bit in every
 * entry a later call reads) of one that ingested the same tokens, so a shared
 * prefix is compressed once and restored into any number of sequences, which
 * then continue with their own tokens. */
#define LCA_SNAPSHOT_MAGIC 0x5341434Cu /* "LCAS" */
#define LCA_SNAPSHOT_VERSION 1u
#define LCA_SNAPSHOT_HEADER 256

typedef struct lca_snapshot_info {
  uint32_t magic;     /* LCA_SNAPSHOT_MAGIC */
  uint32_t version;   /* LCA_SNAPSHOT_VERSION */
  int32_t kind;       /* layer kind of the cache it came from */
  int32_t m;          /* its m (1 for SWA) */
  int32_t tail_width; /* its tail row width in BF16 values (0 for SWA) */
  int32_t reserved;
  int64_t len;        /* tokens of the sequence */
  int64_t n_blocks;   /* compressed entries 0 .. n_blocks-1 (len / m; 0 for SWA) */
  int64_t n_win;      /* window entries of positions len-n_win .. len-1 (min(len, ring)) */
  int64_t n_tail;     /* tail rows of positions len-n_tail .. len-1 (len mod m; 0 for SWA) */
  /* byte offsets in the buffer, each 256-aligned: D1 codes [n_blocks][64] u8, D1 scales [n_blocks] f32,
   * D1 RoPE [n_blocks][64] bf16, D3 codes [n_blocks][32] u8, D3 scales [n_blocks][2] u8, window codes
   * [n_win][64] u8, window scales [n_win] f32, window RoPE [n_win][64] bf16, tail [n_tail][tail_width]
   * bf16, end; sections a kind does not have are empty */
  uint64_t off[10];
  uint64_t bytes;     /* total bytes of the snapshot (= off[9]) */
} lca_snapshot_info;

/* Layout of a snapshot of any sequence of `cache` at its current length:
 * fills *info (bytes included) without touching the device. LCA_ERR_ORDER
 * while a compress waits for its append. */
lca_status lca_snapshot_layout(const lca_cache* cache, lca_snapshot_info* info);

/* Copies sequence `seq` (0 <= seq < B) of `cache` into dst_dev (>= info->bytes
 * device bytes, 256-byte aligned) on `stream` -- the header included -- and
 * fills *info as lca_snapshot_layout does. The cache is not changed. */
lca_status lca_cache_snapshot(const lca_cache* cache, int32_t seq, void* dst_dev, size_t bytes,
                              lca_snapshot_info* info, void* stream);

/* Restores the snapshot in src_dev (described by *info, the header the
 * snapshot wrote or the info its lca_cache_snapshot returned) into sequence
 * `seq` of `cache`, or into every sequence when seq = -1. The cache must have
 * the snapshot's kind, m and tail width, room for its length and a window
 * the snapshot covers (n_win >= min(len, window)); every sequence of a cache
 * holds the same number of tokens, so seq = -1 needs len = 0 or
 * len = info->len and seq >= 0 needs len = info->len (or batch = 1); the
 * cache's len becomes info->len. A ragged cache takes any sequence at any
 * length and keeps len = 0 (the caller's len[seq] becomes info->len). Rejected headers (magic, version, sizes,
 * offsets that do not match the layout) return LCA_ERR_UNSUPPORTED or
 * LCA_ERR_SHAPE and change nothing. */
lca_status lca_cache_restore(lca_cache* cache, int32_t seq, const void* src_dev, size_t bytes,
                             const lca_snapshot_info* info, void* stream);

/* ---- ragged batches (continuous batching) ---------------------------------
 * Sequences of one cache at different lengths, each adding its own number
 * of tokens per call. As serving engines do, the caller tracks the lengths:
 * every ragged call gets len[b] (tokens sequence b holds before the call)
 * and T[b] (tokens it adds, 0 <= T[b] <= T_max; 0 leaves the sequence
 * untouched), both on the host (checks, launch sizes) and on the device (the
 * kernels), with equal contents; afterwards the caller adds T[b] to len[b].
 * Inputs, queries and outputs keep the [B][T_max][...] layout with sequence
 * b's rows 0 .. T[b]-1 in use; other rows are neither read nor written. The
 * first ragged call marks the cache ragged (it must be empty then); from
 * then on its len stays 0, the uniform calls reject it (LCA_ERR_ORDER), and
 * lca_ragged_snapshot takes a sequence's length from the caller. Restoring a
 * snapshot into a sequence of a ragged cache works at any length (the
 * caller's len[b] becomes the snapshot's len). Results per sequence are
 * those of a uniform cache holding that sequence alone (CSA paragraph,
 * Figures 3 and 4 of "DeepSeek-V4: a million-token context that agents can
 * actually use"). */

/* The compressor and the window / tail append for the T[b] new tokens of
 * every sequence (lca_csa_compress / lca_hca_compress followed by
 * lca_swa_tail_append, per sequence); no queries. Any T_max (chunked
 * prefill of newly admitted sequences). Inputs as for the uniform calls;
 * gate, ik, ig, bias, idx_bias may be NULL where the layer kind has no use
 * for them. */
lca_status lca_ragged_ingest(lca_cache* cache, int32_t T_max, const int64_t* len_host, const int32_t* T_host,
                             const int64_t* len_dev, const int32_t* T_dev, const uint16_t* kv_dev,
                             const uint16_t* gate_dev, const uint16_t* ik_dev, const uint16_t* ig_dev,
                             const float* bias_dev, const float* idx_bias_dev, void* stream);

/* One continuous-batching step of any layer kind: lca_ragged_ingest, then
 * the queries of the new tokens (positions len[b] .. len[b]+T[b]-1) attend:
 * CSA as lca_csa_step (indexer scores, top-k, sparse + window attention),
 * HCA as lca_hca_dense_attn, SWA as lca_swa_attn. qI, w and topk are CSA's
 * (topk and lse may be NULL); B * T_max <= 511 (else LCA_ERR_SHAPE);
 * ring >= T_max + window - 1; the workspace (sized for max_tq >= T_max) is
 * required for CSA, optional otherwise. */
lca_status lca_ragged_step(lca_cache* cache, int32_t T_max, const int64_t* len_host, const int32_t* T_host,
                           const int64_t* len_dev, const int32_t* T_dev, const uint16_t* kv_dev,
                           const uint16_t* gate_dev, const uint16_t* ik_dev, const uint16_t* ig_dev,
                           const float* bias_dev, const float* idx_bias_dev, const uint16_t* qI_dev,
                           const float* w_dev, const uint16_t* q_dev, int32_t* topk_dev, uint16_t* out_dev,
                           float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* lca_ragged_step with the lengths on the device only, for a step captured
 * once in a HIP graph and replayed: the call reads no length on the host.
 * Its launches are sized for any step of T[b] <= T_max tokens that ends at
 * or below cap_len tokens (T_max <= cap_len <= max_ctx): grids for cap_len,
 * the compress launch every time (at most ceil(T_max / m) blocks per
 * sequence), the largest append; each kernel takes sequence b's length and
 * token count from len_dev[b] and T_dev[b] when it runs. At the end of the
 * step the attention launch adds T[b] to len_dev[b] on the device, so every
 * replay takes the next tokens (T_dev may change between replays). A
 * sequence whose len + T[b] would exceed cap_len takes no step: its len
 * stays, its rows are neither read nor written. len_dev (int64 [B], device,
 * read and written) and T_dev (int32 [B], device) are the caller's, as are
 * every input and output (fixed addresses: a replay reads and writes the
 * same buffers, refilled by the caller between replays). The workspace
 * (lca_workspace_bytes for max_tq >= T_max) is required for every kind: the
 * launch's length-advance counter lives in it. The results are those of
 * lca_ragged_step at the same lengths; bit for bit where the attention's
 * key splits, which follow the launch sizes (here cap_len), are the same
 * (tested against lca_csa_step and lca_hca_step on an equal cache, replay
 * after replay), else within rounding. Checks as there, with cap_len <
 * T_max or > max_ctx: LCA_ERR_CAPACITY; the cache must be ragged or empty.
 * Enqueues no memset and no host synchronisation: capturable. */
lca_status lca_ragged_step_graph(lca_cache* cache, int32_t T_max, int64_t cap_len, int64_t* len_dev,
                                 const int32_t* T_dev, const uint16_t* kv_dev, const uint16_t* gate_dev,
                                 const uint16_t* ik_dev, const uint16_t* ig_dev, const float* bias_dev,
                                 const float* idx_bias_dev, const uint16_t* qI_dev, const float* w_dev,
                                 const uint16_t* q_dev, int32_t* topk_dev, uint16_t* out_dev, float* lse_dev,
                                 void* ws_dev, size_t ws_bytes, void* stream);

/* lca_cache_snapshot for a sequence of a ragged cache that holds `len`
 * tokens (the caller's len[seq]). With dst_dev = NULL it only fills *info
 * (the layout, for sizing the buffer). */
lca_status lca_ragged_snapshot(const lca_cache* cache, int32_t seq, int64_t len, void* dst_dev, size_t bytes,
                               lca_snapshot_info* info, void* stream);

/* Human-readable name of a status code (static storage). */
const char* lca_status_str(lca_status status);

#ifdef __cplusplus
}
#endif

#endif /* LCA_H */
