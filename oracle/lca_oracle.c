/*
 * lca_oracle.c -- plain, slow CPU oracle for hybrid compressed attention
 * (CSA / HCA compressed KV + sliding window), TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the smoke check and the CPU-baseline leg of the benchmark may
 * load this file's library. The GPU library never links it and it never
 * links the GPU library; the two share no header, helper or constant.
 *
 * Everything is scalar fp64 (or the exact integer / IEEE-rounded operation
 * named in each comment), built with -O2 -fno-fast-math -ffp-contract=off so
 * that every `+ - * /` below is one correctly rounded IEEE operation.
 *
 * What it follows (the method is described in prose on the pages; where a
 * step is left open, the reading taken is stated at the function):
 *  - "DeepSeek-V4: a million-token context that agents can actually use"
 *    (molayo1419.me rendering of the Hugging Face blog), CSA paragraph and
 *    Figure 3: every 4 tokens are pooled into one compressed KV entry by
 *    softmax-gated pooling with a learned positional bias; an FP4 lightning
 *    indexer (ReLU-scored multi-head dot product) picks the top-k compressed
 *    blocks per query; a sliding-window branch covers the most recent
 *    uncompressed tokens.
 *  - same page, HCA paragraph and Figure 4: 128x compression, no sparse
 *    selection, dense attention over the compressed stream plus the window.
 *  - same page, storage paragraph: most KV entries FP8, RoPE dims BF16,
 *    indexer FP4.
 *  - velog.io "DeepSeek V4 논문 정리", KV-cache section: compressed cache,
 *    separate sliding-window state, separately managed uncompressed tail.
 *
 * Parity unpinned (self-consistency only, the pages give nothing numeric):
 * the RoPE base / pairing, per-channel gates, RoPE-before-pooling, the
 * indexer key stream derivation, the indexer weighting form, and the FP4
 * scale rule. Each such function says so.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HEAD_DIM 128
#define NOPE_DIM 64
#define ROPE_DIM 64
#define IDX_DIM 64

/* ------------------------------------------------------------------ */
/* exp used inside pooling: Cody & Waite additive argument reduction   */
/* (Cody & Waite, Software Manual for the Elementary Functions, 1980)  */
/* followed by the degree-13 Taylor polynomial in Horner form with     */
/* explicit fma.  Only correctly rounded operations are used, so any   */
/* host that runs the same operation sequence gets the same bits.      */
/* Constants: 1/ln2 rounded to nearest; ln2 split into a 32-significant */
/* -bit head (so n*LN2_HI is exact for |n| < 2^21) and the rounded     */
/* remainder; Taylor coefficients are 1/i! rounded to nearest.         */
/* ------------------------------------------------------------------ */
static const double O_INV_LN2 = 0x1.71547652b82fep+0;
static const double O_LN2_HI = 0x1.62e42ff000000p-1;
static const double O_LN2_LO = -0x1.718432a1b0e26p-35;
static const double O_TAYLOR[14] = {
    0x1.0000000000000p+0, 0x1.0000000000000p+0, 0x1.0000000000000p-1,
    0x1.5555555555555p-3, 0x1.5555555555555p-5, 0x1.1111111111111p-7,
    0x1.6c16c16c16c17p-10, 0x1.a01a01a01a01ap-13, 0x1.a01a01a01a01ap-16,
    0x1.71de3a556c734p-19, 0x1.27e4fb7789f5cp-22, 0x1.ae64567f544e4p-26,
    0x1.1eed8eff8d898p-29, 0x1.6124613a86d09p-33};

double lcao_exp_det(double x) {
  if (x < -700.0) return 0.0;
  double n = nearbyint(x * O_INV_LN2);
  double r = (x - n * O_LN2_HI) - n * O_LN2_LO;
  double p = O_TAYLOR[13];
  for (int i = 12; i >= 0; --i) p = fma(p, r, O_TAYLOR[i]);
  return ldexp(p, (int)n);
}

void lcao_exp_consts(double* out /* 17 */) {
  out[0] = O_INV_LN2;
  out[1] = O_LN2_HI;
  out[2] = O_LN2_LO;
  for (int i = 0; i < 14; ++i) out[3 + i] = O_TAYLOR[i];
}

/* ------------------------------------------------------------------ */
/* Number formats (storage paragraph of the molayo1419.me page: FP8    */
/* entries, BF16 RoPE dims, FP4 indexer).  The exact variants are a     */
/* reading: OCP FP8 E4M3FN, IEEE-style bfloat16, OCP MX FP4 E2M1 with   */
/* E8M0 block scales over 32 elements.  All encoders round to nearest,  */
/* ties to even, directly from the fp64 value (no intermediate fp32).   */
/* ------------------------------------------------------------------ */

/* E4M3FN: bias 7, 3 mantissa bits, subnormal quantum 2^-9, max 448, no inf,
 * S.1111.111 is NaN. Values at or beyond 448 in magnitude saturate. */
uint8_t lcao_fp8_encode(double v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  int e = (a < 0x1p-6) ? -6 : ilogb(a);
  double q = ldexp(1.0, e - 3);          /* spacing of representable values */
  double val = nearbyint(a / q) * q;     /* a/q exact (power-of-two divisor) */
  if (val == 0.0) return sign;
  if (val < 0x1p-6) return (uint8_t)(sign | (uint8_t)(val * 0x1p9));
  int E = ilogb(val);
  int M = (int)((val / ldexp(1.0, E) - 1.0) * 8.0);
  return (uint8_t)(sign | ((E + 7) << 3) | M);
}

double lcao_fp8_decode(uint8_t c) {
  int s = c >> 7, E = (c >> 3) & 15, M = c & 7;
  double v;
  if (E == 15 && M == 7) return NAN;
  if (E == 0) v = M * 0x1p-9;
  else v = (1.0 + M / 8.0) * ldexp(1.0, E - 7);
  return s ? -v : v;
}

/* bfloat16: 8 significant bits, fp32 exponent range, subnormal quantum 2^-133. */
uint16_t lcao_bf16_encode(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7FC0;
  if (a == 0.0) return sign;
  int e = ilogb(a);
  if (e < -126) e = -126;
  double q = ldexp(1.0, e - 7);
  double val = nearbyint(a / q) * q;
  if (val >= 0x1p128) return (uint16_t)(sign | 0x7F80);
  float f = (float)val; /* exact: val has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

float lcao_bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* E2M1: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; bit 3 is the sign.
 * Ties go to the even mantissa; magnitudes above 6 saturate to 6. */
uint8_t lcao_fp4_encode(double v) {
  uint8_t sign = signbit(v) ? 8 : 0;
  double a = fabs(v);
  if (a >= 6.0) return (uint8_t)(sign | 7);
  int e = (a < 1.0) ? 0 : ilogb(a);
  double q = ldexp(1.0, e - 1);
  double val = nearbyint(a / q) * q;
  if (val > 6.0) val = 6.0;
  if (val < 1.0) return (uint8_t)(sign | (uint8_t)(val * 2.0));
  int E = ilogb(val);
  int M = (int)((val / ldexp(1.0, E) - 1.0) * 2.0);
  return (uint8_t)(sign | ((E + 1) << 1) | M);
}

double lcao_fp4_decode(uint8_t c) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = mag[c & 7];
  return (c & 8) ? -v : v;
}

/* MX block quantisation of n values (n a multiple of 32): per block of 32,
 * E = clamp(floor(log2(amax)) - 2, -127, 127) (emax of E2M1 is 2), scale
 * byte = E + 127, code = E2M1(x * 2^-E). amax == 0 gives byte 0, codes 0.
 * codes: one code per byte (low nibble). Reading of "FP4 indexer" + the
 * per-32 scale in the workload description; parity unpinned beyond the
 * format definition. */
void lcao_mxfp4_quant(const double* x, int n, uint8_t* codes, uint8_t* scales) {
  for (int b = 0; b < n / 32; ++b) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
      double a = fabs(x[32 * b + i]);
      if (a > amax) amax = a;
    }
    if (amax == 0.0) {
      scales[b] = 0;
      for (int i = 0; i < 32; ++i) codes[32 * b + i] = 0;
      continue;
    }
    int E = ilogb(amax) - 2;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    scales[b] = (uint8_t)(E + 127);
    for (int i = 0; i < 32; ++i) codes[32 * b + i] = lcao_fp4_encode(ldexp(x[32 * b + i], -E));
  }
}

/* ------------------------------------------------------------------ */
/* RoPE on dims 64..127 (storage paragraph: RoPE dims are kept BF16).   */
/* Reading (parity unpinned): base 10000, interleaved pairs (2i, 2i+1)  */
/* of the 64 RoPE dims, angle p * 10000^(-2i/64), all fp64.             */
/* ------------------------------------------------------------------ */
void lcao_rope_inv_freq(double* inv_freq /* 32 */) {
  for (int i = 0; i < ROPE_DIM / 2; ++i) inv_freq[i] = pow(10000.0, -(double)(2 * i) / (double)ROPE_DIM);
}

void lcao_rope_rotate(double* x /* HEAD_DIM, in/out */, int64_t pos) {
  double inv_freq[ROPE_DIM / 2];
  lcao_rope_inv_freq(inv_freq);
  for (int i = 0; i < ROPE_DIM / 2; ++i) {
    double phi = (double)pos * inv_freq[i];
    double c = cos(phi), s = sin(phi);
    double x0 = x[NOPE_DIM + 2 * i], x1 = x[NOPE_DIM + 2 * i + 1];
    x[NOPE_DIM + 2 * i] = x0 * c - x1 * s;
    x[NOPE_DIM + 2 * i + 1] = x0 * s + x1 * c;
  }
}

/* ------------------------------------------------------------------ */
/* Softmax-gated pooling with a learned positional bias (CSA paragraph */
/* of the molayo1419.me page; Figure 3: m = 4 tokens per entry;        */
/* HCA paragraph / Figure 4 for 128).  Reading: per-channel gates,      */
/* bias[i][c] per position-in-block and channel, non-overlapping        */
/* blocks.  For each channel c:                                          */
/*   z_i = gate[i][c] + bias[i][c];  mu = max_i z_i;                     */
/*   e_i = exp_det(z_i - mu);  S = e_0 + e_1 + ... (ascending);          */
/*   a_i = e_i / S;  y_c = fma(a_{m-1}, v, ... fma(a_0, v_0, 0)).        */
/* weights (m x C, may be NULL) receives a_i.                            */
/* ------------------------------------------------------------------ */
void lcao_pool(int m, int C, const double* gate, const double* bias, const double* val, double* out,
               double* weights) {
  double* e = (double*)malloc(sizeof(double) * (size_t)m);
  for (int c = 0; c < C; ++c) {
    double mu = -INFINITY;
    for (int i = 0; i < m; ++i) {
      double z = gate[(size_t)i * C + c] + bias[(size_t)i * C + c];
      if (z > mu) mu = z;
    }
    double S = 0.0;
    for (int i = 0; i < m; ++i) {
      double z = gate[(size_t)i * C + c] + bias[(size_t)i * C + c];
      e[i] = lcao_exp_det(z - mu);
      S = S + e[i];
    }
    double y = 0.0;
    for (int i = 0; i < m; ++i) {
      double a = e[i] / S;
      if (weights) weights[(size_t)i * C + c] = a;
      y = fma(a, val[(size_t)i * C + c], y);
    }
    out[c] = y;
  }
  free(e);
}

/* ------------------------------------------------------------------ */
/* One 196-byte KV entry (storage paragraph): 64 "nope" dims as FP8     */
/* E4M3FN with one fp32 scale per entry, 64 RoPE dims as BF16.          */
/* scale = fp32(amax / 448); code = E4M3FN(x / scale). amax == 0 (or a  */
/* scale that rounds to 0) gives scale 0 and all-zero codes.            */
/* ------------------------------------------------------------------ */
void lcao_entry_encode(const double* x, uint8_t* nope, float* scale, uint16_t* rope) {
  double amax = 0.0;
  for (int c = 0; c < NOPE_DIM; ++c) {
    double a = fabs(x[c]);
    if (a > amax) amax = a;
  }
  float s = (float)(amax / 448.0);
  if (amax == 0.0 || s == 0.0f) {
    *scale = 0.0f;
    for (int c = 0; c < NOPE_DIM; ++c) nope[c] = 0;
  } else {
    *scale = s;
    for (int c = 0; c < NOPE_DIM; ++c) nope[c] = lcao_fp8_encode(x[c] / (double)s);
  }
  for (int c = 0; c < ROPE_DIM; ++c) rope[c] = lcao_bf16_encode(x[NOPE_DIM + c]);
}

/* Dequantised entry: nope value = fp32(decode(code) * scale) (one fp32
 * multiply), rope value = the BF16 value. */
void lcao_entry_decode(const uint8_t* nope, float scale, const uint16_t* rope, double* out) {
  for (int c = 0; c < NOPE_DIM; ++c) {
    float d = (float)lcao_fp8_decode(nope[c]);
    float p = d * scale;
    out[c] = (double)p;
  }
  for (int c = 0; c < ROPE_DIM; ++c) out[NOPE_DIM + c] = (double)lcao_bf16_decode(rope[c]);
}

/* ------------------------------------------------------------------ */
/* Compressor for one sequence: entries for blocks [j_begin, j_end).    */
/* Token arrays hold positions tok0 .. tok0+n_tok-1 (BF16 bits):         */
/*   kv[t][128], gate[t][128]; CSA also ik[t][64], ig[t][64] (else NULL) */
/* Block j covers tokens j*m .. j*m+m-1. Each token's key is RoPE'd at  */
/* its own position before pooling (reading: no block position is      */
/* invented). The CSA indexer key pools ik with ig and idx_bias, no     */
/* RoPE, then MX-FP4 (reading: its own pooled stream, one key head).    */
/* Outputs are indexed from j_begin:                                     */
/*   nope[(j-j_begin)*64], scale[j-j_begin], rope[(j-j_begin)*64],       */
/*   idx_codes[(j-j_begin)*64] (one code per byte), idx_scales[..*2].    */
/* ------------------------------------------------------------------ */
void lcao_compress(int m, const uint16_t* kv, const uint16_t* gate, const uint16_t* ik, const uint16_t* ig,
                   int64_t tok0, int64_t n_tok, const float* bias, const float* idx_bias, int64_t j_begin,
                   int64_t j_end, uint8_t* nope, float* scale, uint16_t* rope, uint8_t* idx_codes,
                   uint8_t* idx_scales) {
  double* g = (double*)malloc(sizeof(double) * (size_t)m * HEAD_DIM);
  double* v = (double*)malloc(sizeof(double) * (size_t)m * HEAD_DIM);
  double* bb = (double*)malloc(sizeof(double) * (size_t)m * HEAD_DIM);
  double* ig_d = (double*)malloc(sizeof(double) * (size_t)m * IDX_DIM);
  double* ik_d = (double*)malloc(sizeof(double) * (size_t)m * IDX_DIM);
  double* ib = (double*)malloc(sizeof(double) * (size_t)m * IDX_DIM);
  double y[HEAD_DIM], yi[IDX_DIM], row[HEAD_DIM];
  for (int i = 0; i < m * HEAD_DIM; ++i) bb[i] = (double)bias[i];
  if (idx_bias)
    for (int i = 0; i < m * IDX_DIM; ++i) ib[i] = (double)idx_bias[i];
  for (int64_t j = j_begin; j < j_end; ++j) {
    for (int i = 0; i < m; ++i) {
      int64_t p = j * m + i;
      int64_t t = p - tok0;
      if (t < 0 || t >= n_tok) abort();
      for (int c = 0; c < HEAD_DIM; ++c) {
        row[c] = (double)lcao_bf16_decode(kv[(size_t)t * HEAD_DIM + c]);
        g[(size_t)i * HEAD_DIM + c] = (double)lcao_bf16_decode(gate[(size_t)t * HEAD_DIM + c]);
      }
      lcao_rope_rotate(row, p);
      for (int c = 0; c < HEAD_DIM; ++c) v[(size_t)i * HEAD_DIM + c] = row[c];
      if (ik) {
        for (int c = 0; c < IDX_DIM; ++c) {
          ik_d[(size_t)i * IDX_DIM + c] = (double)lcao_bf16_decode(ik[(size_t)t * IDX_DIM + c]);
          ig_d[(size_t)i * IDX_DIM + c] = (double)lcao_bf16_decode(ig[(size_t)t * IDX_DIM + c]);
        }
      }
    }
    int64_t o = j - j_begin;
    lcao_pool(m, HEAD_DIM, g, bb, v, y, NULL);
    lcao_entry_encode(y, nope + o * NOPE_DIM, scale + o, rope + o * ROPE_DIM);
    if (ik) {
      lcao_pool(m, IDX_DIM, ig_d, ib, ik_d, yi, NULL);
      lcao_mxfp4_quant(yi, IDX_DIM, idx_codes + o * IDX_DIM, idx_scales + o * 2);
    }
  }
  free(g); free(v); free(bb); free(ig_d); free(ik_d); free(ib);
}

/* Sliding-window state: one entry per token, the token's own key RoPE'd at
 * its position and encoded like a compressed entry (reading: one entry
 * format, per-token scale). Tokens tok0 .. tok0+n-1. */
void lcao_window_entries(const uint16_t* kv, int64_t tok0, int64_t n, uint8_t* nope, float* scale, uint16_t* rope) {
  double row[HEAD_DIM];
  for (int64_t t = 0; t < n; ++t) {
    for (int c = 0; c < HEAD_DIM; ++c) row[c] = (double)lcao_bf16_decode(kv[(size_t)t * HEAD_DIM + c]);
    lcao_rope_rotate(row, tok0 + t);
    lcao_entry_encode(row, nope + t * NOPE_DIM, scale + t, rope + t * ROPE_DIM);
  }
}

/* ------------------------------------------------------------------ */
/* Lightning indexer score (CSA paragraph: FP4, ReLU-scored multi-head */
/* dot product).  Reading (parity unpinned): the query per indexer head */
/* is MX-FP4-quantised from BF16; per head the exact dot product of the */
/* dequantised vectors is rounded once to fp32 (s_h); then               */
/*   acc = +0; for h: acc = fmaf(w_h, ReLU(s_h), acc);                   */
/* and a zero result is returned as +0.  No 1/sqrt(d) factor.            */
/* Keys: idx_codes[j][64] one code per byte, idx_scales[j][2].           */
/* ------------------------------------------------------------------ */
void lcao_index_scores(int n_heads, const uint16_t* qI /* [H_I][64] */, const float* w /* [H_I] */,
                       const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t n_blocks, float* scores) {
  uint8_t* qc = (uint8_t*)malloc((size_t)n_heads * IDX_DIM);
  uint8_t* qs = (uint8_t*)malloc((size_t)n_heads * 2);
  double x[IDX_DIM];
  for (int h = 0; h < n_heads; ++h) {
    for (int c = 0; c < IDX_DIM; ++c) x[c] = (double)lcao_bf16_decode(qI[(size_t)h * IDX_DIM + c]);
    lcao_mxfp4_quant(x, IDX_DIM, qc + (size_t)h * IDX_DIM, qs + (size_t)h * 2);
  }
  for (int64_t j = 0; j < n_blocks; ++j) {
    const uint8_t* kc = idx_codes + j * IDX_DIM;
    const uint8_t* ks = idx_scales + j * 2;
    float acc = 0.0f;
    for (int h = 0; h < n_heads; ++h) {
      double D = 0.0;
      for (int b = 0; b < 2; ++b) {
        double part = 0.0; /* sum of products of E2M1 values: exact (multiples of 1/4, |.| <= 1152) */
        for (int c = 32 * b; c < 32 * b + 32; ++c)
          part = part + lcao_fp4_decode(qc[(size_t)h * IDX_DIM + c]) * lcao_fp4_decode(kc[c]);
        int e = ((int)qs[h * 2 + b] - 127) + ((int)ks[b] - 127);
        D = D + ldexp(part, e);
      }
      float s = (float)D;
      float r = s > 0.0f ? s : 0.0f;
      acc = fmaf(w[h], r, acc);
    }
    scores[j] = (acc == 0.0f) ? 0.0f : acc;
  }
  free(qc); free(qs);
}

/* Top-k (CSA paragraph: top-k compressed blocks per query). The min(k, n)
 * largest under (score descending, index ascending), returned in ascending
 * index order, padded with -1. Insertion into a sorted list: O(n k). */
void lcao_topk(const float* scores, int64_t n, int k, int32_t* out) {
  int64_t kk = n < k ? n : k;
  int64_t* best = (int64_t*)malloc(sizeof(int64_t) * (size_t)(kk + 1));
  int64_t cnt = 0;
  for (int64_t j = 0; j < n; ++j) {
    if (!isfinite(scores[j])) abort();
    /* position where j goes: after every element that ranks above it */
    int64_t pos = cnt;
    while (pos > 0) {
      int64_t o = best[pos - 1];
      int above = (scores[o] > scores[j]) || (scores[o] == scores[j] && o < j);
      if (above) break;
      --pos;
    }
    if (pos >= kk) continue;
    int64_t last = cnt < kk ? cnt : kk - 1;
    for (int64_t i = last; i > pos; --i) best[i] = best[i - 1];
    best[pos] = j;
    if (cnt < kk) ++cnt;
  }
  /* ascending index order */
  for (int64_t i = 1; i < cnt; ++i) {
    int64_t v = best[i], p = i;
    while (p > 0 && best[p - 1] > v) { best[p] = best[p - 1]; --p; }
    best[p] = v;
  }
  for (int i = 0; i < k; ++i) out[i] = (i < cnt) ? (int32_t)best[i] : -1;
  free(best);
}

/* ------------------------------------------------------------------ */
/* Attention for one query position t over a multiset of dequantised     */
/* entries (CSA: selected blocks; HCA: every visible block) plus the      */
/* window entries, with one joint softmax over all of them (reading of   */
/* the "sliding-window branch"; compressed and window keys share one     */
/* normalisation). K = V = the whole 128-dim entry (one shared KV head). */
/* q: [H][128] BF16 bits, RoPE'd at t in fp64. keys: n_keys x 128 fp64.  */
/* logits = q~ . x / sqrt(128). out_bf16 [H][128]; out_f64 [H][128] (may */
/* be NULL); lse [H] = max + log(sum) in fp64 (may be NULL).             */
/* ------------------------------------------------------------------ */
void lcao_attend(int n_heads, const uint16_t* q, int64_t t, const double* keys, int64_t n_keys, uint16_t* out_bf16,
                 double* out_f64, double* lse) {
  double qr[HEAD_DIM];
  double* l = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
  double inv = 1.0 / sqrt((double)HEAD_DIM);
  for (int h = 0; h < n_heads; ++h) {
    for (int c = 0; c < HEAD_DIM; ++c) qr[c] = (double)lcao_bf16_decode(q[(size_t)h * HEAD_DIM + c]);
    lcao_rope_rotate(qr, t);
    double mx = -INFINITY;
    for (int64_t i = 0; i < n_keys; ++i) {
      double d = 0.0;
      for (int c = 0; c < HEAD_DIM; ++c) d = d + qr[c] * keys[(size_t)i * HEAD_DIM + c];
      l[i] = d * inv;
      if (l[i] > mx) mx = l[i];
    }
    double S = 0.0;
    for (int64_t i = 0; i < n_keys; ++i) {
      l[i] = exp(l[i] - mx);
      S = S + l[i];
    }
    for (int c = 0; c < HEAD_DIM; ++c) {
      double o = 0.0;
      for (int64_t i = 0; i < n_keys; ++i) o = o + l[i] * keys[(size_t)i * HEAD_DIM + c];
      o = o / S;
      if (out_f64) out_f64[(size_t)h * HEAD_DIM + c] = o;
      out_bf16[(size_t)h * HEAD_DIM + c] = lcao_bf16_encode(o);
    }
    if (lse) lse[h] = mx + log(S);
  }
  free(l);
}
