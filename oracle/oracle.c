/*
 * CPU oracle for the sparse-attention hot path.  TEST INFRASTRUCTURE ONLY:
 * it is linked or called by the test-suite, by the smoke check and by the
 * benchmark's CPU-baseline leg, never by the product library.  It shares no
 * code, header or table with the HIP path.
 *
 * It is the plain definition of what the path computes, in double precision,
 * on logical (unpaged) per-request arrays:
 *
 *  1. Lightning-indexer relevance score.  The pages ("Day-0 Inference
 *     Adaptation and Optimization for Hybrid Attention Architectures", sec. 1;
 *     "Optimizing Inference for Hybrid Attention LLMs", sec. 3.1 pseudocode;
 *     "Day0 Inference Support and Performance Optimization for New-Architecture
 *     LLMs", sec. 4) describe a per-head q.k score against every historical
 *     position followed by a cross-head weighted aggregation.  The pages do not
 *     name the per-head nonlinearity; we read it as ReLU, so
 *         I[t,s] = sum_h w[t,h] * max(0, sum_d q[t,h,d] * k[s,d]),
 *     computed in double and rounded once to fp32 (then +0.0f, so -0 is +0).
 *  2. Top-K selection (same sections): the min(K, visible) positions with the
 *     largest score; among equal scores the lower position ranks first (the
 *     pages are silent on ties).  Output in rank order, padded with -1.
 *  3. Sparse attention over the MLA latent cache ("Day0 Inference Adaptation
 *     and Performance Optimization for a Sparse Hybrid Architecture LLM",
 *     sec. 1 and 2.1): softmax attention that reads only the selected rows.
 *     Keys are the whole 576-wide row (512 latent + 64 rope), values its first
 *     512 entries:  l_j = scale * q.c_j,  p = softmax(l),  o = sum_j p_j c_j[:512],
 *     lse = log sum_j exp(l_j).
 *
 * Storage formats are decoded from their published definitions:
 *  - bf16: the upper 16 bits of an IEEE binary32;
 *  - OCP FP8 E4M3FN ("OCP 8-bit Floating Point Specification"): bias 7, no
 *    infinities, S.1111.111 is NaN, subnormals m * 2^-9, max 448;
 *  - E8M0 (OCP Microscaling Formats v1.0): 2^(e-127), e = 255 is NaN.
 * The pages' quantised layouts ("Optimizing Inference ...", sec. 4 table):
 * indexer q in MXFP8 with one E8M0 scale per 32 elements; FP8 caches carry f32
 * scales per 128-element block (indexer key: one per row; latent: one per row,
 * or one per 128-wide tile of the row, the fifth tile being 64 wide).  The
 * indexer key may also be MXFP8 like the query (E4M3 codes, one E8M0 scale
 * per 32 elements), the group-32 form that table gives for it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

double oracle_e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

double oracle_e8m0(uint8_t e) {
  if (e == 255) return NAN;
  return ldexp(1.0, (int)e - 127);
}

/* fmt 0 = bf16 bits, fmt 1 and 2 = E4M3 codes */
static double elem(int fmt, const void* p, int64_t i) {
  return fmt == 0 ? oracle_bf16(((const uint16_t*)p)[i]) : oracle_e4m3(((const uint8_t*)p)[i]);
}

/*
 * Indexer scores of one query token against positions 0..vis-1.
 *   q        [64][128] bf16 bits (q_fmt 0) or E4M3 codes (q_fmt 1)
 *   q_scales [64][4] E8M0, one per 32 consecutive d (q_fmt 1 only)
 *   w        [64] f32 head weights
 *   k        [vis][128] logical key rows, bf16 (k_fmt 0) or E4M3 (k_fmt 1, 2)
 *   k_scales k_fmt 1: [vis] f32, one per 128-element block = one per row;
 *            k_fmt 2: [vis][4] E8M0, one per 32 consecutive d (MXFP8, the
 *            indexer-key layout of the "Optimizing Inference ..." sec. 4
 *            table: the same group-32 power-of-two scaling as the query)
 *   out      [vis] f32
 */
void oracle_index_scores(int q_fmt, const void* q, const uint8_t* q_scales, const float* w, int k_fmt,
                         const void* k, const void* k_scales, int64_t vis, float* out) {
  double qd[64][128];
  for (int h = 0; h < 64; ++h)
    for (int d = 0; d < 128; ++d) {
      double v = elem(q_fmt, q, h * 128 + d);
      if (q_fmt == 1) v *= oracle_e8m0(q_scales[h * 4 + d / 32]);
      qd[h][d] = v;
    }
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < vis; ++s) {
    double kd[128];
    for (int d = 0; d < 128; ++d) {
      double v = elem(k_fmt, k, s * 128 + d);
      if (k_fmt == 1) v *= (double)((const float*)k_scales)[s];
      if (k_fmt == 2) v *= oracle_e8m0(((const uint8_t*)k_scales)[s * 4 + d / 32]);
      kd[d] = v;
    }
    double acc = 0.0;
    for (int h = 0; h < 64; ++h) {
      double dot = 0.0;
      for (int d = 0; d < 128; ++d) dot += qd[h][d] * kd[d];
      acc += (double)w[h] * (dot > 0.0 ? dot : 0.0);
    }
    out[s] = (float)acc + 0.0f;
  }
}

typedef struct {
  float score;
  int32_t pos;
} scored_pos;

static int by_score_desc_pos_asc(const void* a, const void* b) {
  const scored_pos* x = (const scored_pos*)a;
  const scored_pos* y = (const scored_pos*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

/* Top-K by a full sort of the visible positions.  Returns min(K, vis); the
 * rest of idx_out[0..K) is -1. */
int64_t oracle_topk(const float* scores, int64_t vis, int64_t top_k, int32_t* idx_out) {
  scored_pos* v = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(vis > 0 ? vis : 1));
  for (int64_t s = 0; s < vis; ++s) {
    v[s].score = scores[s];
    v[s].pos = (int32_t)s;
  }
  qsort(v, (size_t)vis, sizeof(scored_pos), by_score_desc_pos_asc);
  int64_t n = top_k < vis ? top_k : vis;
  for (int64_t i = 0; i < top_k; ++i) idx_out[i] = i < n ? v[i].pos : -1;
  free(v);
  return n;
}

/* Dequantised latent element d of row r. */
static double latent(int c_fmt, const void* c, const float* c_scales, int G, int64_t r, int d) {
  if (c_fmt == 0) return oracle_bf16(((const uint16_t*)c)[r * 576 + d]);
  int g = G == 1 ? 0 : d / 128;
  if (c_fmt == 3) {
    /* 640-byte rows: 512 E4M3 latent codes, then the 64 rope elements as bf16 */
    const uint8_t* row = (const uint8_t*)c + r * 640;
    if (d >= 512) return oracle_bf16((uint16_t)(row[512 + 2 * (d - 512)] | (row[513 + 2 * (d - 512)] << 8)));
    return oracle_e4m3(row[d]) * (double)c_scales[r * G + g];
  }
  return oracle_e4m3(((const uint8_t*)c)[r * 576 + d]) * (double)c_scales[r * G + g];
}

/*
 * Sparse attention of one query token.
 *   q        [H][576] bf16 bits
 *   c        [L][576] logical latent rows of the token's request, bf16 (c_fmt 0)
 *            or E4M3 codes (c_fmt 1) with f32 c_scales [L][G], G in {1, 5};
 *            or (c_fmt 3) [L][640] bytes: E4M3 codes of the 512 latent
 *            elements with f32 c_scales [L][G], G in {1, 4} (tiles of 128),
 *            then the 64 rope elements as bf16
 *   idx      [K] selected positions; entries < 0 are skipped
 *   out      [H][512] double,  lse [H] double (-inf when nothing is selected)
 *   p_out    optional [H][K] softmax weights (0 for skipped entries)
 */
void oracle_sparse_attn(const uint16_t* q, int64_t H, int c_fmt, const void* c, const float* c_scales, int G,
                        const int32_t* idx, int64_t K, double sm_scale, double* out, double* lse,
                        double* p_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t h = 0; h < H; ++h) {
    double* l = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double m = -INFINITY;
    for (int64_t j = 0; j < K; ++j) {
      if (idx[j] < 0) continue;
      double dot = 0.0;
      for (int d = 0; d < 576; ++d) dot += oracle_bf16(q[h * 576 + d]) * latent(c_fmt, c, c_scales, G, idx[j], d);
      l[j] = sm_scale * dot;
      if (l[j] > m) m = l[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < K; ++j)
      if (idx[j] >= 0) z += exp(l[j] - m);
    for (int d = 0; d < 512; ++d) out[h * 512 + d] = 0.0;
    for (int64_t j = 0; j < K; ++j) {
      double p = idx[j] >= 0 ? exp(l[j] - m) / z : 0.0;
      if (p_out) p_out[h * K + j] = p;
      if (idx[j] < 0) continue;
      for (int d = 0; d < 512; ++d) out[h * 512 + d] += p * latent(c_fmt, c, c_scales, G, idx[j], d);
    }
    lse[h] = z > 0.0 ? m + log(z) : -INFINITY;
    free(l);
  }
}

/*
 * Quantisers and the cache append (the step before the path in every decode
 * step: "Day-0 Inference Adaptation and Optimization for Hybrid Attention
 * Architectures", sec. 4 -- MXFP8 indexer query with group 32, FP8 KV cache
 * with per-token-head-tile scales of tile 128; "Optimizing Inference for
 * Hybrid Attention LLMs", sec. 4 table; "Day0 Inference Adaptation and
 * Performance Optimization for a Sparse Hybrid Architecture LLM", sec. 3.1 --
 * quantised indexer q and K; the new token's cache rows are written into the
 * paged cache).  Readings where the pages are silent:
 *  - E4M3 encoding is round-to-nearest, ties to the even code, saturating
 *    at +-448 (OCP E4M3FN has no infinity; "satfinite");
 *  - MXFP8 (OCP Microscaling v1.0): per group of 32, shared exponent
 *    X = 2^(floor(log2 amax) - 8) (8 = the largest E4M3 exponent), stored as
 *    E8M0 code floor(log2 amax) - 8 + 127, held to the codes 0..254 (2^-127
 *    .. 2^127); an all-zero group takes X = 1;
 *    elements are x / X encoded as E4M3;
 *  - FP8 cache rows: f32 scale = amax / 448 of the row (or of each 128-wide
 *    tile, the fifth tile of a 576-wide latent row being 64 wide), 1 for an
 *    all-zero block; elements are fl32(x / scale) encoded as E4M3.  The
 *    quotient is taken in fp32 (the kernel's precision decides the code).
 */

/* Nearest E4M3FN code of v (ties to the even code), saturating at 448. */
uint8_t oracle_encode_e4m3(double v) {
  const uint8_t sign = (v < 0 || (v == 0 && signbit(v))) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7e;
  /* magnitude in units of the code grid: below 2^-6 the grid step is 2^-9
   * (subnormals and the smallest binade), above it 2^(e-3) for a in [2^e, 2^(e+1)) */
  int e;
  (void)frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  int ee = e - 1;      /* a in [2^ee, 2^(ee+1)) */
  if (a == 0.0 || ee < -6) ee = -6;
  const double step = ldexp(1.0, ee - 3);
  double units = a / step;           /* exact: a power-of-two division */
  double fl = floor(units);
  double frac = units - fl;
  double r = fl;
  if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
  /* r * step is the rounded magnitude; re-derive the code from it */
  double m = r * step;
  if (m >= 448.0) return sign | 0x7e;
  if (m == 0.0) return sign;
  int e2;
  (void)frexp(m, &e2);
  int ex = e2 - 1; /* m in [2^ex, 2^(ex+1)) */
  if (ex < -6) {   /* subnormal: m = k * 2^-9, k in 1..7 */
    return sign | (uint8_t)(int)ldexp(m, 9);
  }
  int mant = (int)(ldexp(m, -ex) * 8.0) - 8; /* 0..7 */
  return sign | (uint8_t)(((ex + 7) << 3) | mant);
}

static float f32_of_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* MXFP8 quantisation of n_rows rows of row_len bf16 values (row_len % 32 == 0). */
void oracle_quant_mxfp8(const uint16_t* x, int64_t n_rows, int64_t row_len, uint8_t* codes, uint8_t* scales) {
  const int64_t groups = row_len / 32;
  for (int64_t r = 0; r < n_rows; ++r)
    for (int64_t g = 0; g < groups; ++g) {
      const uint16_t* xg = x + r * row_len + g * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)f32_of_bf16(xg[i])));
      int sh = 0; /* log2 X */
      if (amax > 0.0) {
        int e;
        (void)frexp(amax, &e);
        sh = (e - 1) - 8;
      }
      /* E8M0 holds 2^-127 .. 2^127 (code 255 is NaN) */
      if (sh < -127) sh = -127;
      if (sh > 127) sh = 127;
      scales[r * groups + g] = (uint8_t)(sh + 127);
      for (int i = 0; i < 32; ++i)
        codes[r * row_len + g * 32 + i] = oracle_encode_e4m3(ldexp((double)f32_of_bf16(xg[i]), -sh));
    }
}

/* FP8 rows with one f32 scale per block: blocks of `block` elements (the last
 * one may be shorter).  scales: [n_rows][ceil(row_len / block)]. */
void oracle_quant_fp8_rows(const uint16_t* x, int64_t n_rows, int64_t row_len, int64_t block, uint8_t* codes,
                           float* scales) {
  const int64_t nb = (row_len + block - 1) / block;
  for (int64_t r = 0; r < n_rows; ++r)
    for (int64_t bI = 0; bI < nb; ++bI) {
      const int64_t lo = bI * block, hi = lo + block < row_len ? lo + block : row_len;
      float amax = 0.0f;
      for (int64_t d = lo; d < hi; ++d) amax = fmaxf(amax, fabsf(f32_of_bf16(x[r * row_len + d])));
      const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      scales[r * nb + bI] = sc;
      for (int64_t d = lo; d < hi; ++d) {
        const float qv = f32_of_bf16(x[r * row_len + d]) / sc; /* fp32 quotient */
        codes[r * row_len + d] = oracle_encode_e4m3((double)qv);
      }
    }
}
