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
 * or one per 128-wide tile of the row, the fifth tile being 64 wide).
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

/* fmt 0 = bf16 bits, fmt 1 = E4M3 codes */
static double elem(int fmt, const void* p, int64_t i) {
  return fmt == 0 ? oracle_bf16(((const uint16_t*)p)[i]) : oracle_e4m3(((const uint8_t*)p)[i]);
}

/*
 * Indexer scores of one query token against positions 0..vis-1.
 *   q        [64][128] bf16 bits (q_fmt 0) or E4M3 codes (q_fmt 1)
 *   q_scales [64][4] E8M0, one per 32 consecutive d (q_fmt 1 only)
 *   w        [64] f32 head weights
 *   k        [vis][128] logical key rows, bf16 (k_fmt 0) or E4M3 (k_fmt 1)
 *   k_scales [vis] f32, one per 128-element block = one per row (k_fmt 1)
 *   out      [vis] f32
 */
void oracle_index_scores(int q_fmt, const void* q, const uint8_t* q_scales, const float* w, int k_fmt,
                         const void* k, const float* k_scales, int64_t vis, float* out) {
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
      if (k_fmt == 1) v *= (double)k_scales[s];
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
  return oracle_e4m3(((const uint8_t*)c)[r * 576 + d]) * (double)c_scales[r * G + g];
}

/*
 * Sparse attention of one query token.
 *   q        [H][576] bf16 bits
 *   c        [L][576] logical latent rows of the token's request, bf16 (c_fmt 0)
 *            or E4M3 codes (c_fmt 1) with f32 c_scales [L][G], G in {1, 5}
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
