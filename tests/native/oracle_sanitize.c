/*
 * Runs every function of the oracle and of the seeded input generators on
 * small, exactly sized heap buffers, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_native_sanitizers.py).  An access
 * past a buffer or undefined arithmetic stops the run; the few checks of
 * results below only guard that each call did its work.  Built without
 * OpenMP, so every loop runs on the calling thread.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle/oracle.c */
double oracle_bf16(uint16_t b);
double oracle_e4m3(uint8_t c);
double oracle_e8m0(uint8_t e);
void oracle_index_scores(int q_fmt, const void* q, const uint8_t* q_scales, const float* w, int k_fmt,
                         const void* k, const void* k_scales, int64_t vis, float* out);
int64_t oracle_topk(const float* scores, int64_t vis, int64_t top_k, int32_t* idx_out);
void oracle_sparse_attn(const uint16_t* q, int64_t H, int c_fmt, const void* c, const float* c_scales, int G,
                        const int32_t* idx, int64_t K, double sm_scale, double* out, double* lse, double* p_out);
uint8_t oracle_encode_e4m3(double v);
void oracle_quant_mxfp8(const uint16_t* x, int64_t n_rows, int64_t row_len, uint8_t* codes, uint8_t* scales);
void oracle_quant_fp8_rows(const uint16_t* x, int64_t n_rows, int64_t row_len, int64_t block, uint8_t* codes,
                           float* scales);

/* synth/synth.c */
void synth_idxq_int(uint64_t seed, int64_t t0, int64_t nt, int8_t* out);
void synth_w(uint64_t seed, int64_t t0, int64_t nt, float* out);
void synth_w_signed(uint64_t seed, int64_t t0, int64_t nt, float* out);
void synth_int_to_bf16(const int8_t* in, int64_t n, uint16_t* out);
void synth_mx_encode_int(const int8_t* in, int64_t ngroups, uint8_t* codes, uint8_t* scales);
void synth_idxk_int(uint64_t seed, int64_t b, int64_t s0, int64_t ns, int8_t* out);
void synth_kscale(uint64_t seed, int64_t b, int64_t s0, int64_t ns, float* out);
void synth_idxk_rows(uint64_t seed, int fmt, int64_t b, int64_t s0, int64_t ns, void* data, float* scales);
void synth_mlaq_bf16(uint64_t seed, int64_t H, int64_t t0, int64_t nt, uint16_t* out);
void synth_latent_rows(uint64_t seed, int fmt, int G, int64_t b, int64_t s0, int64_t ns, void* data,
                       float* scales);
void synth_fill_idxk_pool(uint64_t seed, int fmt, int64_t B, const int32_t* seq_lens, int64_t max_pages,
                          const int32_t* block_table, void* pool, float* pool_scales);
void synth_fill_latent_pool(uint64_t seed, int fmt, int G, int64_t B, const int32_t* seq_lens,
                            int64_t max_pages, const int32_t* block_table, void* pool, float* pool_scales);

static int failures = 0;
#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                   \
    }                                                               \
  } while (0)

/* exactly n bytes (at least one, so a zero-size buffer still has an address) */
static void* take(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  memset(p, 0xA5, n ? n : 1);
  return p;
}

static uint16_t bf16_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

static void codecs(void) {
  for (int c = 0; c < 256; ++c) {
    if ((c & 0x7f) == 0x7f) continue; /* the NaN codes */
    const double v = oracle_e4m3((uint8_t)c);
    CHECK(oracle_encode_e4m3(v) == (uint8_t)c);
  }
  CHECK(oracle_encode_e4m3(1e30) == 0x7e && oracle_encode_e4m3(-1e30) == 0xfe);
  CHECK(oracle_encode_e4m3(1e-30) == 0x00);
  CHECK(oracle_e8m0(127) == 1.0 && isnan(oracle_e8m0(255)) && oracle_e8m0(0) == ldexp(1.0, -127));
  CHECK(oracle_bf16(0x3f80) == 1.0);
}

/* scores of every query/key format pair, including no visible position */
static void scores(void) {
  const int64_t vis_cases[] = {0, 1, 3, 70};
  for (int vi = 0; vi < 4; ++vi) {
    const int64_t vis = vis_cases[vi];
    int8_t* qi = take(64 * 128);
    synth_idxq_int(11, 0, 1, qi);
    uint16_t* qb = take(64 * 128 * 2);
    synth_int_to_bf16(qi, 64 * 128, qb);
    uint8_t* qc = take(64 * 128);
    uint8_t* qs = take(64 * 4);
    synth_mx_encode_int(qi, 64 * 4, qc, qs);
    float* w = take(64 * 4);
    synth_w(11, 0, 1, w);
    float* ws = take(64 * 4);
    synth_w_signed(11, 0, 1, ws);
    int8_t* ki = take((size_t)vis * 128);
    synth_idxk_int(11, 0, 0, vis, ki);
    float* ksc = take((size_t)vis * 4);
    synth_kscale(11, 0, 0, vis, ksc);
    for (int fmt = 0; fmt < 3; ++fmt) {
      void* k = take((size_t)vis * 128 * (fmt == 0 ? 2 : 1));
      float* kscales = fmt == 0 ? NULL : take((size_t)vis * 4);
      synth_idxk_rows(11, fmt, 0, 0, vis, k, kscales);
      float* out = take((size_t)vis * 4);
      oracle_index_scores(fmt == 0 ? 0 : 1, fmt == 0 ? (const void*)qb : (const void*)qc, fmt == 0 ? NULL : qs,
                          fmt == 2 ? ws : w, fmt, k, kscales, vis, out);
      for (int64_t s = 0; s < vis; ++s) CHECK(isfinite(out[s]));
      free(out);
      free(kscales);
      free(k);
    }
    free(ki);
    free(ksc);
    free(ws);
    free(w);
    free(qs);
    free(qc);
    free(qb);
    free(qi);
  }
}

static void topk(void) {
  const int64_t vis_cases[] = {0, 1, 5, 64};
  const int64_t k_cases[] = {1, 4, 64, 100};
  for (int vi = 0; vi < 4; ++vi)
    for (int ki = 0; ki < 4; ++ki) {
      const int64_t vis = vis_cases[vi], K = k_cases[ki];
      float* s = take((size_t)vis * 4);
      for (int64_t i = 0; i < vis; ++i) s[i] = (float)((i * 7) % 5); /* many ties */
      int32_t* idx = take((size_t)K * 4);
      const int64_t n = oracle_topk(s, vis, K, idx);
      CHECK(n == (K < vis ? K : vis));
      for (int64_t i = 0; i < K; ++i) CHECK(i < n ? (idx[i] >= 0 && idx[i] < vis) : idx[i] == -1);
      for (int64_t i = 1; i < n; ++i)
        CHECK(s[idx[i - 1]] > s[idx[i]] || (s[idx[i - 1]] == s[idx[i]] && idx[i - 1] < idx[i]));
      free(idx);
      free(s);
    }
}

/* attention over every latent format, with skipped (-1) entries, an empty
 * selection, and K = 0 */
static void attention(void) {
  const int64_t L = 40, H = 3;
  uint16_t* q = take((size_t)H * 576 * 2);
  synth_mlaq_bf16(5, H, 0, 1, q);
  const int fmts[][2] = {{0, 1}, {1, 1}, {1, 5}, {2, 1}, {2, 4}};
  for (int f = 0; f < 5; ++f) {
    const int fmt = fmts[f][0], G = fmts[f][1];
    const int64_t row = fmt == 0 ? 1152 : fmt == 1 ? 576 : 640;
    void* c = take((size_t)L * row);
    float* sc = fmt == 0 ? NULL : take((size_t)L * G * 4);
    synth_latent_rows(5, fmt, G, 0, 0, L, c, sc);
    const int c_fmt = fmt == 2 ? 3 : fmt;
    const int64_t k_cases[] = {0, 1, 7, 12};
    for (int kc = 0; kc < 4; ++kc) {
      const int64_t K = k_cases[kc];
      int32_t* idx = take((size_t)K * 4);
      for (int64_t j = 0; j < K; ++j) idx[j] = kc == 1 ? -1 : (j % 3 == 2 ? -1 : (int32_t)((j * 13) % L));
      double* out = take((size_t)H * 512 * 8);
      double* lse = take((size_t)H * 8);
      double* p = take((size_t)H * K * 8);
      oracle_sparse_attn(q, H, c_fmt, c, sc, G, idx, K, 0.04, out, lse, p);
      const int any = K > 0 && kc != 1;
      for (int64_t h = 0; h < H; ++h) {
        CHECK(any ? isfinite(lse[h]) : (isinf(lse[h]) && lse[h] < 0));
        double z = 0;
        for (int64_t j = 0; j < K; ++j) z += p[h * K + j];
        CHECK(any ? fabs(z - 1.0) < 1e-12 : z == 0.0);
      }
      free(p);
      free(lse);
      free(out);
      free(idx);
    }
    free(sc);
    free(c);
  }
  free(q);
}

/* quantisers: an all-zero group, tiny and huge magnitudes, a short last tile */
static void quantisers(void) {
  const int64_t rows = 3, len = 576;
  uint16_t* x = take((size_t)rows * len * 2);
  for (int64_t i = 0; i < rows * len; ++i) {
    const int64_t r = i / len, d = i % len;
    float v = (float)sin((double)i * 0.37) * (r == 0 ? 1.0f : r == 1 ? 1e-38f : 3e38f);
    if (r == 0 && d < 32) v = 0.0f;
    x[i] = bf16_of(v);
  }
  uint8_t* codes = take((size_t)rows * len);
  uint8_t* scales = take((size_t)rows * (len / 32));
  oracle_quant_mxfp8(x, rows, len, codes, scales);
  CHECK(scales[0] == 127);
  for (int64_t i = 0; i < rows * (len / 32); ++i) CHECK(scales[i] != 255);
  const int64_t blocks[] = {128, 576, 100};
  for (int bi = 0; bi < 3; ++bi) {
    const int64_t nb = (len + blocks[bi] - 1) / blocks[bi];
    float* fs = take((size_t)rows * nb * 4);
    oracle_quant_fp8_rows(x, rows, len, blocks[bi], codes, fs);
    for (int64_t i = 0; i < rows * nb; ++i) CHECK(fs[i] > 0.0f && isfinite(fs[i]));
    free(fs);
  }
  free(scales);
  free(codes);
  free(x);
}

/* paged pools of every format: requests of 0, 1, 65 and 130 positions */
static void pools(void) {
  const int64_t B = 4, max_pages = 3, num_pages = 7;
  int32_t* lens = take(B * 4);
  lens[0] = 0;
  lens[1] = 1;
  lens[2] = 65;
  lens[3] = 130;
  int32_t* bt = take(B * max_pages * 4);
  for (int64_t i = 0; i < B * max_pages; ++i) bt[i] = (int32_t)((i * 5) % num_pages);
  bt[1 * max_pages + 0] = 0;
  bt[2 * max_pages + 0] = 1;
  bt[2 * max_pages + 1] = 2;
  bt[3 * max_pages + 0] = 3;
  bt[3 * max_pages + 1] = 4;
  bt[3 * max_pages + 2] = 5;
  for (int fmt = 0; fmt < 3; ++fmt) {
    void* pool = take((size_t)num_pages * 64 * (fmt == 0 ? 256 : 128));
    float* ps = fmt == 0 ? NULL : take((size_t)num_pages * 64 * 4);
    synth_fill_idxk_pool(9, fmt, B, lens, max_pages, bt, pool, ps);
    free(ps);
    free(pool);
  }
  const int fmts[][2] = {{0, 1}, {1, 1}, {1, 5}, {2, 1}, {2, 4}};
  for (int f = 0; f < 5; ++f) {
    const int fmt = fmts[f][0], G = fmts[f][1];
    void* pool = take((size_t)num_pages * 64 * (fmt == 0 ? 1152 : fmt == 1 ? 576 : 640));
    float* ps = fmt == 0 ? NULL : take((size_t)num_pages * 64 * G * 4);
    synth_fill_latent_pool(9, fmt, G, B, lens, max_pages, bt, pool, ps);
    free(ps);
    free(pool);
  }
  free(bt);
  free(lens);
}

int main(void) {
  codecs();
  scores();
  topk();
  attention();
  quantisers();
  pools();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle_sanitize: ok\n");
  return 0;
}
