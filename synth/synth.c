/*
 * Seeded synthetic-input generator for the sparse-attention hot path.
 *
 * This file is test and benchmark infrastructure.  It produces the bytes that
 * both the CPU oracle and the HIP library consume, and it holds none of the
 * method's arithmetic (no scoring, no selection, no attention).  What it does
 * hold is value generation and the encodings of the storage formats used by
 * the caches: bf16 bit patterns, OCP FP8 E4M3FN codes and E8M0 exponents.
 *
 * Every value is a pure function of (seed, stream, counter), where counter is
 * the logical element index, so any slice of any tensor can be regenerated on
 * its own (for example one request of a 32K-token cache, or one page).
 *
 * Generator: splitmix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014; the finaliser constants are the published
 * ones).  Normal deviates use Box-Muller on the two 32-bit halves of one draw.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ST_IDXQ 1u    /* indexer query, integers in [-4,4]      per (t,h,d)  */
#define ST_W 2u       /* indexer head weights, (floor(32u)+1)/32 per (t,h)    */
#define ST_IDXK 3u    /* indexer key, integers in [-4,4]        per (b,s,d)  */
#define ST_KSCALE 4u  /* indexer key FP8 block scale in {1/2,1} per (b,s)    */
#define ST_MLAQ 5u    /* MLA query, N(0,1)                      per (t,h,d)  */
#define ST_LATENT 6u  /* MLA latent row, N(0,1)                 per (b,s,d)  */

static inline uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint32_t stream) {
  return splitmix64(splitmix64(seed) ^ ((uint64_t)stream << 56));
}

static inline uint64_t draw(uint64_t base, uint64_t counter) {
  return splitmix64(base + counter);
}

static inline int draw_int9(uint64_t u) { return (int)((u >> 32) % 9u) - 4; }

static inline double draw_normal(uint64_t u) {
  double u1 = ((double)(u >> 32) + 0.5) * (1.0 / 4294967296.0);
  double u2 = ((double)(u & 0xffffffffu) + 0.5) * (1.0 / 4294967296.0);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* Counter of element (b, s, d) of a per-request tensor with row width D. */
static inline uint64_t ctr_bsd(int64_t b, int64_t s, int64_t d, int64_t D) {
  return (((uint64_t)b << 26) + (uint64_t)s) * (uint64_t)D + (uint64_t)d;
}

/* ---- storage-format encoders (generation side only) ---- */

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* Magnitudes of the 127 non-negative finite E4M3FN codes 0x00..0x7e. */
static double g_e4m3_mag[127];
static int g_e4m3_ready = 0;
static void e4m3_table(void) {
  if (g_e4m3_ready) return;
  for (int c = 0; c < 127; ++c) {
    int e = (c >> 3) & 15, m = c & 7;
    g_e4m3_mag[c] = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  }
  g_e4m3_ready = 1;
}

/* Nearest E4M3FN code (ties to even code), saturating at 448. */
static uint8_t e4m3_encode(double v) {
  uint8_t sign = v < 0 ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7e;
  int lo = 0, hi = 126;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (g_e4m3_mag[mid] <= a) lo = mid; else hi = mid;
  }
  double dl = a - g_e4m3_mag[lo], dh = g_e4m3_mag[hi] - a;
  int c = (dl < dh) ? lo : (dh < dl) ? hi : ((lo & 1) ? hi : lo);
  return sign | (uint8_t)c;
}

/* ---- indexer query ---- */

/* Integer values of the indexer query for tokens [t0, t0+nt): out[nt][64][128]. */
void synth_idxq_int(uint64_t seed, int64_t t0, int64_t nt, int8_t* out) {
  uint64_t base = stream_base(seed, ST_IDXQ);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nt * 64 * 128; ++i)
    out[i] = (int8_t)draw_int9(draw(base, (uint64_t)(t0 * 64 * 128 + i)));
}

void synth_w(uint64_t seed, int64_t t0, int64_t nt, float* out) {
  uint64_t base = stream_base(seed, ST_W);
  for (int64_t i = 0; i < nt * 64; ++i) {
    uint64_t u = draw(base, (uint64_t)(t0 * 64 + i));
    out[i] = (float)((double)((u >> 32) % 32u + 1u) / 32.0);
  }
}

/* Head weights of either sign: +-(floor(32u)+1)/32, the sign from the low
 * bit of the same draw (the magnitude uses the high half).  The head weight is
 * a projection output, so scores may be negative; on the 1/32 grid they stay
 * exact in fp32. */
void synth_w_signed(uint64_t seed, int64_t t0, int64_t nt, float* out) {
  uint64_t base = stream_base(seed, ST_W);
  for (int64_t i = 0; i < nt * 64; ++i) {
    uint64_t u = draw(base, (uint64_t)(t0 * 64 + i));
    double m = (double)((u >> 32) % 32u + 1u) / 32.0;
    out[i] = (float)((u & 1u) ? -m : m);
  }
}

/* bf16 bits of small integers (exact). */
void synth_int_to_bf16(const int8_t* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)in[i]);
}

/*
 * MXFP8 encoding of integer-valued groups of 32 (OCP MX: one E8M0 scale per
 * 32 consecutive elements, elements E4M3FN).  The shared exponent is
 * floor(log2(amax)) - 8 (amax = 0 gives exponent 0); for integers in [-4,4]
 * every element code is exact.
 */
void synth_mx_encode_int(const int8_t* in, int64_t ngroups, uint8_t* codes, uint8_t* scales) {
  e4m3_table();
  for (int64_t g = 0; g < ngroups; ++g) {
    int amax = 0;
    for (int i = 0; i < 32; ++i) {
      int a = in[g * 32 + i] < 0 ? -in[g * 32 + i] : in[g * 32 + i];
      if (a > amax) amax = a;
    }
    int e = 0;
    if (amax > 0) {
      int fl = 0;
      while ((1 << (fl + 1)) <= amax) ++fl;
      e = fl - 8;
    }
    scales[g] = (uint8_t)(e + 127);
    for (int i = 0; i < 32; ++i) codes[g * 32 + i] = e4m3_encode(ldexp((double)in[g * 32 + i], -e));
  }
}

/* ---- indexer key rows of one request ---- */

void synth_idxk_int(uint64_t seed, int64_t b, int64_t s0, int64_t ns, int8_t* out) {
  uint64_t base = stream_base(seed, ST_IDXK);
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < ns; ++s)
    for (int d = 0; d < 128; ++d)
      out[s * 128 + d] = (int8_t)draw_int9(draw(base, ctr_bsd(b, s0 + s, d, 128)));
}

void synth_kscale(uint64_t seed, int64_t b, int64_t s0, int64_t ns, float* out) {
  uint64_t base = stream_base(seed, ST_KSCALE);
  for (int64_t s = 0; s < ns; ++s)
    out[s] = (draw(base, ctr_bsd(b, s0 + s, 0, 1)) >> 63) ? 1.0f : 0.5f;
}

/* fmt 0: bf16 rows [ns][128].  fmt 1: E4M3 codes [ns][128] of the integers and
 * a per-row (= per 128-element block) f32 scale in {1/2, 1}.  fmt 2: the same
 * codes with four E8M0 scale codes per row (one per 32 elements), each 126 or
 * 127 (1/2 or 1), stored as 4 bytes per row where fmt 1 stores the f32. */
void synth_idxk_rows(uint64_t seed, int fmt, int64_t b, int64_t s0, int64_t ns, void* data, float* scales) {
  e4m3_table();
  uint64_t base = stream_base(seed, ST_IDXK);
  uint64_t sbase = stream_base(seed, ST_KSCALE);
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < ns; ++s) {
    for (int d = 0; d < 128; ++d) {
      int v = draw_int9(draw(base, ctr_bsd(b, s0 + s, d, 128)));
      if (fmt == 0) ((uint16_t*)data)[s * 128 + d] = f32_to_bf16_rne((float)v);
      else ((uint8_t*)data)[s * 128 + d] = e4m3_encode((double)v);
    }
    if (fmt == 1) scales[s] = (draw(sbase, ctr_bsd(b, s0 + s, 0, 1)) >> 63) ? 1.0f : 0.5f;
    if (fmt == 2)
      for (int g = 0; g < 4; ++g)
        ((uint8_t*)scales)[s * 4 + g] = (draw(sbase, ctr_bsd(b, s0 + s, g, 4)) >> 63) ? 127 : 126;
  }
}

/* ---- MLA query ---- */

void synth_mlaq_bf16(uint64_t seed, int64_t H, int64_t t0, int64_t nt, uint16_t* out) {
  uint64_t base = stream_base(seed, ST_MLAQ);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nt * H * 576; ++i)
    out[i] = f32_to_bf16_rne((float)draw_normal(draw(base, (uint64_t)(t0 * H * 576 + i))));
}

/* ---- latent rows of one request ----
 * fmt 0: bf16 [ns][576] of N(0,1).
 * fmt 1: E4M3 codes [ns][576] with f32 scales [ns][G]; G = 1 (one scale per
 * row) or G = 5 (tiles of 128 along the row: 4 x 128 + 1 x 64).  Each scale is
 * amax/448 of its tile (1 for an all-zero tile), codes are nearest-even.
 * fmt 2: rows of 640 bytes, E4M3 codes of the 512 latent elements then the 64
 * rope elements as bf16; f32 scales [ns][G] over the latent only, G = 1 (one
 * per row) or G = 4 (tiles of 128). */
void synth_latent_rows(uint64_t seed, int fmt, int G, int64_t b, int64_t s0, int64_t ns, void* data,
                       float* scales) {
  e4m3_table();
  uint64_t base = stream_base(seed, ST_LATENT);
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < ns; ++s) {
    double x[576];
    for (int d = 0; d < 576; ++d) x[d] = draw_normal(draw(base, ctr_bsd(b, s0 + s, d, 576)));
    if (fmt == 0) {
      for (int d = 0; d < 576; ++d) ((uint16_t*)data)[s * 576 + d] = f32_to_bf16_rne((float)x[d]);
      continue;
    }
    if (fmt == 2) {
      uint8_t* row = (uint8_t*)data + s * 640;
      int tw = G == 1 ? 512 : 128;
      for (int g = 0; g < G; ++g) {
        double amax = 0;
        for (int d = g * tw; d < (g + 1) * tw; ++d) amax = fabs(x[d]) > amax ? fabs(x[d]) : amax;
        float sc = amax > 0 ? (float)(amax / 448.0) : 1.0f;
        scales[s * G + g] = sc;
        for (int d = g * tw; d < (g + 1) * tw; ++d) row[d] = e4m3_encode(x[d] / (double)sc);
      }
      for (int d = 512; d < 576; ++d) {
        uint16_t h = f32_to_bf16_rne((float)x[d]);
        memcpy(row + 512 + 2 * (d - 512), &h, 2);
      }
      continue;
    }
    int tw = G == 1 ? 576 : 128;
    for (int g = 0; g < G; ++g) {
      int lo = g * tw, hi = lo + tw > 576 ? 576 : lo + tw;
      double amax = 0;
      for (int d = lo; d < hi; ++d) amax = fabs(x[d]) > amax ? fabs(x[d]) : amax;
      float sc = amax > 0 ? (float)(amax / 448.0) : 1.0f;
      scales[s * G + g] = sc;
      for (int d = lo; d < hi; ++d) ((uint8_t*)data)[s * 576 + d] = e4m3_encode(x[d] / (double)sc);
    }
  }
}

/* ---- paged pools ----
 * Scatter logical rows of every request into a page pool: row s of request b
 * goes to page block_table[b*max_pages + s/64], slot s%64.  row_bytes is the
 * byte width of one row of `pool`, nsc the number of f32 scales per row. */
static void fill_pool(uint64_t seed, int fmt, int G, int which, int64_t B, const int32_t* seq_lens,
                      int64_t max_pages, const int32_t* block_table, void* pool, float* pool_scales,
                      int64_t row_bytes, int64_t nsc) {
  /* one work item per (request, logical page); inner row loops run serially
   * because OpenMP does not nest parallel regions by default */
  e4m3_table();
  int64_t total = 0;
  for (int64_t b = 0; b < B; ++b) total += (seq_lens[b] + 63) / 64;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t item = 0; item < total; ++item) {
    int64_t b = 0, p = item;
    while (p >= (seq_lens[b] + 63) / 64) { p -= (seq_lens[b] + 63) / 64; ++b; }
    int64_t L = seq_lens[b];
    int64_t s0 = p * 64, ns = L - s0 < 64 ? L - s0 : 64;
    int64_t page = block_table[b * max_pages + p];
    uint8_t* dst = (uint8_t*)pool + page * 64 * row_bytes;
    float* sdst = pool_scales ? pool_scales + page * 64 * nsc : 0;
    if (which == 0) synth_idxk_rows(seed, fmt, b, s0, ns, dst, sdst);
    else synth_latent_rows(seed, fmt, G, b, s0, ns, dst, sdst);
  }
}

void synth_fill_idxk_pool(uint64_t seed, int fmt, int64_t B, const int32_t* seq_lens, int64_t max_pages,
                          const int32_t* block_table, void* pool, float* pool_scales) {
  /* fmt 2 stores its four scale bytes per row where fmt 1 stores one f32 */
  fill_pool(seed, fmt, 1, 0, B, seq_lens, max_pages, block_table, pool, pool_scales, fmt == 0 ? 256 : 128, 1);
}

void synth_fill_latent_pool(uint64_t seed, int fmt, int G, int64_t B, const int32_t* seq_lens,
                            int64_t max_pages, const int32_t* block_table, void* pool, float* pool_scales) {
  fill_pool(seed, fmt, G, 1, B, seq_lens, max_pages, block_table, pool, pool_scales,
            fmt == 0 ? 1152 : fmt == 1 ? 576 : 640, G);
}
