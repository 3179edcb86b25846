/*
 * synth_host.c - host side of the seeded synthetic-input generator.
 *
 * Holds no arithmetic of the MoE layer. It builds the value tables that the
 * counter-based draws of synth_core.h index, fills host buffers from them, and
 * draws the small host-only inputs (the log-Zipf router bias).
 *
 * Distributions (the workloads of the decode layer):
 *   "~N(0, sigma)"  one of 2^14 equiprobable normal quantiles
 *                   z_i = Phi^-1((i + 0.5) / 2^14) (a discretised normal whose
 *                   extreme value is about 3.99 sigma), times sigma, rounded
 *                   once to the storage type;
 *   fp8 e4m3 weights with a bf16 scale per 128 output rows: each row group g
 *                   draws a scale class c_g in {0,1,2,3}; its scale is
 *                   s_c = bf16(sigma * zmax / 448 * (1 + c/4)) and its codes are
 *                   the e4m3 round-to-nearest-even (saturating) of z * sigma / s_c,
 *                   so q * s stays a quantised N(0, sigma) while scales differ
 *                   between groups;
 *   router bias     b_e = ln(r_e^-s / H_{E,s}) with r a random permutation of
 *                   1..E (log of a Zipf(s) popularity).
 * Build: gcc -O2 -shared -fPIC synth_host.c -lm -lpthread
 */
#define SYNTH_FN static inline
#include "synth_core.h"

#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ---- the discretised normal ------------------------------------------- */

/* Standard normal CDF from the complementary error function. */
static double phi(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

/* z_i = Phi^-1((i + 0.5) / N), by bisection (Phi is increasing, so 200 halvings
 * of [-40, 40] reach the double nearest the root). The lower half is solved
 * (where erfc keeps full relative precision) and mirrored, z_{N-1-i} = -z_i. */
void synth_normal_table(double *z) {
  for (uint32_t i = 0; i < SYNTH_TABLE_SIZE / 2; ++i) {
    double p = ((double)i + 0.5) / (double)SYNTH_TABLE_SIZE;
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 200; ++it) {
      double mid = 0.5 * (lo + hi);
      if (mid == lo || mid == hi) break;
      if (phi(mid) < p) lo = mid; else hi = mid;
    }
    z[i] = 0.5 * (lo + hi);
    z[SYNTH_TABLE_SIZE - 1u - i] = -z[i];
  }
}

/* ---- storage-type encoders used to build the tables -------------------- */

/* float -> bf16 bits, round to nearest even (NaN stays a quiet NaN). */
static uint16_t gen_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static float gen_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* double -> OCP e4m3fn code, round to nearest even, saturating at +-448. */
static uint8_t gen_e4m3_code(double v) {
  uint8_t sign = (v < 0) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;  /* 1111.110 = 448 */
  if (a < ldexp(1.0, -6)) {            /* subnormal: m * 2^-9, m in 0..8 */
    double m = rint(a / ldexp(1.0, -9));
    return sign | (uint8_t)m;          /* m == 8 is the smallest normal, 0001.000 */
  }
  int e;
  double fr = frexp(a, &e);            /* a = fr * 2^e, fr in [0.5, 1) */
  int ex = e - 1;                      /* a = (2 fr) * 2^ex, 2 fr in [1, 2) */
  double m = rint((2.0 * fr - 1.0) * 8.0);
  if (m == 8.0) { m = 0.0; ex += 1; }
  int field = ex + 7;
  if (field > 15 || (field == 15 && m > 6.0)) return sign | 0x7E;
  return sign | (uint8_t)((field << 3) | (int)m);
}

/* ---- tables ------------------------------------------------------------ */

/* dtype: 0 = f32 (4-byte entries), 1 = bf16 (2-byte entries) */
void synth_value_table(const double *z, double sigma, int dtype, void *out) {
  for (uint32_t i = 0; i < SYNTH_TABLE_SIZE; ++i) {
    float f = (float)(z[i] * sigma);
    if (dtype == 0) ((float *)out)[i] = f;
    else ((uint16_t *)out)[i] = gen_bf16_bits(f);
  }
}

/* fp8 scale of class c (bf16 bits) and the code table of that class. */
uint16_t synth_fp8_scale_bits(const double *z, double sigma, int c) {
  double zmax = z[SYNTH_TABLE_SIZE - 1];
  return gen_bf16_bits((float)(sigma * zmax / 448.0 * (1.0 + 0.25 * c)));
}

void synth_fp8_code_table(const double *z, double sigma, int c, uint8_t *out) {
  double s = (double)gen_bf16_value(synth_fp8_scale_bits(z, sigma, c));
  for (uint32_t i = 0; i < SYNTH_TABLE_SIZE; ++i) out[i] = gen_e4m3_code(z[i] * sigma / s);
}

/* ---- fills ------------------------------------------------------------- */

typedef struct {
  void *dst;
  uint64_t begin, end;
  uint64_t key;
  const void *table;
  int elem_bytes;
} fill_job;

static void fill_range(void *dst, uint64_t begin, uint64_t end, uint64_t key,
                       const void *table, int elem_bytes) {
  if (elem_bytes == 4) {
    const uint32_t *t = (const uint32_t *)table;
    uint32_t *d = (uint32_t *)dst;
    for (uint64_t i = begin; i < end; ++i) d[i] = t[synth_index(key, i)];
  } else if (elem_bytes == 2) {
    const uint16_t *t = (const uint16_t *)table;
    uint16_t *d = (uint16_t *)dst;
    for (uint64_t i = begin; i < end; ++i) d[i] = t[synth_index(key, i)];
  } else {
    const uint8_t *t = (const uint8_t *)table;
    uint8_t *d = (uint8_t *)dst;
    for (uint64_t i = begin; i < end; ++i) d[i] = t[synth_index(key, i)];
  }
}

static void *fill_worker(void *arg) {
  fill_job *j = (fill_job *)arg;
  fill_range(j->dst, j->begin, j->end, j->key, j->table, j->elem_bytes);
  return NULL;
}

/* dst[i] = table[index(key, i)] for i in [0, n). elem_bytes in {1, 2, 4}. */
void synth_fill(void *dst, uint64_t n, uint64_t key, const void *table, int elem_bytes,
                int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (n < (1u << 20)) nthreads = 1;
  pthread_t th[64];
  fill_job jobs[64];
  uint64_t chunk = ((n + (uint64_t)nthreads - 1) / (uint64_t)nthreads + 3) & ~(uint64_t)3;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t b = (uint64_t)t * chunk, e = b + chunk;
    if (b >= n) break;
    if (e > n) e = n;
    jobs[t] = (fill_job){dst, b, e, key, table, elem_bytes};
    if (nthreads == 1 || pthread_create(&th[t], NULL, fill_worker, &jobs[t]) != 0) {
      fill_worker(&jobs[t]);
      th[t] = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (th[t]) pthread_join(th[t], NULL);
}

/* Scale class (0..3) of row group g of a weight whose class stream is class_key. */
uint32_t synth_scale_class(uint64_t class_key, uint64_t g) {
  return (uint32_t)(synth_bits(class_key, g) >> 62);
}

/* fp8 weight [rows][cols] (rows a multiple of 128): row group g uses the code
 * table of its class, codes[c * SYNTH_TABLE_SIZE + i]; scales_out[g] gets the
 * class's bf16 scale from scale_bits[c]. */
void synth_fill_fp8(uint8_t *dst, uint64_t rows, uint64_t cols, uint64_t key, uint64_t class_key,
                    const uint8_t *codes, const uint16_t *scale_bits, uint16_t *scales_out) {
  uint64_t groups = rows / 128u;
  for (uint64_t g = 0; g < groups; ++g) {
    uint32_t c = synth_scale_class(class_key, g);
    const uint8_t *t = codes + (uint64_t)c * SYNTH_TABLE_SIZE;
    if (scales_out) scales_out[g] = scale_bits[c];
    for (uint64_t i = g * 128u * cols; i < (g + 1u) * 128u * cols; ++i) dst[i] = t[synth_index(key, i)];
  }
}

uint64_t synth_key_c(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t sub, uint32_t attempt) {
  return synth_key(seed, layer, tensor, sub, attempt);
}

uint32_t synth_index_c(uint64_t key, uint64_t i) { return synth_index(key, i); }

/* log-Zipf router bias: b_e = ln(r_e^-s / H_{E,s}), r a permutation of 1..E
 * (Fisher-Yates driven by the BIAS_PERM stream of `seed`). */
void synth_zipf_bias(uint64_t seed, int E, double s, float *out) {
  int r[4096];
  if (E < 1 || E > 4096) return;
  for (int e = 0; e < E; ++e) r[e] = e + 1;
  uint64_t key = synth_key(seed, 0, SYNTH_T_BIAS_PERM, 0, 0);
  for (int i = E - 1; i >= 1; --i) {
    uint64_t j = synth_bits(key, (uint64_t)i) % (uint64_t)(i + 1);
    int t = r[i]; r[i] = r[j]; r[j] = t;
  }
  double hsum = 0.0;
  for (int q = 1; q <= E; ++q) hsum += pow((double)q, -s);
  for (int e = 0; e < E; ++e) out[e] = (float)(-s * log((double)r[e]) - log(hsum));
}
