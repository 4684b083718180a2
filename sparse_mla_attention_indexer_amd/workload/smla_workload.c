/*
 * smla_workload.c — seeded synthetic inputs and neutral comparisons (see smla_workload.h).
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) evaluated at a counter: draw(seed, stream, i) is the SplitMix64
 * output for state seed + (c + 1) * gamma, c = (stream << 48) | i. Normals use the Box-Muller
 * transform on the two 32-bit halves of one draw: normal element i of a stream takes draw i/2
 * and its cosine branch when i is even, its sine branch when i is odd.
 *
 * Storage formats written here (both sides of every comparison read these bytes):
 *  - bf16: IEEE binary32 rounded to the upper 16 bits, round-to-nearest-even.
 *  - e4m3: OCP 8-bit floating point E4M3 ("FN"): 1 sign, 4 exponent bits with bias 7, 3 mantissa
 *    bits; no infinities; S.1111.111 is NaN; largest finite magnitude 448. Encoding rounds to
 *    nearest even and saturates to +-448.
 *  - 656-byte latent row: bytes [0,512) e4m3 codes of dims 0..511; [512,528) four little-endian
 *    fp32 scales, one per 128-dim block; [528,656) 64 bf16 rope dims 512..575. A block's scale is
 *    fp32(amax / 448) (1 when the block is all zero) and its codes encode value / scale.
 */
#include "smla_workload.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

enum { STREAM_Q = 1, STREAM_LATENT = 2, STREAM_QIDX = 3, STREAM_KIDX = 4, STREAM_W = 5 };

static inline uint64_t draw(uint64_t seed, uint64_t stream, uint64_t i) {
  uint64_t z = seed + (((stream << 48) | i) + 1ULL) * GAMMA;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline void normal_pair(uint64_t x, double* z0, double* z1) {
  const double two32 = 4294967296.0;
  double u1 = ((double)(x >> 32) + 0.5) / two32;
  double u2 = ((double)(x & 0xFFFFFFFFULL) + 0.5) / two32;
  double r = sqrt(-2.0 * log(u1));
  *z0 = r * cos(2.0 * M_PI * u2);
  *z1 = r * sin(2.0 * M_PI * u2);
}

/* normal element i of `stream` */
static inline double normal_at(uint64_t seed, uint64_t stream, uint64_t i) {
  double z0, z1;
  normal_pair(draw(seed, stream, i >> 1), &z0, &z1);
  return (i & 1) ? z1 : z0;
}

/* normal elements [i0, i0 + n) of `stream`, i0 even, n even */
static inline void normal_run(uint64_t seed, uint64_t stream, uint64_t i0, int n, double* out) {
  for (int j = 0; j < n; j += 2) normal_pair(draw(seed, stream, (i0 + j) >> 1), out + j, out + j + 1);
}

static inline int8_t int8_m8_7(uint64_t x) { return (int8_t)((int)(x >> 60) - 8); }
static inline int32_t int_1_4(uint64_t x) { return (int32_t)(x >> 62) + 1; }

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* e4m3 encoding of y (already divided by the block scale): round to nearest even on the
 * e4m3 grid, saturating to +-448. Integer arithmetic on the binary64 bits keeps it exact. */
static uint8_t e4m3_encode(double y) {
  uint64_t u;
  memcpy(&u, &y, 8);
  uint8_t sign = (uint8_t)((u >> 56) & 0x80);
  u &= 0x7FFFFFFFFFFFFFFFULL;
  if (u > 0x7FF0000000000000ULL) return 0x7F; /* NaN */
  double a;
  memcpy(&a, &u, 8);
  if (a >= 448.0) return sign | 0x7E;
  if (a < 0.015625) { /* below 2^-6: subnormal grid of step 2^-9 */
    double m = a * 512.0; /* exact, in [0, 8) */
    int f = (int)m;
    double rem = m - (double)f;
    if (rem > 0.5 || (rem == 0.5 && (f & 1))) ++f;
    return sign | (uint8_t)f; /* f == 8 is the smallest normal, 2^-6 */
  }
  int E = (int)(u >> 52) - 1023;              /* a = 1.mant * 2^E, E in [-6, 8] */
  uint64_t mant = u & 0xFFFFFFFFFFFFFULL;     /* 52 fraction bits */
  uint64_t top = mant >> 49;                  /* 3 kept bits */
  uint64_t rem = mant & ((1ULL << 49) - 1);
  const uint64_t half = 1ULL << 48;
  if (rem > half || (rem == half && (top & 1))) ++top;
  if (top == 8) { top = 0; ++E; }
  int biased = E + 7;
  if (biased > 15 || (biased == 15 && top == 7)) return sign | 0x7E;
  return sign | (uint8_t)((biased << 3) | (int)top);
}

int32_t smla_workload_default_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  if (n < 1) n = 1;
  if (n > 256) n = 256;
  return (int32_t)n;
}

int smla_workload_dims_finish(smla_workload_dims* d) {
  if (!d) return SMLA_W_E_INVALID;
  if (d->batch < 1 || d->n_q < 1 || d->cached < 0 || d->H < 1 || d->D_qk < 1 || d->D_v < 1 ||
      d->D_v > d->D_qk || d->H_I < 1 || d->D_I < 1 || d->top_k < 1)
    return SMLA_W_E_INVALID;
  if (d->kv_format == SMLA_W_KV_FP8_656) {
    if (d->D_qk != 576 || d->D_v != 512) return SMLA_W_E_INVALID;
    d->row_bytes = 656;
  } else if (d->kv_format == SMLA_W_KV_BF16) {
    d->row_bytes = 2 * d->D_qk;
  } else {
    return SMLA_W_E_INVALID;
  }
  d->max_kv = d->cached + d->n_q;
  d->total_q = (int64_t)d->batch * d->n_q;
  d->total_rows = (int64_t)d->batch * d->max_kv;
  d->sm_scale = 1.0 / sqrt((double)d->D_qk);
  return SMLA_W_OK;
}

int smla_workload_dims_get(int32_t id, smla_workload_dims* out) {
  if (!out || id < 0 || id > 4) return SMLA_W_E_INVALID;
  smla_workload_dims d;
  memset(&d, 0, sizeof d);
  d.config_id = id;
  if (id == 0) {
    d.batch = 1; d.n_q = 512; d.cached = 0;
    d.H = 8; d.D_qk = 80; d.D_v = 64; d.H_I = 4; d.D_I = 32; d.top_k = 64;
    d.kv_format = SMLA_W_KV_BF16;
  } else {
    d.H = 64; d.D_qk = 576; d.D_v = 512; d.H_I = 64; d.D_I = 128; d.top_k = 2048;
    d.kv_format = SMLA_W_KV_FP8_656;
    if (id == 1) { d.batch = 32; d.n_q = 1; d.cached = 65536; }
    if (id == 2) { d.batch = 1; d.n_q = 2048; d.cached = 65536; }
    if (id == 3) { d.batch = 1; d.n_q = 32768; d.cached = 0; }
    if (id == 4) { d.batch = 4; d.n_q = 4; d.cached = 1048576; }
  }
  d.seed = 0x5EED0000ULL + (uint64_t)id;
  int rc = smla_workload_dims_finish(&d);
  d.config_id = id;
  *out = d;
  return rc;
}

/* ---- generation ------------------------------------------------------------------------- */

typedef struct {
  const smla_workload_dims* d;
  uint64_t seed;
  uint16_t* q; uint8_t* kv; int8_t* q_idx; int8_t* k_idx;
  int64_t t0, t1;   /* token range */
  int64_t r0, r1;   /* row range */
} gen_job;

static void gen_row(const smla_workload_dims* d, uint64_t seed, int64_t r, uint8_t* row) {
  const int D = d->D_qk;
  if (d->kv_format == SMLA_W_KV_BF16) {
    for (int j = 0; j < D; ++j) {
      uint16_t b = f32_to_bf16_rne((float)normal_at(seed, STREAM_LATENT, (uint64_t)(r * D + j)));
      row[2 * j] = (uint8_t)(b & 0xFF);
      row[2 * j + 1] = (uint8_t)(b >> 8);
    }
    return;
  }
  double x[576];
  normal_run(seed, STREAM_LATENT, (uint64_t)(r * 576), 576, x);
  for (int blk = 0; blk < 4; ++blk) {
    double amax = 0.0;
    for (int j = 0; j < 128; ++j) {
      double a = fabs(x[blk * 128 + j]);
      if (a > amax) amax = a;
    }
    float scale = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
    for (int j = 0; j < 128; ++j) row[blk * 128 + j] = e4m3_encode(x[blk * 128 + j] / (double)scale);
    memcpy(row + 512 + 4 * blk, &scale, 4); /* host is little-endian (x86-64) */
  }
  for (int j = 0; j < 64; ++j) {
    uint16_t b = f32_to_bf16_rne((float)x[512 + j]);
    row[528 + 2 * j] = (uint8_t)(b & 0xFF);
    row[528 + 2 * j + 1] = (uint8_t)(b >> 8);
  }
}

static void* gen_worker(void* arg) {
  gen_job* j = (gen_job*)arg;
  const smla_workload_dims* d = j->d;
  const uint64_t s = j->seed;
  if (j->q) {
    const int64_t per = (int64_t)d->H * d->D_qk;
    for (int64_t t = j->t0; t < j->t1; ++t)
      for (int64_t e = 0; e < per; ++e) {
        int64_t i = t * per + e;
        j->q[i] = f32_to_bf16_rne((float)normal_at(s, STREAM_Q, (uint64_t)i));
      }
  }
  if (j->q_idx) {
    const int64_t per = (int64_t)d->H_I * d->D_I;
    for (int64_t t = j->t0; t < j->t1; ++t)
      for (int64_t e = 0; e < per; ++e) {
        int64_t i = t * per + e;
        j->q_idx[i] = int8_m8_7(draw(s, STREAM_QIDX, (uint64_t)i));
      }
  }
  if (j->kv)
    for (int64_t r = j->r0; r < j->r1; ++r) gen_row(d, s, r, j->kv + r * d->row_bytes);
  if (j->k_idx)
    for (int64_t r = j->r0; r < j->r1; ++r)
      for (int e = 0; e < d->D_I; ++e) {
        int64_t i = r * d->D_I + e;
        j->k_idx[i] = int8_m8_7(draw(s, STREAM_KIDX, (uint64_t)i));
      }
  return NULL;
}

int smla_workload_gen(const smla_workload_dims* d, uint64_t seed, int32_t nthreads, uint16_t* q,
                      uint8_t* kv, int8_t* q_idx, int8_t* k_idx, int32_t* w) {
  if (!d || d->total_q < 1 || d->total_rows < 1 || d->row_bytes < 1) return SMLA_W_E_INVALID;
  if (d->kv_format == SMLA_W_KV_FP8_656 && (d->D_qk != 576 || d->row_bytes != 656))
    return SMLA_W_E_INVALID;
  if (d->kv_format == SMLA_W_KV_BF16 && d->row_bytes != 2 * d->D_qk) return SMLA_W_E_INVALID;
  if (w)
    for (int h = 0; h < d->H_I; ++h) w[h] = int_1_4(draw(seed, STREAM_W, (uint64_t)h));
  int nt = nthreads > 0 ? nthreads : smla_workload_default_threads();
  if (nt > 256) nt = 256;
  gen_job jobs[256];
  pthread_t th[256];
  for (int i = 0; i < nt; ++i) {
    jobs[i].d = d; jobs[i].seed = seed;
    jobs[i].q = q; jobs[i].kv = kv; jobs[i].q_idx = q_idx; jobs[i].k_idx = k_idx;
    jobs[i].t0 = d->total_q * i / nt; jobs[i].t1 = d->total_q * (i + 1) / nt;
    jobs[i].r0 = d->total_rows * i / nt; jobs[i].r1 = d->total_rows * (i + 1) / nt;
  }
  for (int i = 1; i < nt; ++i) pthread_create(&th[i], NULL, gen_worker, &jobs[i]);
  gen_worker(&jobs[0]);
  for (int i = 1; i < nt; ++i) pthread_join(th[i], NULL);
  return SMLA_W_OK;
}

int smla_workload_latent_f64(const smla_workload_dims* d, uint64_t seed, int64_t row0,
                             int64_t nrows, double* out) {
  if (!d || !out || row0 < 0 || nrows < 0 || row0 + nrows > d->total_rows) return SMLA_W_E_INVALID;
  const int D = d->D_qk;
  for (int64_t r = 0; r < nrows; ++r)
    for (int j = 0; j < D; ++j)
      out[r * D + j] = normal_at(seed, STREAM_LATENT, (uint64_t)((row0 + r) * D + j));
  return SMLA_W_OK;
}

/* ---- comparisons ------------------------------------------------------------------------ */

typedef struct { int32_t idx, score; } pair_t;

static int cmp_pair(const void* a, const void* b) {
  const pair_t* x = (const pair_t*)a;
  const pair_t* y = (const pair_t*)b;
  /* -1 padding sorts last */
  uint32_t ux = (uint32_t)x->idx, uy = (uint32_t)y->idx;
  return ux < uy ? -1 : (ux > uy ? 1 : 0);
}

int smla_check_topk(const int32_t* got_idx, const int32_t* got_score, const int32_t* ref_idx,
                    const int32_t* ref_score, int64_t rows, int32_t top_k, smla_topk_report* rep) {
  if (!got_idx || !ref_idx || rows < 0 || top_k < 1) return SMLA_W_E_INVALID;
  pair_t* a = (pair_t*)malloc(sizeof(pair_t) * (size_t)top_k);
  pair_t* b = (pair_t*)malloc(sizeof(pair_t) * (size_t)top_k);
  if (!a || !b) { free(a); free(b); return SMLA_W_E_INVALID; }
  const int use_scores = got_score && ref_score;
  smla_topk_report r = {rows, 0, -1, 0};
  for (int64_t i = 0; i < rows; ++i) {
    for (int j = 0; j < top_k; ++j) {
      int64_t o = i * top_k + j;
      a[j].idx = got_idx[o] < 0 ? -1 : got_idx[o];
      b[j].idx = ref_idx[o] < 0 ? -1 : ref_idx[o];
      a[j].score = (use_scores && a[j].idx >= 0) ? got_score[o] : 0;
      b[j].score = (use_scores && b[j].idx >= 0) ? ref_score[o] : 0;
    }
    qsort(a, (size_t)top_k, sizeof(pair_t), cmp_pair);
    qsort(b, (size_t)top_k, sizeof(pair_t), cmp_pair);
    int64_t bad = 0;
    for (int j = 0; j < top_k; ++j)
      if (a[j].idx != b[j].idx || a[j].score != b[j].score) ++bad;
    if (bad) {
      if (r.first_bad < 0) r.first_bad = i;
      r.rows_bad++;
      r.bad_entries += bad;
    }
  }
  free(a);
  free(b);
  if (rep) *rep = r;
  return r.rows_bad ? SMLA_W_E_MISMATCH : SMLA_W_OK;
}

int smla_check_attn(const uint16_t* got, const double* ref, int64_t n, double atol,
                    double rel_l2_tol, smla_attn_report* rep) {
  if (!got || !ref || n < 0) return SMLA_W_E_INVALID;
  smla_attn_report r = {0.0, 0.0, -1, 0};
  double num = 0.0, den = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)got[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    double g = (double)f;
    if (!isfinite(g)) { r.n_nonfinite++; continue; }
    double e = fabs(g - ref[i]);
    if (e > r.max_abs) { r.max_abs = e; r.argmax = i; }
    num += (g - ref[i]) * (g - ref[i]);
    den += ref[i] * ref[i];
  }
  r.rel_l2 = den > 0 ? sqrt(num / den) : sqrt(num);
  if (rep) *rep = r;
  return (r.n_nonfinite || r.max_abs > atol || r.rel_l2 > rel_l2_tol) ? SMLA_W_E_MISMATCH : SMLA_W_OK;
}
