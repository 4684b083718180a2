/*
 * smla_oracle.c — CPU oracle (TEST INFRASTRUCTURE ONLY; see smla_oracle.h for the definitions
 * and the passages they follow). Every quantity is computed straight from its definition:
 * integer indexer scores in int64, a full sort for top-k, and fp64 softmax attention over the
 * dequantised rows. Worker threads split the listed query tokens; they never reorder the
 * arithmetic inside one token.
 */
#include "smla_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

int32_t smla_oracle_default_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  if (n < 1) n = 1;
  if (n > 256) n = 256;
  return (int32_t)n;
}

/* OCP 8-bit floating point, E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent field 0 is subnormal: (m/8) * 2^(1-7). S.1111.111 is NaN; there is no infinity. */
double smla_oracle_e4m3(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, 1 - 7);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double smla_oracle_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round to nearest-even on the E4M3 grid: exponents -6..8 carry 3 fraction bits, below 2^-6
 * the grid is the multiples of 2^-9; rint() rounds half to even in the default mode. */
uint8_t smla_oracle_e4m3_encode(double v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E; /* the largest finite magnitude (S.1111.110) */
  if (a < 0.015625) return sign | (uint8_t)rint(a * 512.0); /* 0..8; 8 is the code of 2^-6 */
  int e;
  const double f = frexp(a, &e); /* a = f * 2^e, 0.5 <= f < 1 */
  int E = e - 1;                  /* a = (2f) * 2^E, 1 <= 2f < 2 */
  double m = rint((2.0 * f - 1.0) * 8.0);
  if (m == 8.0) {
    m = 0.0;
    E += 1;
  }
  if (E > 8 || (E == 8 && m == 7.0)) return sign | 0x7E;
  return sign | (uint8_t)(((E + 7) << 3) | (int)m);
}

int smla_oracle_fp8_row_encode(const uint16_t* latent, uint8_t* row) {
  for (int b = 0; b < 4; ++b) {
    double amax = 0.0;
    for (int d = 128 * b; d < 128 * (b + 1); ++d) amax = fmax(amax, fabs(smla_oracle_bf16(latent[d])));
    const float scale = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
    for (int d = 128 * b; d < 128 * (b + 1); ++d)
      row[d] = smla_oracle_e4m3_encode(smla_oracle_bf16(latent[d]) / (double)scale);
    memcpy(row + 512 + 4 * b, &scale, 4);
  }
  for (int d = 0; d < 64; ++d) {
    row[528 + 2 * d] = (uint8_t)(latent[512 + d] & 0xFF);
    row[529 + 2 * d] = (uint8_t)(latent[512 + d] >> 8);
  }
  return 0;
}

int smla_oracle_dequant_row(const uint8_t* row, int32_t fmt, int32_t D_qk, double* out) {
  if (!row || !out) return -1;
  if (fmt == 0) {
    for (int d = 0; d < D_qk; ++d) out[d] = smla_oracle_bf16((uint16_t)(row[2 * d] | (row[2 * d + 1] << 8)));
    return 0;
  }
  if (fmt != 1 || D_qk != 576) return -1;
  /* 656-byte row: [512 e4m3 codes][4 fp32 block scales][64 bf16 rope values] */
  float scale[4];
  memcpy(scale, row + 512, 16);
  for (int d = 0; d < 512; ++d) out[d] = smla_oracle_e4m3(row[d]) * (double)scale[d / 128];
  for (int d = 0; d < 64; ++d) {
    const uint8_t* b = row + 528 + 2 * d;
    out[512 + d] = smla_oracle_bf16((uint16_t)(b[0] | (b[1] << 8)));
  }
  return 0;
}

int smla_oracle_indexer_scores(const int8_t* q_tok, const int8_t* keys, const int32_t* w,
                               int32_t H_I, int32_t D_I, int64_t n, int64_t* out) {
  /* |q_d * k_d| <= 2^14, so a dot product over D_I <= 2^16 dims is exact in int32 */
  if (D_I < 1 || D_I > 65536 || H_I < 1) return -1;
  int bad = 0;
  for (int64_t s = 0; s < n; ++s) {
    const int8_t* k = keys + s * D_I;
    int64_t score = 0;
    for (int h = 0; h < H_I; ++h) {
      const int8_t* qh = q_tok + (int64_t)h * D_I;
      int32_t dot = 0;
      for (int d = 0; d < D_I; ++d) dot += (int32_t)qh[d] * (int32_t)k[d];
      int64_t relu = dot > 0 ? dot : 0;
      score += (int64_t)w[h] * relu;
    }
    if (score < 0 || score > 2147483647LL) bad = 1;
    out[s] = score;
  }
  return bad ? -1 : 0;
}

int smla_oracle_indexer_scores_fp8(const uint8_t* q_tok, const uint8_t* keys, const float* k_scale,
                                   const float* w, int32_t H_I, int32_t D_I, int64_t n,
                                   double* out, double* abs_out) {
  /* every E4M3 value is a multiple of 2^-9 below 2^9, so each product is a multiple of 2^-18
   * below 2^18 and a sum of D_I <= 2^16 of them needs at most 52 bits: exact in binary64 */
  if (D_I < 1 || D_I > 65536 || H_I < 1) return -1;
  for (int32_t h = 0; h < H_I; ++h)
    if (!(w[h] >= 0.0f) || !isfinite(w[h])) return -1;
  for (int64_t i = 0; i < (int64_t)H_I * D_I; ++i)
    if (isnan(smla_oracle_e4m3(q_tok[i]))) return -1;
  for (int64_t s = 0; s < n; ++s) {
    const uint8_t* k = keys + s * D_I;
    const double scale = (double)k_scale[s];
    if (!(scale >= 0.0) || !isfinite(scale)) return -1;
    double acc = 0.0, mag = 0.0;
    for (int32_t h = 0; h < H_I; ++h) {
      const uint8_t* qh = q_tok + (int64_t)h * D_I;
      double dot = 0.0, dabs = 0.0;
      for (int32_t d = 0; d < D_I; ++d) {
        const double kv = smla_oracle_e4m3(k[d]);
        if (isnan(kv)) return -1;
        const double prod = smla_oracle_e4m3(qh[d]) * kv;
        dot += prod;
        dabs += fabs(prod);
      }
      acc += (double)w[h] * (dot > 0.0 ? dot : 0.0);
      mag += (double)w[h] * dabs;
    }
    out[s] = scale * acc;
    if (abs_out) abs_out[s] = scale * mag;
  }
  return 0;
}

typedef struct {
  int64_t score;
  int64_t s;
} cand_t;

/* Total order of the selection: larger score first; among equal scores, lower index first. */
static int cmp_cand(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->score != y->score) return x->score > y->score ? -1 : 1;
  return x->s < y->s ? -1 : (x->s > y->s ? 1 : 0);
}

int smla_oracle_topk(const int64_t* scores, int64_t n, int32_t top_k, int32_t* idx,
                     int32_t* score) {
  if (n < 0 || top_k < 1) return -1;
  cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
  if (!c) return -1;
  for (int64_t s = 0; s < n; ++s) {
    c[s].score = scores[s];
    c[s].s = s;
  }
  qsort(c, (size_t)n, sizeof(cand_t), cmp_cand);
  for (int32_t j = 0; j < top_k; ++j) {
    if (j < n) {
      idx[j] = (int32_t)c[j].s;
      if (score) score[j] = (int32_t)c[j].score;
    } else {
      idx[j] = -1;
      if (score) score[j] = -1;
    }
  }
  free(c);
  return 0;
}

int smla_oracle_topk_merge(const int32_t* idx_lists, const int32_t* score_lists, int32_t n_lists,
                           int32_t k_in, int32_t top_k, int32_t* idx, int32_t* score) {
  if (n_lists < 1 || k_in < 1 || top_k < 1) return -1;
  cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)n_lists * (size_t)k_in);
  if (!c) return -1;
  int64_t n = 0;
  for (int32_t l = 0; l < n_lists; ++l)
    for (int32_t j = 0; j < k_in; ++j) {
      const int32_t local = idx_lists[(int64_t)l * k_in + j];
      if (local < 0) continue;
      c[n].score = score_lists[(int64_t)l * k_in + j];
      c[n].s = (int64_t)local * n_lists + l;  /* shard l holds tokens l, l + n_lists, ... */
      ++n;
    }
  qsort(c, (size_t)n, sizeof(cand_t), cmp_cand);
  for (int32_t j = 0; j < top_k; ++j) {
    idx[j] = j < n ? (int32_t)c[j].s : -1;
    if (score) score[j] = j < n ? (int32_t)c[j].score : -1;
  }
  free(c);
  return 0;
}

int smla_oracle_lse_merge(int32_t n_parts, int32_t H, int32_t D_v, const double* outs,
                          const double* lses, double* out, double* lse) {
  if (n_parts < 1 || H < 1 || D_v < 1) return -1;
  for (int32_t h = 0; h < H; ++h) {
    double m = -INFINITY;
    for (int32_t i = 0; i < n_parts; ++i) m = fmax(m, lses[(int64_t)i * H + h]);
    double z = 0.0;
    for (int32_t d = 0; d < D_v; ++d) out[(int64_t)h * D_v + d] = 0.0;
    if (m == -INFINITY) {  /* no part saw a row */
      lse[h] = -INFINITY;
      continue;
    }
    for (int32_t i = 0; i < n_parts; ++i) {
      const double li = lses[(int64_t)i * H + h];
      if (li == -INFINITY) continue;
      const double wi = exp(li - m);
      z += wi;
      for (int32_t d = 0; d < D_v; ++d)
        out[(int64_t)h * D_v + d] += wi * outs[((int64_t)i * H + h) * D_v + d];
    }
    for (int32_t d = 0; d < D_v; ++d) out[(int64_t)h * D_v + d] /= z;
    lse[h] = m + log(z);
  }
  return 0;
}

static int cmp_i64(const void* a, const void* b) {
  const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return x < y ? -1 : (x > y ? 1 : 0);
}

int smla_oracle_hot_resolve(int32_t n_q, int32_t top_k, const int32_t* idx, int64_t kv_len,
                            int64_t resident_from, int32_t H, int32_t* hot_tok, int32_t* hot_age,
                            int32_t step, int64_t hot_base, int32_t* idx_out, int32_t* copy_src,
                            int32_t* n_copy) {
  /* the hot buffer must lie in rows every query token of the request sees: token j sits at
   * position kv_len - n_q + j and attends to rows up to it, so the offloaded prefix (and the
   * buffer inside it) ends at or before the first token's position */
  if (kv_len >= 0) {
    if (resident_from < 0 || resident_from > kv_len - n_q + 1) return -3;
    if (resident_from > 0 && (hot_base < 0 || hot_base + H > resident_from)) return -3;
  }
  /* the distinct offloaded selections of the request, ascending */
  int64_t* u = (int64_t*)malloc(sizeof(int64_t) * ((size_t)n_q * top_k + 1));
  int32_t* slot_of = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n_q * top_k + 1));
  unsigned char* used = (unsigned char*)calloc((size_t)H + 1, 1);
  if (!u || !slot_of || !used) { free(u); free(slot_of); free(used); return -1; }
  int64_t n = 0;
  for (int64_t i = 0; i < (int64_t)n_q * top_k; ++i)
    if (idx[i] >= 0 && idx[i] < resident_from) u[n++] = idx[i];
  qsort(u, (size_t)n, sizeof(int64_t), cmp_i64);
  int64_t m = 0;
  for (int64_t i = 0; i < n; ++i)
    if (m == 0 || u[m - 1] != u[i]) u[m++] = u[i];
  /* the misses fit the slots not hit exactly when the distinct rows fit all slots; a request
   * that does not fit is rejected before anything changes */
  if (m > H) { free(u); free(slot_of); free(used); return -2; }
  /* hits: a slot already holding the token is used again (its age becomes this step) */
  int64_t hits = 0;
  for (int64_t i = 0; i < m; ++i) {
    slot_of[i] = -1;
    for (int32_t j = 0; j < H; ++j)
      if (hot_tok[j] == u[i]) {
        slot_of[i] = j;
        used[j] = 1;
        hot_age[j] = step;
        ++hits;
        break;
      }
  }
  /* misses, ascending, take the least recently used free slots: (age, slot) ascending */
  int32_t nc = 0;
  for (int64_t i = 0; i < m; ++i) {
    if (slot_of[i] >= 0) continue;
    int32_t best = -1;
    for (int32_t j = 0; j < H; ++j) {
      if (used[j]) continue;
      if (best < 0 || hot_age[j] < hot_age[best]) best = j;  /* ties: the lower slot */
    }
    used[best] = 1;
    slot_of[i] = best;
    hot_tok[best] = (int32_t)u[i];
    hot_age[best] = step;
    if (copy_src) copy_src[2 * nc] = (int32_t)u[i], copy_src[2 * nc + 1] = best;
    ++nc;
  }
  if (n_copy) *n_copy = nc;
  /* every selection: resident rows in place, offloaded ones at their slot */
  for (int64_t i = 0; i < (int64_t)n_q * top_k; ++i) {
    const int32_t s = idx[i];
    if (s < 0) { idx_out[i] = -1; continue; }
    if (s >= resident_from) { idx_out[i] = s; continue; }
    int64_t lo = 0, hi = m - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (u[mid] < s) lo = mid + 1; else hi = mid;
    }
    idx_out[i] = (int32_t)(hot_base + slot_of[lo]);
  }
  free(u);
  free(slot_of);
  free(used);
  return 0;
}

int smla_oracle_attend(const uint16_t* q_tok, const uint8_t* rows, int32_t fmt, int32_t row_bytes,
                       int32_t H, int32_t D_qk, int32_t D_v, const int32_t* idx, int32_t top_k,
                       double sm_scale, double* out, double* lse) {
  int32_t nsel = 0;
  for (int32_t i = 0; i < top_k; ++i) nsel += idx[i] >= 0;
  if (nsel == 0) return -1;
  double* v = (double*)malloc(sizeof(double) * (size_t)nsel * (size_t)D_qk);
  double* q = (double*)malloc(sizeof(double) * (size_t)D_qk);
  double* l = (double*)malloc(sizeof(double) * (size_t)nsel);
  if (!v || !q || !l) { free(v); free(q); free(l); return -1; }
  /* dequantise each selected row once; every head reads the same rows */
  int32_t r = 0;
  for (int32_t i = 0; i < top_k; ++i) {
    if (idx[i] < 0) continue;
    if (smla_oracle_dequant_row(rows + (int64_t)idx[i] * row_bytes, fmt, D_qk, v + (int64_t)r * D_qk)) {
      free(v); free(q); free(l);
      return -1;
    }
    ++r;
  }
  for (int32_t h = 0; h < H; ++h) {
    for (int d = 0; d < D_qk; ++d) q[d] = smla_oracle_bf16(q_tok[(int64_t)h * D_qk + d]);
    double m = -INFINITY;
    for (int32_t i = 0; i < nsel; ++i) {
      const double* vi = v + (int64_t)i * D_qk;
      double dot = 0.0;
      for (int d = 0; d < D_qk; ++d) dot += q[d] * vi[d];
      l[i] = sm_scale * dot;
      if (l[i] > m) m = l[i];
    }
    double Z = 0.0;
    for (int32_t i = 0; i < nsel; ++i) {
      l[i] = exp(l[i] - m); /* l now holds e_i */
      Z += l[i];
    }
    if (out) {
      double* o = out + (int64_t)h * D_v;
      for (int d = 0; d < D_v; ++d) o[d] = 0.0;
      for (int32_t i = 0; i < nsel; ++i) {
        const double p = l[i] / Z;
        const double* vi = v + (int64_t)i * D_qk;
        for (int d = 0; d < D_v; ++d) o[d] += p * vi[d];
      }
    }
    if (lse) lse[h] = m + log(Z);
  }
  free(v);
  free(q);
  free(l);
  return 0;
}

/* ---- batched drivers -------------------------------------------------------------------- */

typedef struct {
  int32_t batch;
  const int32_t* n_q;
  const int64_t* kv_len;
  int64_t* q0; /* [batch+1] token prefix */
  int64_t* r0; /* [batch+1] row prefix */
} layout_t;

static int layout_init(layout_t* L, int32_t batch, const int32_t* n_q, const int64_t* kv_len) {
  L->batch = batch;
  L->n_q = n_q;
  L->kv_len = kv_len;
  L->q0 = (int64_t*)calloc((size_t)batch + 1, sizeof(int64_t));
  L->r0 = (int64_t*)calloc((size_t)batch + 1, sizeof(int64_t));
  if (!L->q0 || !L->r0) return -1;
  for (int32_t b = 0; b < batch; ++b) {
    if (n_q[b] < 0 || kv_len[b] < n_q[b]) return -1;
    L->q0[b + 1] = L->q0[b] + n_q[b];
    L->r0[b + 1] = L->r0[b] + kv_len[b];
  }
  return 0;
}

static void layout_free(layout_t* L) {
  free(L->q0);
  free(L->r0);
}

/* request, position and first row of global token t; -1 if t is out of range */
static int32_t locate(const layout_t* L, int64_t t, int64_t* p, int64_t* row0) {
  for (int32_t b = 0; b < L->batch; ++b)
    if (t >= L->q0[b] && t < L->q0[b + 1]) {
      *p = L->kv_len[b] - L->n_q[b] + (t - L->q0[b]);
      *row0 = L->r0[b];
      return b;
    }
  return -1;
}

typedef struct {
  const layout_t* L;
  const int8_t* q_idx; const int8_t* k_idx; const int32_t* w;
  int32_t H_I, D_I, top_k;
  const uint16_t* q; const uint8_t* kv; int32_t fmt, row_bytes, H, D_qk, D_v;
  const int32_t* idx; double sm_scale;
  const int64_t* tokens; int64_t i0, i1;
  int32_t* idx_out; int32_t* score_out; double* out; double* lse;
  int rc;
} job_t;

static void* topk_worker(void* arg) {
  job_t* j = (job_t*)arg;
  int64_t* sc = NULL;
  int64_t cap = 0;
  for (int64_t i = j->i0; i < j->i1; ++i) {
    int64_t p, row0;
    int64_t t = j->tokens[i];
    if (locate(j->L, t, &p, &row0) < 0) { j->rc = -1; break; }
    int64_t n = p + 1;
    if (n > cap) {
      free(sc);
      sc = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
      cap = n;
      if (!sc) { j->rc = -1; break; }
    }
    if (smla_oracle_indexer_scores(j->q_idx + t * (int64_t)j->H_I * j->D_I, j->k_idx + row0 * j->D_I,
                                   j->w, j->H_I, j->D_I, n, sc))
      j->rc = -1;
    if (smla_oracle_topk(sc, n, j->top_k, j->idx_out + i * j->top_k,
                         j->score_out ? j->score_out + i * j->top_k : NULL))
      j->rc = -1;
  }
  free(sc);
  return NULL;
}

static void* mla_worker(void* arg) {
  job_t* j = (job_t*)arg;
  for (int64_t i = j->i0; i < j->i1; ++i) {
    int64_t p, row0;
    int64_t t = j->tokens[i];
    if (locate(j->L, t, &p, &row0) < 0) { j->rc = -1; break; }
    /* every selected index must be a row this token may see */
    const int32_t* ix = j->idx + t * j->top_k;
    for (int32_t k = 0; k < j->top_k; ++k)
      if (ix[k] > p) j->rc = -1;
    if (j->rc) break;
    if (smla_oracle_attend(j->q + t * (int64_t)j->H * j->D_qk, j->kv + row0 * j->row_bytes, j->fmt,
                           j->row_bytes, j->H, j->D_qk, j->D_v, ix, j->top_k, j->sm_scale,
                           j->out ? j->out + i * (int64_t)j->H * j->D_v : NULL,
                           j->lse ? j->lse + i * (int64_t)j->H : NULL))
      j->rc = -1;
  }
  return NULL;
}

static int run_jobs(job_t* proto, int64_t n_tokens, int32_t nthreads, void* (*fn)(void*)) {
  int nt = nthreads > 0 ? nthreads : smla_oracle_default_threads();
  if (nt > 256) nt = 256;
  if (nt > n_tokens) nt = (int)(n_tokens > 0 ? n_tokens : 1);
  job_t jobs[256];
  pthread_t th[256];
  for (int i = 0; i < nt; ++i) {
    jobs[i] = *proto;
    jobs[i].i0 = n_tokens * i / nt;
    jobs[i].i1 = n_tokens * (i + 1) / nt;
    jobs[i].rc = 0;
  }
  for (int i = 1; i < nt; ++i) pthread_create(&th[i], NULL, fn, &jobs[i]);
  fn(&jobs[0]);
  int rc = jobs[0].rc;
  for (int i = 1; i < nt; ++i) {
    pthread_join(th[i], NULL);
    if (jobs[i].rc) rc = jobs[i].rc;
  }
  return rc;
}

int smla_oracle_indexer_topk_batch(int32_t batch, const int32_t* n_q, const int64_t* kv_len,
                                   const int8_t* q_idx, const int8_t* k_idx, const int32_t* w,
                                   int32_t H_I, int32_t D_I, int32_t top_k, const int64_t* tokens,
                                   int64_t n_tokens, int32_t* idx_out, int32_t* score_out,
                                   int32_t nthreads) {
  if (batch < 1 || !n_q || !kv_len || !q_idx || !k_idx || !w || !tokens || !idx_out || top_k < 1)
    return -1;
  layout_t L;
  if (layout_init(&L, batch, n_q, kv_len)) { layout_free(&L); return -1; }
  job_t proto;
  memset(&proto, 0, sizeof proto);
  proto.L = &L; proto.q_idx = q_idx; proto.k_idx = k_idx; proto.w = w;
  proto.H_I = H_I; proto.D_I = D_I; proto.top_k = top_k; proto.tokens = tokens;
  proto.idx_out = idx_out; proto.score_out = score_out;
  int rc = run_jobs(&proto, n_tokens, nthreads, topk_worker);
  layout_free(&L);
  return rc;
}

int smla_oracle_sparse_mla_batch(int32_t batch, const int32_t* n_q, const int64_t* kv_len,
                                 const uint16_t* q, const uint8_t* kv, int32_t fmt,
                                 int32_t row_bytes, int32_t H, int32_t D_qk, int32_t D_v,
                                 const int32_t* idx, int32_t top_k, double sm_scale,
                                 const int64_t* tokens, int64_t n_tokens, double* out, double* lse,
                                 int32_t nthreads) {
  if (batch < 1 || !n_q || !kv_len || !q || !kv || !idx || !tokens || top_k < 1) return -1;
  layout_t L;
  if (layout_init(&L, batch, n_q, kv_len)) { layout_free(&L); return -1; }
  job_t proto;
  memset(&proto, 0, sizeof proto);
  proto.L = &L; proto.q = q; proto.kv = kv; proto.fmt = fmt; proto.row_bytes = row_bytes;
  proto.H = H; proto.D_qk = D_qk; proto.D_v = D_v; proto.idx = idx; proto.top_k = top_k;
  proto.sm_scale = sm_scale; proto.tokens = tokens; proto.out = out; proto.lse = lse;
  int rc = run_jobs(&proto, n_tokens, nthreads, mla_worker);
  layout_free(&L);
  return rc;
}
