/*
 * gqa_oracle.c -- plain fp64 CPU oracle (see gqa_oracle.h for the contract).
 *
 * TEST INFRASTRUCTURE ONLY: called by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.
 *
 * The code follows the plain definition of the pages and nothing else: no
 * tiling, no online softmax, no split of the key range.  Each (query, head)
 * row materialises its whole score vector, takes its maximum, exponentiates
 * and normalises.  Work items (query, head) are spread over POSIX threads;
 * that changes nothing in the arithmetic of any one item.
 *
 * Sources (cited by page title and section):
 *  - "Deep dive into Muse Glimmer" (shishifenxi.com), section 01: 32 query
 *    heads share 2 KV heads of dimension 128; local layers see the nearby
 *    2048 tokens, global layers the whole context.
 *  - "Tomas Koutsky explains how Meta fits Muse Glimmer into 24 GB"
 *    (runtimewire.com), "Narrow cache": 39 of 52 layers use a 2048-token
 *    sliding window, 13 see the full sequence; "Long context still costs
 *    compute": global layers omit RoPE, order reaches them through the causal
 *    mask, the local layers carry RoPE.
 * Readings where the pages are silent: the window holds 2048 positions
 * including the query itself; query head h reads KV head h / (hq/hkv); RoPE
 * rotates the pairs (c, c + d/2) by t * theta^(-c/(d/2)).
 */
#include "gqa_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

static double widen_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void gqa_oracle_rope(const double* x, int32_t d, double t, double theta,
                     double* out) {
  const int32_t half = d / 2;
  for (int32_t c = 0; c < half; ++c) {
    const double omega = pow(theta, -(double)c / (double)half);
    const double a = t * omega;
    const double cs = cos(a), sn = sin(a);
    const double x0 = x[c], x1 = x[c + half];
    out[c] = x0 * cs - x1 * sn;
    out[c + half] = x1 * cs + x0 * sn;
  }
}

/* ------------------------------------------------------------------ */
/* a tiny parallel-for over [0, n)                                      */

typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);

typedef struct {
  range_fn fn;
  void* ctx;
  int64_t lo, hi;
} range_job;

static void* range_thread(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static void parallel_for(int64_t n, int32_t nthreads, range_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > n) nthreads = (int32_t)(n > 0 ? n : 1);
  if (nthreads == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  range_job* jobs = (range_job*)malloc(sizeof(range_job) * (size_t)nthreads);
  int32_t started = 0;
  for (int32_t t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].lo = n * t / nthreads;
    jobs[t].hi = n * (t + 1) / nthreads;
    if (pthread_create(&th[t], NULL, range_thread, &jobs[t]) != 0) {
      fn(ctx, jobs[t].lo, jobs[t].hi); /* run inline if a thread fails */
      jobs[t].fn = NULL;
    } else {
      ++started;
    }
  }
  for (int32_t t = 0; t < nthreads; ++t)
    if (jobs[t].fn) pthread_join(th[t], NULL);
  (void)started;
  free(th);
  free(jobs);
}

/* ------------------------------------------------------------------ */

typedef struct {
  const gqa_oracle_cfg* cfg;
  const uint16_t* q;
  const int64_t* qpos;
  const uint16_t* k;
  const uint16_t* v;
  const double* k64;  /* keys / values given as exact doubles (a quantised */
  const double* v64;  /* cache, dequantised) instead of bf16 bits, or NULL */
  int64_t kpos0, nk;
  const double* krot; /* [nk][hkv][d] rotated keys when cfg->rope, else NULL */
  int64_t jlo, jhi;   /* extra key restriction for partial sums */
  int32_t normalise;  /* 1: out = o / l ; 0: write m, l, o       */
  double* out;        /* [nq][hq][d] */
  double* m;          /* [nq][hq]    */
  double* l;          /* [nq][hq]    */
} attend_ctx;

typedef struct {
  attend_ctx* a;
} rot_ctx;

static void rotate_keys(void* p, int64_t lo, int64_t hi) {
  attend_ctx* a = ((rot_ctx*)p)->a;
  const int32_t d = a->cfg->d, hkv = a->cfg->hkv;
  double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t r = lo; r < hi; ++r) {
    for (int32_t g = 0; g < hkv; ++g) {
      if (a->k64) {
        memcpy(tmp, a->k64 + (r * hkv + g) * d, sizeof(double) * (size_t)d);
      } else {
        const uint16_t* src = a->k + (r * hkv + g) * d;
        for (int32_t c = 0; c < d; ++c) tmp[c] = widen_bf16(src[c]);
      }
      gqa_oracle_rope(tmp, d, (double)(a->kpos0 + r), a->cfg->theta,
                      (double*)a->krot + (r * hkv + g) * d);
    }
  }
  free(tmp);
}

/* Visible key positions of a query at position i: [lo, i]. */
static int64_t visible_lo(const gqa_oracle_cfg* cfg, int64_t i) {
  if (cfg->window > 0) {
    int64_t lo = i - (int64_t)cfg->window + 1;
    return lo > 0 ? lo : 0;
  }
  return 0;
}

static void attend_rows(void* p, int64_t lo_item, int64_t hi_item) {
  attend_ctx* a = (attend_ctx*)p;
  const gqa_oracle_cfg* cfg = a->cfg;
  const int32_t d = cfg->d, hq = cfg->hq, hkv = cfg->hkv;
  const int32_t group = hq / hkv;
  double* qv = (double*)malloc(sizeof(double) * (size_t)d);
  double* kw = (double*)malloc(sizeof(double) * (size_t)d);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  double* s = NULL;
  int64_t s_cap = 0;

  for (int64_t item = lo_item; item < hi_item; ++item) {
    const int64_t n = item / hq;
    const int32_t h = (int32_t)(item % hq);
    const int32_t g = h / group;
    const int64_t i = a->qpos[n];
    int64_t jlo = visible_lo(cfg, i), jhi = i + 1; /* [jlo, jhi) */
    if (jlo < a->jlo) jlo = a->jlo;
    if (jhi > a->jhi) jhi = a->jhi;
    const int64_t cnt = jhi > jlo ? jhi - jlo : 0;

    const uint16_t* qsrc = a->q + (n * hq + h) * d;
    for (int32_t c = 0; c < d; ++c) qv[c] = widen_bf16(qsrc[c]);
    if (cfg->rope) gqa_oracle_rope(qv, d, (double)i, cfg->theta, qv);

    if (cnt > s_cap) {
      free(s);
      s = (double*)malloc(sizeof(double) * (size_t)cnt);
      s_cap = cnt;
    }
    /* scores */
    double mx = -INFINITY;
    for (int64_t t = 0; t < cnt; ++t) {
      const int64_t r = jlo + t - a->kpos0;
      const double* kr;
      if (a->krot) {
        kr = a->krot + (r * hkv + g) * d;
      } else if (a->k64) {
        kr = a->k64 + (r * hkv + g) * d;
      } else {
        const uint16_t* ksrc = a->k + (r * hkv + g) * d;
        for (int32_t c = 0; c < d; ++c) kw[c] = widen_bf16(ksrc[c]);
        kr = kw;
      }
      double dot = 0.0;
      for (int32_t c = 0; c < d; ++c) dot += qv[c] * kr[c];
      s[t] = dot * cfg->scale;
      if (s[t] > mx) mx = s[t];
    }
    /* softmax-weighted sum of values */
    for (int32_t c = 0; c < d; ++c) acc[c] = 0.0;
    double lsum = 0.0;
    for (int64_t t = 0; t < cnt; ++t) {
      const double w = exp(s[t] - mx);
      lsum += w;
      const int64_t vr = ((jlo + t - a->kpos0) * hkv + g) * d;
      if (a->v64) {
        for (int32_t c = 0; c < d; ++c) acc[c] += w * a->v64[vr + c];
      } else {
        for (int32_t c = 0; c < d; ++c) acc[c] += w * widen_bf16(a->v[vr + c]);
      }
    }
    double* o = a->out + (n * hq + h) * d;
    if (a->normalise) {
      for (int32_t c = 0; c < d; ++c) o[c] = cnt ? acc[c] / lsum : 0.0;
    } else {
      for (int32_t c = 0; c < d; ++c) o[c] = acc[c];
      a->m[n * hq + h] = mx;
      a->l[n * hq + h] = lsum;
    }
  }
  free(qv);
  free(kw);
  free(acc);
  free(s);
}

static int check_cfg(const gqa_oracle_cfg* cfg) {
  if (!cfg || cfg->hq <= 0 || cfg->hkv <= 0 || cfg->d <= 0) return 0;
  if (cfg->hq % cfg->hkv != 0 || cfg->d % 2 != 0 || cfg->window < 0) return 0;
  return 1;
}

static int run(const gqa_oracle_cfg* cfg, const uint16_t* q,
               const int64_t* qpos, int64_t nq, const uint16_t* k,
               const uint16_t* v, const double* k64, const double* v64,
               int64_t kpos0, int64_t nk, int64_t jlo, int64_t jhi,
               int32_t normalise, double* out, double* m, double* l,
               int32_t nthreads) {
  if (!check_cfg(cfg) || nq < 0 || nk < 0 || (nq > 0 && (!q || !qpos || !out)))
    return GQA_ORACLE_EARG;
  if (!normalise && nq > 0 && (!m || !l)) return GQA_ORACLE_EARG;
  for (int64_t n = 0; n < nq; ++n) {
    const int64_t i = qpos[n];
    if (i < 0) return GQA_ORACLE_ERANGE;
    int64_t lo = visible_lo(cfg, i), hi = i + 1;
    if (lo < jlo) lo = jlo;
    if (hi > jhi) hi = jhi;
    if (hi > lo && (lo < kpos0 || hi > kpos0 + nk)) return GQA_ORACLE_ERANGE;
  }
  if (nq == 0) return GQA_ORACLE_OK;
  if (nk > 0 && (!(k || k64) || !(v || v64))) return GQA_ORACLE_EARG;

  attend_ctx a;
  memset(&a, 0, sizeof a);
  a.cfg = cfg;
  a.q = q;
  a.qpos = qpos;
  a.k = k;
  a.v = v;
  a.k64 = k64;
  a.v64 = v64;
  a.kpos0 = kpos0;
  a.nk = nk;
  a.jlo = jlo;
  a.jhi = jhi;
  a.normalise = normalise;
  a.out = out;
  a.m = m;
  a.l = l;
  double* krot = NULL;
  if (cfg->rope && nk > 0) {
    krot = (double*)malloc(sizeof(double) * (size_t)(nk * cfg->hkv * cfg->d));
    if (!krot) return GQA_ORACLE_EARG;
    a.krot = krot;
    rot_ctx rc = {&a};
    parallel_for(nk, nthreads, rotate_keys, &rc);
  }
  parallel_for(nq * cfg->hq, nthreads, attend_rows, &a);
  free(krot);
  return GQA_ORACLE_OK;
}

int gqa_oracle_attend(const gqa_oracle_cfg* cfg, const uint16_t* q,
                      const int64_t* qpos, int64_t nq, const uint16_t* k,
                      const uint16_t* v, int64_t kpos0, int64_t nk,
                      double* out, int32_t nthreads) {
  return run(cfg, q, qpos, nq, k, v, NULL, NULL, kpos0, nk, INT64_MIN,
             INT64_MAX, 1, out, NULL, NULL, nthreads);
}

int gqa_oracle_attend_kv64(const gqa_oracle_cfg* cfg, const uint16_t* q,
                           const int64_t* qpos, int64_t nq, const double* k,
                           const double* v, int64_t kpos0, int64_t nk,
                           double* out, int32_t nthreads) {
  return run(cfg, q, qpos, nq, NULL, NULL, k, v, kpos0, nk, INT64_MIN,
             INT64_MAX, 1, out, NULL, NULL, nthreads);
}

int gqa_oracle_partial(const gqa_oracle_cfg* cfg, const uint16_t* q,
                       const int64_t* qpos, int64_t nq, const uint16_t* k,
                       const uint16_t* v, int64_t kpos0, int64_t nk,
                       int64_t jlo, int64_t jhi, double* m, double* l,
                       double* o, int32_t nthreads) {
  return run(cfg, q, qpos, nq, k, v, NULL, NULL, kpos0, nk, jlo, jhi, 0, o, m,
             l, nthreads);
}
