/*
 * gqa_oracle.h -- plain fp64 CPU oracle for grouped-query attention with a
 * hybrid local (sliding-window, RoPE) / global (full causal, no RoPE) layout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no source, header, table or
 * helper with the HIP library.
 *
 * What it computes (page "Tomas Koutsky explains how Meta fits Muse Glimmer
 * into 24 GB", runtimewire.com, sections "Narrow cache" and "Long context
 * still costs compute"; page "Deep dive into Muse Glimmer", shishifenxi.com,
 * section 01): for a query token at position i and query head h, attention
 * over the keys j of KV head g(h) = floor(h / (Hq/Hkv)) with
 *   global layers: 0 <= j <= i                       (full causal, no RoPE)
 *   local layers:  max(0, i-W+1) <= j <= i           (window of W incl. self,
 *                                                     RoPE on q and k)
 *   s_j = <R_i q, R_j k_j> * scale,  o = sum_j softmax(s)_j v_j.
 * Inputs are bf16 bit patterns, widened exactly to double; all arithmetic is
 * in double precision.  The oracle reads a logical, position-indexed K/V
 * stream and knows nothing about how a cache stores it.
 */
#ifndef GQA_ORACLE_H
#define GQA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gqa_oracle_cfg {
  int32_t hq;       /* query heads                                  */
  int32_t hkv;      /* key/value heads, hq % hkv == 0               */
  int32_t d;        /* head dimension, even                         */
  int32_t window;   /* 0: full causal; >0: sliding window incl. self */
  int32_t rope;     /* 1: rotate q and k by absolute position       */
  int32_t pad_;
  double theta;     /* RoPE base                                    */
  double scale;     /* softmax scale, e.g. 1/sqrt(d)                */
} gqa_oracle_cfg;

/* Error codes. */
#define GQA_ORACLE_OK 0
#define GQA_ORACLE_EARG (-1)
#define GQA_ORACLE_ERANGE (-2) /* a needed key lies outside the stream */

/* Rotate one head vector x[d] (bf16 values already widened to double) by
 * position t: pairs (c, c + d/2), angle t * theta^(-c/(d/2)).  out may
 * alias x. */
void gqa_oracle_rope(const double* x, int32_t d, double t, double theta,
                     double* out);

/* Full attention.
 *   q    [nq][hq][d]  bf16 bits, query n sits at position qpos[n]
 *   k, v [nk][hkv][d] bf16 bits, row r holds the token at position kpos0 + r
 *   out  [nq][hq][d]  double
 * Returns GQA_ORACLE_ERANGE when a query needs a key outside
 * [kpos0, kpos0 + nk). */
int gqa_oracle_attend(const gqa_oracle_cfg* cfg, const uint16_t* q,
                      const int64_t* qpos, int64_t nq, const uint16_t* k,
                      const uint16_t* v, int64_t kpos0, int64_t nk,
                      double* out, int32_t nthreads);

/* The same attention over keys and values given as exact doubles instead of
 * bf16 bits: k, v [nk][hkv][d] (e.g. a quantised cache's dequantised
 * values).  Everything else as gqa_oracle_attend. */
int gqa_oracle_attend_kv64(const gqa_oracle_cfg* cfg, const uint16_t* q,
                           const int64_t* qpos, int64_t nq, const double* k,
                           const double* v, int64_t kpos0, int64_t nk,
                           double* out, int32_t nthreads);

/* The same sums restricted to keys with position in [jlo, jhi) (intersected
 * with each query's visible set), left unnormalised:
 *   m[n][h] = max s_j (or -inf when no key is visible),
 *   l[n][h] = sum exp(s_j - m),  o[n][h][:] = sum exp(s_j - m) v_j. */
int gqa_oracle_partial(const gqa_oracle_cfg* cfg, const uint16_t* q,
                       const int64_t* qpos, int64_t nq, const uint16_t* k,
                       const uint16_t* v, int64_t kpos0, int64_t nk,
                       int64_t jlo, int64_t jhi, double* m, double* l,
                       double* o, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
