/*
 * attnres_oracle_multi.c -- plain FP64 CPU oracle for the multi-query AttnRes read, forward and
 * backward.
 *
 * TEST INFRASTRUCTURE, not product code: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares nothing with the GPU library.
 *
 * "Fast Attention Residuals" PyPI page, section "Multi-query AttnRes": M learned queries read the
 * same sources; each query has its own routing weights over the sources and its own full-width
 * output. Per query, the steps are those of the page's "Equation" section in its notation
 * (t_s, r_s, k_s, score_s, p_s, output); the keys t_s / r_s are the same for every query. The
 * backward is reverse-mode differentiation of those steps in reverse order, with the gradients of
 * the shared sources summed over the queries. Only tokens run in parallel (they are independent);
 * per-thread partial sums of dq are added in thread order.
 *
 * Reading of what the page leaves open: the multi-query read is the page's operator as written,
 * with neither a key-norm weight nor an output norm.
 */
#include "attnres_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double mload(const void* base, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
  if (dtype == ORACLE_F64) return ((const double*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;  /* bfloat16 = high half of f32 */
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef struct {
  double *t, *k, *dk;       /* [S*R]: slices, normalised keys, key gradients (summed over m) */
  double *r;                /* [S] */
  double *score, *p, *dp;   /* [M*S] */
  double *o, *dyv;          /* [D] */
  double *dq;               /* [M*R] per-thread partial sums */
} mwork;

static void mwork_free(mwork* w) {
  free(w->t); free(w->k); free(w->dk); free(w->r); free(w->score); free(w->p); free(w->dp);
  free(w->o); free(w->dyv); free(w->dq);
}

static int mwork_alloc(mwork* w, int S, int D, int R, int M) {
  memset(w, 0, sizeof *w);
  const size_t sr = (size_t)S * R, ms = (size_t)M * S;
  w->t = calloc(sr, sizeof(double)); w->k = calloc(sr, sizeof(double));
  w->dk = calloc(sr, sizeof(double)); w->r = calloc(S, sizeof(double));
  w->score = calloc(ms, sizeof(double)); w->p = calloc(ms, sizeof(double));
  w->dp = calloc(ms, sizeof(double)); w->o = calloc(D, sizeof(double));
  w->dyv = calloc(D, sizeof(double)); w->dq = calloc((size_t)M * R, sizeof(double));
  if (!w->t || !w->k || !w->dk || !w->r || !w->score || !w->p || !w->dp || !w->o || !w->dyv ||
      !w->dq) {
    mwork_free(w);
    return -1;
  }
  return 0;
}

static double mvalue(const attnres_oracle_multi_problem* P, int s, int64_t n, int i) {
  return mload(P->values[s], P->dtype, n * (int64_t)P->D + i);
}

static void multi_token(const attnres_oracle_multi_problem* P, int64_t n, int64_t row, int64_t T,
                        attnres_oracle_multi_rows* out, mwork* w) {
  const int S = P->S, D = P->D, R = P->R, M = P->M, dt = P->dtype;
  const int off = D - R;

  /* keys, shared by every query: t_s = v_s[..., D-R:D], r_s, k_s = t_s / r_s */
  for (int s = 0; s < S; ++s) {
    double* t = w->t + (size_t)s * R;
    double* k = w->k + (size_t)s * R;
    for (int j = 0; j < R; ++j) t[j] = mvalue(P, s, n, off + j);
    double sumsq = 0.0;
    for (int j = 0; j < R; ++j) sumsq += t[j] * t[j];
    w->r[s] = sqrt(sumsq / R + P->eps);
    for (int j = 0; j < R; ++j) k[j] = t[j] / w->r[s];
  }
  for (int m = 0; m < M; ++m) {
    double* score = w->score + (size_t)m * S;
    double* p = w->p + (size_t)m * S;
    /* score_{m,s} = scale * dot(k_s, query_m) */
    for (int s = 0; s < S; ++s) {
      const double* k = w->k + (size_t)s * R;
      double dot = 0.0;
      for (int j = 0; j < R; ++j) dot += k[j] * mload(P->queries, dt, (int64_t)m * R + j);
      score[s] = P->scale * dot;
    }
    /* p_m = softmax over sources, lse_m */
    double mx = score[0];
    for (int s = 1; s < S; ++s) if (score[s] > mx) mx = score[s];
    double l = 0.0;
    for (int s = 0; s < S; ++s) l += exp(score[s] - mx);
    for (int s = 0; s < S; ++s) p[s] = exp(score[s] - mx) / l;
    /* output_m = sum_s p_{m,s} v_s */
    for (int i = 0; i < D; ++i) {
      double acc = 0.0;
      for (int s = 0; s < S; ++s) acc += p[s] * mvalue(P, s, n, i);
      w->o[i] = acc;
    }
    if (out && out->y)
      for (int i = 0; i < D; ++i) out->y[((size_t)m * T + row) * D + i] = w->o[i];
    if (out && out->lse) out->lse[(size_t)m * T + row] = mx + log(l);
  }
  if (!P->dout) return;

  /* ---- backward ---- */
  double* dv = out ? out->dvalues : NULL;
  if (dv)
    for (int s = 0; s < S; ++s)
      for (int i = 0; i < D; ++i) dv[((size_t)s * T + row) * D + i] = 0.0;
  for (int j = 0; j < S * R; ++j) w->dk[j] = 0.0;
  for (int m = 0; m < M; ++m) {
    const double* p = w->p + (size_t)m * S;
    double* dp = w->dp + (size_t)m * S;
    for (int i = 0; i < D; ++i)
      w->dyv[i] = mload(P->dout, dt, ((int64_t)m * P->N + n) * D + i);
    /* output_m = sum_s p v_s  ->  dp_{m,s} = <dY_m, v_s>, dv_s += p_{m,s} dY_m */
    for (int s = 0; s < S; ++s) {
      double acc = 0.0;
      for (int i = 0; i < D; ++i) acc += w->dyv[i] * mvalue(P, s, n, i);
      dp[s] = acc;
      if (dv)
        for (int i = 0; i < D; ++i) dv[((size_t)s * T + row) * D + i] += p[s] * w->dyv[i];
    }
    /* p_m = softmax(score_m)  ->  dscore = p (dp - sum_r p_r dp_r) */
    double bar = 0.0;
    for (int s = 0; s < S; ++s) bar += p[s] * dp[s];
    for (int s = 0; s < S; ++s) {
      const double dscore = p[s] * (dp[s] - bar);
      const double* k = w->k + (size_t)s * R;
      double* dk = w->dk + (size_t)s * R;
      /* score = scale <k_s, q_m>  ->  dk_s += scale dscore q_m, dq_m += scale dscore k_s */
      for (int j = 0; j < R; ++j) {
        dk[j] += P->scale * dscore * mload(P->queries, dt, (int64_t)m * R + j);
        w->dq[(size_t)m * R + j] += P->scale * dscore * k[j];
      }
    }
  }
  /* k = t / r, r = sqrt(sum(t^2)/R + eps)  ->  dt_j = dk_j / r - t_j <dk, t> / (R r^3) */
  if (dv)
    for (int s = 0; s < S; ++s) {
      const double* t = w->t + (size_t)s * R;
      const double* dk = w->dk + (size_t)s * R;
      double dkt = 0.0;
      for (int j = 0; j < R; ++j) dkt += dk[j] * t[j];
      const double r = w->r[s];
      for (int j = 0; j < R; ++j)
        dv[((size_t)s * T + row) * D + off + j] += dk[j] / r - t[j] * dkt / (R * r * r * r);
    }
}

int attnres_oracle_multi_run(const attnres_oracle_multi_problem* P, const int64_t* tokens,
                             int64_t T, attnres_oracle_multi_rows* rows, double* dq,
                             int threads) {
  if (!P || P->S < 1 || P->D < 1 || P->R < 1 || P->R > P->D || P->N < 0 || P->M < 1) return -1;
  if (P->dtype != ORACLE_F32 && P->dtype != ORACLE_BF16 && P->dtype != ORACLE_F64) return -2;
  if (!P->values || !P->queries) return -3;
  for (int s = 0; s < P->S; ++s) if (!P->values[s]) return -3;
  if (!tokens) T = P->N;
  if (T < 0) return -4;
  if (tokens)
    for (int64_t t = 0; t < T; ++t) if (tokens[t] < 0 || tokens[t] >= P->N) return -5;
  if ((dq || (rows && rows->dvalues)) && !P->dout) return -6;

  const int nth = attnres_oracle_threads(threads);
  mwork* ws = calloc((size_t)nth, sizeof(mwork));
  if (!ws) return -100;
  int bad = 0;
  for (int i = 0; i < nth; ++i) if (mwork_alloc(&ws[i], P->S, P->D, P->R, P->M)) bad = 1;
  if (bad) {
    for (int i = 0; i < nth; ++i) mwork_free(&ws[i]);
    free(ws);
    return -100;
  }
#ifdef _OPENMP
#pragma omp parallel num_threads(nth)
#endif
  {
#ifdef _OPENMP
    const int me = omp_get_thread_num();
    const int cnt = omp_get_num_threads();
#else
    const int me = 0, cnt = 1;
#endif
    const int64_t lo = T * me / cnt, hi = T * (me + 1) / cnt;
    for (int64_t row = lo; row < hi; ++row)
      multi_token(P, tokens ? tokens[row] : row, row, T, rows, &ws[me]);
  }
  if (dq) {
    const size_t mr = (size_t)P->M * P->R;
    for (size_t j = 0; j < mr; ++j) dq[j] = 0.0;
    for (int i = 0; i < nth; ++i)
      for (size_t j = 0; j < mr; ++j) dq[j] += ws[i].dq[j];
  }
  for (int i = 0; i < nth; ++i) mwork_free(&ws[i]);
  free(ws);
  return 0;
}

/* ---------------------------------------------------------------- selected-query read
 * "Fast Attention Residuals" PyPI page, section "Multi-query AttnRes" (per-token query selection):
 * token n reads the sources with the K queries bank[ids[n, k]]; everything else is the
 * multi-query read of that token. The bank's gradient sums, for every bank row e, the query
 * gradients of all (n, k) with ids[n, k] = e. This reuses the multi-query steps above, one token
 * at a time, with the token's own query list. */
int attnres_oracle_selected_run(const attnres_oracle_selected_problem* P, const int64_t* tokens,
                                int64_t T, attnres_oracle_multi_rows* rows, double* dbank,
                                int threads) {
  if (!P || P->S < 1 || P->D < 1 || P->R < 1 || P->R > P->D || P->N < 0 || P->K < 1 || P->E < 1)
    return -1;
  if (P->dtype != ORACLE_F32 && P->dtype != ORACLE_BF16 && P->dtype != ORACLE_F64) return -2;
  if (!P->values || !P->bank || !P->ids) return -3;
  for (int s = 0; s < P->S; ++s) if (!P->values[s]) return -3;
  if (!tokens) T = P->N;
  if (T < 0) return -4;
  if (tokens)
    for (int64_t t = 0; t < T; ++t) if (tokens[t] < 0 || tokens[t] >= P->N) return -5;
  for (int64_t i = 0; i < P->N * (int64_t)P->K; ++i)
    if (P->ids[i] < 0 || P->ids[i] >= P->E) return -9;
  if ((dbank || (rows && rows->dvalues)) && !P->dout) return -6;
  const int S = P->S, D = P->D, R = P->R, K = P->K;
  const int esz = P->dtype == ORACLE_F32 ? 4 : P->dtype == ORACLE_BF16 ? 2 : 8;
  const int nth = attnres_oracle_threads(threads);
  double* part = dbank ? calloc((size_t)nth * P->E * R, sizeof(double)) : NULL;
  if (dbank && !part) return -100;
  int bad = 0;
#ifdef _OPENMP
#pragma omp parallel num_threads(nth) reduction(| : bad)
#endif
  {
#ifdef _OPENMP
    const int me = omp_get_thread_num();
    const int cnt = omp_get_num_threads();
#else
    const int me = 0, cnt = 1;
#endif
    /* the token's own queries [K, R] (copied in storage format) and its dY rows [K, 1, D] */
    char* q = malloc((size_t)K * R * esz);
    char* g = P->dout ? malloc((size_t)K * D * esz) : NULL;
    double* dq = calloc((size_t)K * R, sizeof(double));
    double *y = NULL, *lse = NULL, *dv = NULL;
    if (rows && rows->y) y = malloc((size_t)K * D * sizeof(double));
    if (rows && rows->lse) lse = malloc((size_t)K * sizeof(double));
    if (rows && rows->dvalues) dv = malloc((size_t)S * D * sizeof(double));
    if (!q || (P->dout && !g) || !dq || (rows && rows->y && !y) || (rows && rows->lse && !lse) ||
        (rows && rows->dvalues && !dv))
      bad = 1;
    const int64_t lo = T * me / cnt, hi = T * (me + 1) / cnt;
    for (int64_t row = lo; row < hi && !bad; ++row) {
      const int64_t n = tokens ? tokens[row] : row;
      const void* src[64];
      for (int s = 0; s < S; ++s)
        src[s] = (const char*)P->values[s] + (size_t)n * D * esz;
      for (int k = 0; k < K; ++k) {
        memcpy(q + (size_t)k * R * esz, (const char*)P->bank + (size_t)P->ids[n * K + k] * R * esz,
               (size_t)R * esz);
        if (g)
          memcpy(g + (size_t)k * D * esz, (const char*)P->dout + ((size_t)n * K + k) * D * esz,
                 (size_t)D * esz);
      }
      /* one-token multi-query problem over this token's rows and queries */
      attnres_oracle_multi_problem mp = {S, D, R, K, 1, P->dtype, P->eps, P->scale,
                                         (const void* const*)src, q, g};
      attnres_oracle_multi_rows mr = {y, lse, dv};
      if (attnres_oracle_multi_run(&mp, NULL, 1, &mr, dbank ? dq : NULL, 1) != 0) {
        bad = 1;
        break;
      }
      if (rows && rows->y)
        for (int k = 0; k < K; ++k)
          memcpy(rows->y + ((size_t)row * K + k) * D, y + (size_t)k * D, (size_t)D * sizeof(double));
      if (rows && rows->lse)
        for (int k = 0; k < K; ++k) rows->lse[(size_t)row * K + k] = lse[k];
      if (rows && rows->dvalues)
        for (int s = 0; s < S; ++s)
          memcpy(rows->dvalues + ((size_t)s * T + row) * D, dv + (size_t)s * D,
                 (size_t)D * sizeof(double));
      if (dbank)
        for (int k = 0; k < K; ++k) {
          double* pe = part + ((size_t)me * P->E + P->ids[n * K + k]) * R;
          for (int j = 0; j < R; ++j) pe[j] += dq[(size_t)k * R + j];
        }
    }
    free(q); free(g); free(dq); free(y); free(lse); free(dv);
  }
  if (!bad && dbank) {
    const size_t er = (size_t)P->E * R;
    for (size_t j = 0; j < er; ++j) dbank[j] = 0.0;
    for (int i = 0; i < nth; ++i)
      for (size_t j = 0; j < er; ++j) dbank[j] += part[(size_t)i * er + j];
  }
  free(part);
  return bad ? -100 : 0;
}
