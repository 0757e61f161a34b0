/*
 * attnres_oracle.c -- plain FP64 CPU oracle for the Attention Residuals (AttnRes) read,
 * forward and backward.
 *
 * TEST INFRASTRUCTURE, not product code: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares nothing with the GPU library.
 *
 * The forward follows the "Equation" section of the "Fast Attention Residuals" PyPI page step by
 * step, in its notation (t_s, r_s, k_s, score_s, p_s, output), one token at a time. The backward
 * is ordinary reverse-mode differentiation of exactly those steps, taken in reverse order
 * (the page's "Why use Fast-AttnRes" section: first-order gradients through the routing keys).
 * Nothing is fused, blocked or reordered beyond what the steps themselves state; the only
 * parallelism is over tokens, which the Equation section makes independent, and the per-thread
 * partial sums of dq/dw/dow are added in thread order.
 *
 * Readings of points the pages leave open (see attnres_oracle.h):
 *   norm weight w multiplies the normalised key; the output RMSNorm uses the call's eps and a
 *   mean over D; dq/dw/dow are sums over tokens.
 */
#include "attnres_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Reads element i of an input array in its storage format, exactly, as a double. */
static double load(const void* base, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
  if (dtype == ORACLE_F64) return ((const double*)base)[i];
  /* bfloat16: the stored 16 bits are the high half of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* v_s[n, i] */
static double value(const attnres_oracle_problem* P, int s, int64_t n, int i) {
  return load(P->values[s], P->dtype, n * (int64_t)P->D + i);
}

/* Per-thread working memory for one token. */
typedef struct {
  double *t, *k, *kn, *dk, *dkn;   /* [S*R] each: slice, key, normalised slice and their grads */
  double *r, *score, *p, *dp, *dscore;  /* [S] */
  double *o, *yhat, *dyhat, *dout_o;    /* [D] */
  double *dq, *dw, *dow;                /* per-thread partial sums */
} work;

static void work_free(work* w) {
  free(w->t); free(w->k); free(w->kn); free(w->dk); free(w->dkn);
  free(w->r); free(w->score); free(w->p); free(w->dp); free(w->dscore);
  free(w->o); free(w->yhat); free(w->dyhat); free(w->dout_o);
  free(w->dq); free(w->dw); free(w->dow);
}

static int work_alloc(work* w, int S, int D, int R) {
  memset(w, 0, sizeof *w);
  size_t sr = (size_t)S * R;
  w->t = calloc(sr, sizeof(double)); w->k = calloc(sr, sizeof(double));
  w->kn = calloc(sr, sizeof(double)); w->dk = calloc(sr, sizeof(double));
  w->dkn = calloc(sr, sizeof(double));
  w->r = calloc(S, sizeof(double)); w->score = calloc(S, sizeof(double));
  w->p = calloc(S, sizeof(double)); w->dp = calloc(S, sizeof(double));
  w->dscore = calloc(S, sizeof(double));
  w->o = calloc(D, sizeof(double)); w->yhat = calloc(D, sizeof(double));
  w->dyhat = calloc(D, sizeof(double)); w->dout_o = calloc(D, sizeof(double));
  w->dq = calloc(R, sizeof(double)); w->dw = calloc(R, sizeof(double));
  w->dow = calloc(D, sizeof(double));
  if (!w->t || !w->k || !w->kn || !w->dk || !w->dkn || !w->r || !w->score || !w->p || !w->dp ||
      !w->dscore || !w->o || !w->yhat || !w->dyhat || !w->dout_o || !w->dq || !w->dw || !w->dow) {
    work_free(w);
    return -1;
  }
  return 0;
}

/* Forward and backward of one token n; per-token outputs go to row `row` of `out`. */
static void one_token(const attnres_oracle_problem* P, int64_t n, int64_t row, int64_t T,
                      attnres_oracle_rows* out, work* w) {
  const int S = P->S, D = P->D, R = P->R, dt = P->dtype;
  const int off = D - R;  /* the key is the final R coordinates: v_s[D-R .. D-1] */

  /* ---- forward, Equation section ---- */
  for (int s = 0; s < S; ++s) {
    double* t = w->t + (size_t)s * R;
    double* kn = w->kn + (size_t)s * R;
    double* k = w->k + (size_t)s * R;
    /* t_s = v_s[..., D-R:D] */
    for (int j = 0; j < R; ++j) t[j] = value(P, s, n, off + j);
    /* r_s = sqrt(mean(t_s ** 2) + eps) */
    double sumsq = 0.0;
    for (int j = 0; j < R; ++j) sumsq += t[j] * t[j];
    w->r[s] = sqrt(sumsq / R + P->eps);
    /* k_s = t_s / r_s, then the optional key-norm weight */
    for (int j = 0; j < R; ++j) {
      kn[j] = t[j] / w->r[s];
      k[j] = kn[j] * (P->norm_w ? load(P->norm_w, dt, j) : 1.0);
    }
    /* score_s = scale * dot(k_s, query) */
    double dot = 0.0;
    for (int j = 0; j < R; ++j) dot += k[j] * load(P->query, dt, j);
    w->score[s] = P->scale * dot;
  }
  /* p = softmax(score) over sources, with its log-sum-exp */
  double m = w->score[0];
  for (int s = 1; s < S; ++s) if (w->score[s] > m) m = w->score[s];
  double l = 0.0;
  for (int s = 0; s < S; ++s) l += exp(w->score[s] - m);
  for (int s = 0; s < S; ++s) w->p[s] = exp(w->score[s] - m) / l;
  const double lse = m + log(l);
  /* output = sum_s p_s * v_s */
  for (int i = 0; i < D; ++i) {
    double acc = 0.0;
    for (int s = 0; s < S; ++s) acc += w->p[s] * value(P, s, n, i);
    w->o[i] = acc;
  }
  /* optional output RMSNorm: yhat = o / sqrt(mean(o^2) + eps), y = yhat * ow */
  double rho_o = 1.0;
  if (P->out_norm) {
    double sq = 0.0;
    for (int i = 0; i < D; ++i) sq += w->o[i] * w->o[i];
    rho_o = 1.0 / sqrt(sq / D + P->eps);
    for (int i = 0; i < D; ++i) w->yhat[i] = w->o[i] * rho_o;
  } else {
    for (int i = 0; i < D; ++i) w->yhat[i] = w->o[i];
  }

  if (out) {
    if (out->y)
      for (int i = 0; i < D; ++i)
        out->y[row * D + i] = w->yhat[i] * ((P->out_norm && P->out_w) ? load(P->out_w, dt, i) : 1.0);
    if (out->lse) out->lse[row] = lse;
    if (out->o_rstd) out->o_rstd[row] = rho_o;
    if (out->p) for (int s = 0; s < S; ++s) out->p[row * S + s] = w->p[s];
    if (out->score) for (int s = 0; s < S; ++s) out->score[row * S + s] = w->score[s];
  }
  if (!P->dout) return;

  /* ---- backward: the forward steps in reverse ---- */
  /* y = yhat * ow  ->  dyhat = dY * ow, dow += dY * yhat */
  for (int i = 0; i < D; ++i) {
    const double g = load(P->dout, dt, n * (int64_t)D + i);
    const double ow = (P->out_norm && P->out_w) ? load(P->out_w, dt, i) : 1.0;
    w->dyhat[i] = g * ow;
    if (P->out_norm && P->out_w) w->dow[i] += g * w->yhat[i];
  }
  /* yhat = o * rho_o, rho_o = (sum(o^2)/D + eps)^(-1/2), d rho_o / d o_i = -rho_o^3 o_i / D */
  if (P->out_norm) {
    double go = 0.0;
    for (int i = 0; i < D; ++i) go += w->dyhat[i] * w->o[i];
    for (int i = 0; i < D; ++i)
      w->dout_o[i] = rho_o * w->dyhat[i] - rho_o * rho_o * rho_o * go * w->o[i] / D;
  } else {
    for (int i = 0; i < D; ++i) w->dout_o[i] = w->dyhat[i];
  }
  /* output = sum_s p_s v_s  ->  dp_s = <d output, v_s>, dv_s += p_s * d output */
  for (int s = 0; s < S; ++s) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i) acc += w->dout_o[i] * value(P, s, n, i);
    w->dp[s] = acc;
  }
  double* dv = out ? out->dvalues : NULL;
  if (dv)
    for (int s = 0; s < S; ++s)
      for (int i = 0; i < D; ++i) dv[((size_t)s * T + row) * D + i] = w->p[s] * w->dout_o[i];
  /* p = softmax(score)  ->  dscore_s = p_s (dp_s - sum_r p_r dp_r) */
  double bar = 0.0;
  for (int s = 0; s < S; ++s) bar += w->p[s] * w->dp[s];
  for (int s = 0; s < S; ++s) w->dscore[s] = w->p[s] * (w->dp[s] - bar);
  for (int s = 0; s < S; ++s) {
    double* t = w->t + (size_t)s * R;
    double* kn = w->kn + (size_t)s * R;
    double* k = w->k + (size_t)s * R;
    double* dk = w->dk + (size_t)s * R;
    double* dkn = w->dkn + (size_t)s * R;
    /* score_s = scale * <k_s, q>  ->  dk = scale dscore q, dq += scale dscore k */
    for (int j = 0; j < R; ++j) {
      dk[j] = P->scale * w->dscore[s] * load(P->query, dt, j);
      w->dq[j] += P->scale * w->dscore[s] * k[j];
    }
    /* k = kn * w  ->  dkn = dk * w, dw += dk * kn */
    for (int j = 0; j < R; ++j) {
      const double wj = P->norm_w ? load(P->norm_w, dt, j) : 1.0;
      dkn[j] = dk[j] * wj;
      if (P->norm_w) w->dw[j] += dk[j] * kn[j];
    }
    /* kn = t / r, r = sqrt(sum(t^2)/R + eps), d r / d t_j = t_j / (R r)
     *   ->  dt_j = dkn_j / r - t_j * <dkn, t> / (R r^3) */
    double dknt = 0.0;
    for (int j = 0; j < R; ++j) dknt += dkn[j] * t[j];
    const double r = w->r[s];
    if (dv)
      for (int j = 0; j < R; ++j) {
        const double dtj = dkn[j] / r - t[j] * dknt / (R * r * r * r);
        dv[((size_t)s * T + row) * D + off + j] += dtj;
      }
  }
}

int attnres_oracle_threads(int threads) {
#ifdef _OPENMP
  return threads > 0 ? threads : omp_get_max_threads();
#else
  (void)threads;
  return 1;
#endif
}

int attnres_oracle_run(const attnres_oracle_problem* P, const int64_t* tokens, int64_t T,
                       attnres_oracle_rows* rows, double* dq, double* dw, double* dow,
                       int threads) {
  if (!P || P->S < 1 || P->D < 1 || P->R < 1 || P->R > P->D || P->N < 0) return -1;
  if (P->dtype != ORACLE_F32 && P->dtype != ORACLE_BF16 && P->dtype != ORACLE_F64) return -2;
  if (!P->values || !P->query) return -3;
  for (int s = 0; s < P->S; ++s) if (!P->values[s]) return -3;
  if (!tokens) T = P->N;
  if (T < 0) return -4;
  if (tokens)
    for (int64_t t = 0; t < T; ++t) if (tokens[t] < 0 || tokens[t] >= P->N) return -5;
  if ((dq || dw || dow) && !P->dout) return -6;
  if (dw && !P->norm_w) return -7;
  if (dow && !(P->out_w && P->out_norm)) return -8;
  if (rows && rows->dvalues && !P->dout) return -6;

  const int S = P->S, D = P->D, R = P->R;
  const int nth = attnres_oracle_threads(threads);
  work* ws = calloc((size_t)nth, sizeof(work));
  if (!ws) return -100;
  int bad = 0;
  for (int i = 0; i < nth; ++i) if (work_alloc(&ws[i], S, D, R)) bad = 1;
  if (bad) {
    for (int i = 0; i < nth; ++i) work_free(&ws[i]);
    free(ws);
    return -100;
  }

  /* contiguous static split of the token range: thread i takes a block, in order */
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
    for (int64_t row = lo; row < hi; ++row) {
      const int64_t n = tokens ? tokens[row] : row;
      one_token(P, n, row, T, rows, &ws[me]);
    }
  }

  /* per-thread partial sums, added in thread order */
  if (dq) for (int j = 0; j < R; ++j) dq[j] = 0.0;
  if (dw) for (int j = 0; j < R; ++j) dw[j] = 0.0;
  if (dow) for (int i = 0; i < D; ++i) dow[i] = 0.0;
  for (int i = 0; i < nth; ++i) {
    if (dq) for (int j = 0; j < R; ++j) dq[j] += ws[i].dq[j];
    if (dw) for (int j = 0; j < R; ++j) dw[j] += ws[i].dw[j];
    if (dow) for (int k = 0; k < D; ++k) dow[k] += ws[i].dow[k];
  }
  for (int i = 0; i < nth; ++i) work_free(&ws[i]);
  free(ws);
  return 0;
}
