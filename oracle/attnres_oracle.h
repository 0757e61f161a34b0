/*
 * attnres_oracle.h -- plain FP64 CPU oracle for the Attention Residuals (AttnRes) read.
 *
 * TEST INFRASTRUCTURE. This library exists only to check the GPU library. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load or call it; the product path
 * never does. It shares no code, header, table or helper with the GPU library.
 *
 * What is computed (one token at a time, tokens independent):
 *   "Fast Attention Residuals" PyPI page, section "Equation": the key of source s is the final R
 *   coordinates t_s of that source's value row; r_s = sqrt(mean(t_s^2) + eps); k_s = t_s / r_s;
 *   score_s = scale * <k_s, q>; p = softmax over sources; output = sum_s p_s v_s.
 * Readings where the pages leave a step open (each listed in the repository's design notes):
 *   - optional key-norm weight w[R] multiplies the normalised key: k_s = (t_s / r_s) * w;
 *   - optional output RMSNorm ("[Perf] Parallelize AttnRes long-sequence reduction", FLA PR page,
 *     Summary): y = o * (mean_D(o^2) + eps)^(-1/2) * ow, ow optional; its inverse RMS is the saved
 *     per-row statistic o_rstd;
 *   - gradients are exact first-order derivatives; dq, dw, dow are sums over all tokens.
 */
#ifndef ATTNRES_ORACLE_H
#define ATTNRES_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats the oracle can read. Every element is converted exactly to double on load. */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

typedef struct {
  int32_t S;              /* number of ordered residual sources, >= 1 */
  int32_t D;              /* width of every value row, >= 1 */
  int32_t R;              /* routing rank: the key is the final R coordinates, 1 <= R <= D */
  int64_t N;              /* tokens per source */
  int32_t dtype;          /* ORACLE_F32 / ORACLE_BF16 / ORACLE_F64, for every input array */
  int32_t out_norm;       /* 1: apply the output RMSNorm after the mixture */
  double eps;             /* shared by the key norm and the output norm */
  double scale;           /* score multiplier */
  const void* const* values;  /* host array of S host pointers, each a contiguous [N, D] */
  const void* query;      /* [R] */
  const void* norm_w;     /* [R] or NULL (then w == 1) */
  const void* out_w;      /* [D] or NULL (then ow == 1); only meaningful with out_norm */
  const void* dout;       /* [N, D] upstream gradient of the output, or NULL (forward only) */
} attnres_oracle_problem;

/* Per-token outputs, all FP64 and optional (NULL = not wanted). For a run over a token list of
 * length T, row t of each array belongs to token tokens[t]. */
typedef struct {
  double* y;        /* [T, D] output */
  double* lse;      /* [T] log-sum-exp of the scores */
  double* o_rstd;   /* [T] inverse RMS of the mixture (only with out_norm) */
  double* p;        /* [T, S] routing weights */
  double* score;    /* [T, S] scores */
  double* dvalues;  /* [S, T, D] gradient of every source row */
} attnres_oracle_rows;

/* Runs forward (and backward if prob->dout != NULL) over tokens.
 *   tokens == NULL: all N tokens in order (T = N).
 *   tokens != NULL: the T listed tokens (each in [0, N)).
 * dq, dw, dow (each optional) receive the sums over the processed tokens; dw needs norm_w,
 * dow needs out_w and out_norm. threads <= 0 uses the OpenMP default. Returns 0 on success,
 * a negative code for an invalid argument, -100 when memory runs out. */
int attnres_oracle_run(const attnres_oracle_problem* prob, const int64_t* tokens, int64_t T,
                       attnres_oracle_rows* rows, double* dq, double* dw, double* dow,
                       int threads);

/* Multi-query read ("Fast Attention Residuals" PyPI page, section "Multi-query AttnRes"): M
 * queries read the same sources, each with its own routing weights and output. No key-norm
 * weight and no output norm (the page's operator as written). Layouts are query-major. */
typedef struct {
  int32_t S, D, R, M;     /* sources, width, routing rank, queries (M >= 1) */
  int64_t N;
  int32_t dtype;
  double eps, scale;
  const void* const* values;  /* host array of S pointers, each a contiguous [N, D] */
  const void* queries;    /* [M, R] */
  const void* dout;       /* [M, N, D] upstream gradients of the outputs, or NULL */
} attnres_oracle_multi_problem;

typedef struct {
  double* y;        /* [M, T, D] outputs */
  double* lse;      /* [M, T] */
  double* dvalues;  /* [S, T, D], summed over the queries */
} attnres_oracle_multi_rows;

/* Like attnres_oracle_run; dq (optional) is [M, R], summed over the processed tokens. */
int attnres_oracle_multi_run(const attnres_oracle_multi_problem* prob, const int64_t* tokens,
                             int64_t T, attnres_oracle_multi_rows* rows, double* dq,
                             int threads);

/* Selected-query read (same section: per-token query selection): token n reads with the K queries
 * bank[ids[n, k]]; outputs are token-major [T, K, D] and lse [T, K]; dbank [E, R] sums the query
 * gradients of every (n, k) by id. S <= 64. */
typedef struct {
  int32_t S, D, R, E, K;  /* sources, width, rank, bank rows, queries per token */
  int64_t N;
  int32_t dtype;
  double eps, scale;
  const void* const* values;  /* S pointers, each a contiguous [N, D] */
  const void* bank;       /* [E, R] */
  const int64_t* ids;     /* [N, K], each in [0, E) */
  const void* dout;       /* [N, K, D] or NULL */
} attnres_oracle_selected_problem;

/* rows->y is [T, K, D], rows->lse [T, K], rows->dvalues [S, T, D]; dbank (optional) [E, R]. */
int attnres_oracle_selected_run(const attnres_oracle_selected_problem* prob,
                                const int64_t* tokens, int64_t T, attnres_oracle_multi_rows* rows,
                                double* dbank, int threads);

/* Number of OpenMP threads a run with the given request would use (for reporting). */
int attnres_oracle_threads(int threads);

#ifdef __cplusplus
}
#endif
#endif
