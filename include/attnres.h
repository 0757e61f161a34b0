/*
 * attnres.h -- C ABI of the MI355X (gfx950) Attention Residuals (AttnRes) read library.
 *
 * The operation ("Fast Attention Residuals" PyPI page, section "Equation"): for every token n and
 * each of S ordered residual sources v_s[n, 0..D-1], the key is the final R coordinates
 * t_s = v_s[n, D-R..D-1]; r_s = sqrt(mean(t_s^2) + eps); k_s = (t_s / r_s) * w (w = optional
 * key-norm weight, 1 when absent); score_s = scale * <k_s, q>; p = softmax over the S sources;
 * o = sum_s p_s v_s. Tokens are independent; the output keeps width D. Optionally
 * ("[Perf] Parallelize AttnRes long-sequence reduction", FLA PR page, Summary) an output RMSNorm
 * follows: y = o * rho_o * ow with rho_o = (mean_D(o^2) + eps)^(-1/2) saved per row (o_rstd) for
 * the backward, ow optional. Without it y = o.
 * The backward (same PR page: dq/dw/dow reduced over the flattened token dimension through FP32
 * partial sums, merged in a fixed order) returns dvalues for every source row and the gradients
 * of q, w and ow summed over all N tokens. It recomputes the routing weights from the saved
 * per-row log-sum-exp.
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers of the current HIP device unless stated otherwise.
 *     The caller owns every buffer; the library never allocates, frees or synchronises.
 *   - Every kernel is enqueued on `stream` (a hipStream_t; NULL = the null stream). Calls return
 *     once the work is enqueued. They record no memset or copy node, so they can be captured
 *     into a HIP graph.
 *   - Storage dtype (values, query, weights, outputs and gradients) is the descriptor's dtype;
 *     all arithmetic is FP32; FP32 -> bfloat16 stores round to nearest even.
 *   - Errors: argument checks run before anything is enqueued; on failure nothing is launched
 *     or written and a nonzero status is returned. attnres_last_error() gives the calling
 *     thread's detail text. No exception or abort crosses this boundary.
 *   - Concurrency: calls on different streams may run concurrently as long as they share no
 *     output buffer and no workspace.
 */
#ifndef ATTNRES_H
#define ATTNRES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTNRES_OK = 0,
  ATTNRES_ERR_INVALID_ARG = 1,   /* a size, pointer or flag is out of contract */
  ATTNRES_ERR_UNSUPPORTED = 2,   /* within the math's domain but outside what is built */
  ATTNRES_ERR_ALIGNMENT = 3,     /* a pointer or row stride is not 16-byte aligned */
  ATTNRES_ERR_WORKSPACE = 4,     /* workspace missing or smaller than attnres_workspace_bytes */
  ATTNRES_ERR_HIP = 5            /* a HIP runtime call failed (text in attnres_last_error) */
} attnres_status;

typedef enum { ATTNRES_F32 = 0, ATTNRES_BF16 = 1 } attnres_dtype;

/* Problem descriptor, passed by pointer and validated on every call. */
typedef struct {
  int32_t S;               /* sources, 1 <= S <= 64 */
  int32_t D;               /* width; D % 8 == 0 (bf16) or D % 4 == 0 (f32); 8 <= D <= 16384 */
  int32_t R;               /* routing rank, 1 <= R <= D; key = final R coordinates */
  int32_t dtype;           /* attnres_dtype */
  int64_t N;               /* tokens, N >= 0. N == 0: nothing is read and the per-token arrays
                              may be NULL; the backward still writes zero dq/dw/dow */
  float eps;               /* inside both square roots; the pages' default is 2^-23 */
  float scale;             /* score multiplier; default 1 */
  int32_t has_norm_weight; /* key-norm weight w[R] present */
  int32_t out_norm;        /* output RMSNorm after the mixture */
  int32_t has_out_weight;  /* output-norm weight ow[D] present (requires out_norm) */
  int32_t deterministic;   /* Backward reductions. Tokens go out in batches through a
                              device-wide counter as workgroups finish in both modes (a static
                              split when N is below twice the workgroup count); y, lse and
                              dvalues are bitwise reproducible in both.
                              1: dq/dw/dow bitwise reproducible across calls. The token-resident
                              backward adds each batch's q/w gradient into exact FP64 bins (a
                              multiple of 2^-20 and a remainder rounded to 2^-53, each summed
                              exactly while per-batch contributions stay below 2^31 in magnitude,
                              a workgroup's 2^-20 bin below 2^33 and it bins fewer than 2^20
                              batches; data outside these bounds loses the guarantee), so the sums
                              do not depend on which workgroup took which batch; the streaming
                              backward gives each workgroup a fixed share and each counter batch
                              of the last quarter its own partial row.
                              0 (default): the same, except that the bf16 token-resident backward
                              keeps one FP32 running sum per workgroup (about 1.6% faster; when
                              accumulating into dvalues the binned kernel spills and runs ~13%
                              slower), so its dq/dw reproduce to FP32 rounding only.
                              The two modes may differ from each other in the last bits of
                              dq/dw/dow. Multi- and selected-query reads: their one-pass
                              matrix-core backward (three or more bf16 queries or slots, see
                              attnres_multi_bwd) always splits statically, bitwise reproducible;
                              their query-group kernels with 0 reproduce dq/dbank to FP32
                              rounding only, with 1 a static split, bitwise reproducible. */
  int32_t accumulate_dvalues; /* backward only. 0: dvalues are overwritten with this read's
                              gradient. 1: the gradient is added to the existing dvalues (read,
                              summed in FP32, rounded once to storage), so a source shared by
                              several reads (the embedding and writer outputs of Full / Block
                              schedules) collects all of them without a separate add pass. */
} attnres_desc;

/* S row blocks of shape [N, D]: either one packed [S, N, D] tensor or a list of S pointers.
 * Exactly one of `packed` / `list` is non-NULL.
 *   packed:     base of source 0; source s starts at packed + s * src_stride elements.
 *   list:       HOST array of S device pointers (read during the call only). A list may repeat a
 *               pointer when it describes inputs (a source read twice); for outputs every
 *               pointer must be distinct.
 *   row_stride: elements between token n and token n+1 inside a source (>= D); elements of a
 *               row are contiguous. */
typedef struct {
  void* packed;
  int64_t src_stride;
  void* const* list;
  int64_t row_stride;
} attnres_sources;

/* Number of FP32 elements of the saved mixture o32 that the forward must write for a later
 * backward: N*D when the backward streams the sources (output RMSNorm on, or S*D too large to
 * keep a token's rows on chip), else 0. */
attnres_status attnres_o32_elems(const attnres_desc* desc, size_t* elems);

/* Bytes of device workspace attnres_bwd needs on the CURRENT device: 256 bytes of counters, then
 * partial sums of the q/w/ow gradients, one row of D (2D with ow) columns per workgroup (exact
 * FP64 bins, 16 bytes a column, for the token-resident backward; FP32 per fixed token set for the
 * streaming one). The first 256 bytes must be ZERO before the first call that uses the buffer
 * (allocate it zero-filled); every call leaves them zero again when its finaliser completes, so
 * one buffer serves any number of later calls and graph replays. The rest needs no
 * initialisation. */
attnres_status attnres_workspace_bytes(const attnres_desc* desc, size_t* bytes);

/* Bytes of the optional forward workspace (a device-wide token counter); currently 256. */
attnres_status attnres_fwd_workspace_bytes(const attnres_desc* desc, size_t* bytes);

/* Forward.
 *   values   [S][N, D] sources (read).
 *   query    [R]; norm_w [R] iff has_norm_weight; out_w [D] iff has_out_weight.
 *   out      [N, D] contiguous output y (written).
 *   lse      [N] FP32 log-sum-exp of the scores (written; the backward's saved statistic).
 *   out_rstd [N] FP32 rho_o (written iff out_norm, else must be NULL).
 *   o32      [N, D] FP32 mixture o (written iff attnres_o32_elems > 0, else must be NULL).
 *   workspace, workspace_bytes: optional. With a 256-byte aligned buffer of at least
 *            attnres_fwd_workspace_bytes bytes (zero before its first use, like the backward's
 *            counters, and left zero by every call; not shared with a concurrent call),
 *            workgroups take tokens from a counter kept there as they finish. NULL with 0 bytes:
 *            a static token split. The outputs are bitwise identical either way.
 * All device pointers 16-byte aligned; row strides multiples of 16 bytes. */
attnres_status attnres_fwd(const attnres_desc* desc, const attnres_sources* values,
                           const void* query, const void* norm_w, const void* out_w,
                           void* out, float* lse, float* out_rstd, float* o32,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Backward, given the forward's inputs and saved statistics.
 *   dout            [N, D] upstream gradient dL/dy with row stride dout_row_stride (read).
 *   dvalues         [S][N, D] gradients of the sources (written; with accumulate_dvalues read
 *                   first and added to); must not alias values or each other.
 *   dq [R]          gradient of the query, summed over tokens (written).
 *   dw [R]          gradient of the key-norm weight (iff has_norm_weight, else NULL).
 *   dow [D]         gradient of the output-norm weight (iff has_out_weight, else NULL).
 *   workspace       at least attnres_workspace_bytes(desc) bytes, 256-byte aligned, first 256
 *                   bytes zero before its first use (see attnres_workspace_bytes); not shared
 *                   with any concurrent call.
 * Two kernel launches: the backward, then a finaliser that sums each column's partial rows in a
 * fixed order, writes dq, dw and dow and returns the workspace's counters to zero, so repeated
 * calls give bitwise-identical results with desc->deterministic = 1 (dq/dw/dow to FP32 rounding
 * with 0, every other output bitwise). */
attnres_status attnres_bwd(const attnres_desc* desc, const attnres_sources* values,
                           const void* query, const void* norm_w, const void* out_w,
                           const float* lse, const float* out_rstd, const float* o32,
                           const void* dout, int64_t dout_row_stride,
                           const attnres_sources* dvalues,
                           void* dq, void* dw, void* dow,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free backward, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. Arguments, results and
 * errors as attnres_bwd, without the workspace: it lives in a 64 MiB device array that the library
 * holds on every device it runs on until the process ends. Every call first zeroes the array's
 * counter words with a kernel on `stream`. ATTNRES_ERR_WORKSPACE: the call's partial rows do not
 * fit the array (the streaming backward first shrinks its counter-scheduled tail, down to a static
 * split). All calls on one device share the one array, so calls that overlap on a device (other
 * streams, other threads) race: the caller must order them. */
attnres_status attnres_bwd_noalloc(const attnres_desc* desc, const attnres_sources* values,
                                   const void* query, const void* norm_w, const void* out_w,
                                   const float* lse, const float* out_rstd, const float* o32,
                                   const void* dout, int64_t dout_row_stride,
                                   const attnres_sources* dvalues,
                                   void* dq, void* dw, void* dow, void* stream);

/* ---------------------------------------------------------------- multi-query read
 * "Fast Attention Residuals" PyPI page, section "Multi-query AttnRes": M queries q_m (1 <= M <= 16)
 * read the same S sources; each has its own routing weights
 * p_{m,s} = softmax_s(scale * <t_s / r_s, q_m>) and its own full-width output
 * y_m = sum_s p_{m,s} v_s (t_s, r_s as in the single-query read). The operator is the page's as
 * written: no key-norm weight and no output norm. The backward returns dvalues summed over the
 * queries and dq [M, R], each row summed over all tokens.
 * Token-resident only: a token's S rows must fit on chip (attnres_multi_*_workspace_bytes and the
 * entry points return ATTNRES_ERR_UNSUPPORTED otherwise; at D = 4096, bf16, S <= 24). The forward
 * of 3 <= M <= 16 bf16 queries over 2 <= S <= 16 sources with D <= 4096 runs in one pass on matrix
 * cores (tokens strided over the grid). With 5 <= M, D = 1024, 2048, 3072 or 4096, R and the row
 * stride multiples of 8, and queries, sources and y 16-byte aligned (y strides multiples of 8
 * elements), that pass runs in the backward's tile layout; otherwise, with 9 to 16 queries and the
 * optional forward workspace, tokens come from its counter (outputs are the same either way, bit
 * for bit). Other shapes run queries in groups of at most four, each group reading the sources
 * again. The backward of 3 <= M <= 16 bf16 queries over 2 <= S <= 16 sources with D = 1024, 2048,
 * 3072 or 4096, R and the row strides multiples of 8 and 16-byte aligned queries, runs in one pass
 * on matrix cores (dvalues written and rounded once; with S + M <= 16 the sources and dY rows share
 * one register tile (used from five queries on) and two tokens are in flight; a second pass over
 * the key slice forms dq unless M <= 4, or, in the shared tile, M <= 8 with the dq sums fitting the
 * workgroup's LDS beside the queries: M <= 6 at D = 4096), except M = 3 with S <= 12 accumulating
 * into dvalues, which is one launch of the query-group kernel; otherwise
 * backward groups after the first add into dvalues. ATTNRES_MULTI_MFMA=0 (read once) turns the
 * matrix-core kernels off.
 * Layout of y, dout [.., D] and lse: ATTNRES_QUERY_MAJOR = [M, N] rows (the page's default),
 * ATTNRES_TOKEN_MAJOR = [N, M] rows (the page's output_layout="token_major"). */
typedef enum { ATTNRES_QUERY_MAJOR = 0, ATTNRES_TOKEN_MAJOR = 1 } attnres_layout;

typedef struct {
  int32_t S, D, R;         /* as in attnres_desc */
  int32_t M;               /* queries, 1 <= M <= 16 */
  int32_t dtype;
  int64_t N;
  float eps, scale;
  int32_t layout;          /* attnres_layout of y, dout and lse */
  int32_t deterministic;   /* as in attnres_desc (backward) */
  int32_t accumulate_dvalues; /* as in attnres_desc (backward) */
} attnres_multi_desc;

/* Bytes of the optional forward workspace (a token counter): 256. */
attnres_status attnres_multi_fwd_workspace_bytes(const attnres_multi_desc* desc, size_t* bytes);

/* Bytes of the backward workspace (counter words, per-token coefficients and FP32 partial dq
 * rows), enough for either backward kernel. Its first 256 bytes must be zero when the workspace is
 * first used; the calls leave them zero. */
attnres_status attnres_multi_workspace_bytes(const attnres_multi_desc* desc, size_t* bytes);

/* Forward. queries [M, R] contiguous; y [M, N, D] or [N, M, D] contiguous (layout); lse [M, N] or
 * [N, M] FP32 (written). workspace / workspace_bytes: optional, as for attnres_fwd. */
attnres_status attnres_multi_fwd(const attnres_multi_desc* desc, const attnres_sources* values,
                                 const void* queries, void* y, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Backward. lse as written by the forward; dout like y (contiguous, same layout); dvalues as for
 * attnres_bwd (overwritten, or added to with accumulate_dvalues); dq [M, R] (written). */
attnres_status attnres_multi_bwd(const attnres_multi_desc* desc, const attnres_sources* values,
                                 const void* queries, const float* lse, const void* dout,
                                 const attnres_sources* dvalues, void* dq, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- selected-query read
 * Same section, per-token query selection: token n reads the sources with the K queries
 * bank[ids[n, k]] (1 <= K <= 16) of an [E, R] bank; outputs are token-major y [N, K, D] and lse
 * [N, K]. The backward returns dvalues (summed over the K reads) and dbank [E, R]: for every bank
 * row e, the sum of the query gradients of all (n, k) with ids[n, k] = e. ids are int64 on the
 * device; an id outside [0, E) reads a zero query and its bank gradient is dropped, and the
 * forward, when given its workspace, then sets the workspace's id flag (see
 * attnres_selected_ids_flag). Token-resident
 * with one or two chunks per thread (D <= 8192 bf16 / 4096 f32). The forward of 3 <= K <= 16 bf16
 * slots over 2 <= S <= 16 sources with D <= 4096 runs in one pass on matrix cores when the bank
 * (E + 1 rows of D bf16) fits in a workgroup's LDS (in the tile layout under the multi-query read's
 * conditions for it; else the optional forward workspace holds the token counter of 9 to 16 slots,
 * as in the multi-query read); otherwise slots run in groups of at most four. The backward runs
 * slots in groups of at most four (two with S > 10 or two chunks per thread); when that takes two
 * or more groups, or with 4 <= K and S + K <= 16, bf16 slots instead run in one pass on matrix
 * cores under the multi-query read's conditions when E <= 16 and the bank fits in a workgroup's
 * LDS (as E + 1 rows, and unless S + K <= 16 also as transposed groups of four: E <= 8 at
 * D = 4096), dbank formed by a second pass over the key slice; otherwise later groups add into
 * dvalues.
 * The bank gradient goes through per-workgroup FP32 partial rows of the whole bank (the workspace
 * is 256 + P * E * R * 4 bytes, P = backward workgroups, or the matrix-core backward's
 * coefficients and partial rows), so a large bank costs workspace and traffic; E * R * 4 must stay
 * below 2 GiB (else ATTNRES_ERR_UNSUPPORTED). */
typedef struct {
  int32_t S, D, R;
  int32_t E;               /* bank rows, >= 1 */
  int32_t K;               /* queries per token, 1 <= K <= 16 */
  int32_t dtype;
  int64_t N;
  float eps, scale;
  int32_t deterministic;   /* as in attnres_desc (backward) */
  int32_t accumulate_dvalues;
} attnres_selected_desc;

attnres_status attnres_selected_fwd_workspace_bytes(const attnres_selected_desc* desc,
                                                    size_t* bytes);
attnres_status attnres_selected_workspace_bytes(const attnres_selected_desc* desc, size_t* bytes);

/* Forward. bank [E, R]; ids [N, K] int64 (device); y [N, K, D] and lse [N, K] FP32 (written);
 * workspace optional as for attnres_fwd. With a workspace, the 32-bit word at byte offset 192 is
 * the id flag: any id outside [0, E) that the call reads sets it to 1 (an ordinary store from the
 * kernel). No kernel clears it: it stays set over later calls until the caller clears it
 * (attnres_selected_ids_flag with clear = 1, or a zeroed workspace). */
attnres_status attnres_selected_fwd(const attnres_selected_desc* desc,
                                    const attnres_sources* values, const void* bank,
                                    const int64_t* ids, void* y, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* The id flag of a selected-query forward workspace (device memory, workspace_bytes as given to
 * the forward): *flag = 1 if a forward that used this workspace met an id outside [0, E) since it
 * was last cleared, else 0. clear = 1 zeroes the flag afterwards. Runs on `stream` after the work
 * already queued there and waits for it (a device-to-host copy and a stream synchronisation), so
 * it is not for use under graph capture. ATTNRES_ERR_WORKSPACE for a NULL, short or misaligned
 * workspace; ATTNRES_ERR_HIP if the copy fails. */
attnres_status attnres_selected_ids_flag(const void* workspace, size_t workspace_bytes,
                                         int32_t clear, int32_t* flag, void* stream);

/* Backward. dout [N, K, D] (contiguous); dbank [E, R] (written). */
attnres_status attnres_selected_bwd(const attnres_selected_desc* desc,
                                    const attnres_sources* values, const void* bank,
                                    const int64_t* ids, const float* lse, const void* dout,
                                    const attnres_sources* dvalues, void* dbank, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- measurement aid
 * Not part of the AttnRes computation: streams n_rows rows of row_bytes bytes (a multiple of 16)
 * from each of the n_in input streams to each of the n_out output streams (1 .. 128 each; host
 * arrays of device pointers, rows contiguous, 16-byte aligned): output j (1 <= j < n_in) receives a
 * copy of input j, output 0 and outputs j >= n_in the bitwise XOR of all inputs. Outputs must not
 * overlap inputs
 * (ATTNRES_ERR_INVALID_ARG). Timed beside a read's kernels with the same streams (for example
 * S + 1 inputs and S outputs for the single-query backward), it gives the rate the device reaches
 * on that traffic pattern with no arithmetic: the practical ceiling the kernels are measured
 * against besides the 8 TB/s peak. Launch shape: chunks_per_thread (1, 2 or 4 16-byte chunks per
 * thread and step, their loads in flight together) and blocks_per_cu (1 .. 64 blocks of 256
 * threads per CU); callers try several and keep the fastest. Asynchronous on `stream`. */
attnres_status attnres_stream_probe(const void* const* in_rows, int32_t n_in,
                                    void* const* out_rows, int32_t n_out, int64_t n_rows,
                                    int64_t row_bytes, int32_t chunks_per_thread,
                                    int32_t blocks_per_cu, void* stream);

/* Static text for a status code. */
const char* attnres_status_str(attnres_status status);

/* Detail of the calling thread's most recent failure ("" if none). Valid until the thread's
 * next call into this library. */
const char* attnres_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ATTNRES_H */
