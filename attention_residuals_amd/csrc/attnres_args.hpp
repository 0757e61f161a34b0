// attnres_args.hpp -- kernel argument blocks, shared by the kernels and the host dispatcher.
#pragma once

#include <stdint.h>

namespace attnres {

constexpr int kMaxSources = 64;

// Finaliser workgroups: 64 columns x 16 row phases (multi- and selected-query reads); 16 columns x
// 64 row phases (single-query read: more workgroups over its wider binned rows).
constexpr int kFinCols = 64;
constexpr int kFinPhases = 16;
constexpr int kFinRowsCols = 16;
constexpr int kFinRowsPhases = 64;

// Counter words of a forward or backward workspace (uint32 indices, each in its own 128-byte
// line). They are zero when a kernel starts and are returned to zero by the same call (the
// forward's last workgroup, the backward's finaliser), so a workspace is zeroed once when it is
// allocated and then serves any number of calls.
constexpr int kCtrTicket = 0;    // next batch handed out by ticket
constexpr int kCtrArrive = 32;   // forward: workgroups that have taken their last ticket
constexpr int kCtrIdFlag = 48;   // selected-query forward: set to 1 when an id outside [0, E)
                                 // was read (sticky: never cleared by a kernel)
constexpr int kCtrWords = 64;    // 256 bytes

// Exact accumulation of the backward's per-token gradient contributions (token-resident kernel):
// each FP32 contribution c is split into a multiple of 2^-20 (bin A) and a multiple of 2^-53
// (bin B, the remainder rounded, |.| <= 2^-21), and each bin is summed in FP64. Every partial sum
// of bin A stays a multiple of 2^-20 below 2^33 in magnitude and every partial sum of bin B a
// multiple of 2^-53 below 1 (for fewer than 2^21 tokens), so both sums are exact and their values
// do not depend on which workgroup summed which tokens, or in which order.
constexpr double kBinMagicA = 6442450944.0;  // 1.5 * 2^32: (c + M) - M rounds c to 2^-20
constexpr double kBinMagicB = 0.75;          // 1.5 * 2^-1: rounds to 2^-53

struct FwdArgs {
  const void* src[kMaxSources];  // base of source s ([N, D] rows, row_stride elements apart)
  int64_t row_stride;
  int64_t N;
  int S, D, R, lo;               // lo = D - R: first column of the key slice
  float eps, scale, inv_R, inv_D;
  const void* query;             // [R]
  const void* norm_w;            // [R] or nullptr
  const void* out_w;             // [D] or nullptr
  void* y;                       // [N, D] contiguous
  float* lse;                    // [N]
  float* o_rstd;                 // [N] or nullptr
  float* o32;                    // [N, D] or nullptr
  uint32_t* ticket;              // counter words (kCtr*; nullptr: static split)
  int64_t tpt;                   // tokens per ticket (batch size of the dynamic schedule)
  int out_norm;
};

// Backward token schedule: batches of tpt consecutive tokens, nbatch = ceil(N / tpt). Head
// batches [0, hb_end): workgroup g takes g, g + P, g + 2P, ... (P = gridDim.x). Tail batches
// [hb_end, nbatch): handed out by the ticket counter as workgroups finish. The token-resident
// kernel sums every token's q/w gradient into exact bins (kBinMagic*), so it writes one partial
// row per workgroup whatever tokens it ran (hb_end = P: only each workgroup's first batch is
// fixed). The streaming kernel sums in FP32 and writes one row per fixed token set: row g for its
// head batches and row P + (b - hb_end) for tail batch b.
struct BwdArgs {
  const void* src[kMaxSources];
  void* dsrc[kMaxSources];
  int64_t row_stride, drow_stride, dout_stride;
  int64_t N;
  int S, D, R, lo;
  float eps, scale, inv_R, inv_D;
  const void* query;
  const void* norm_w;
  const void* out_w;
  const float* lse;
  const float* o_rstd;
  const float* o32;
  const void* dout;
  void* part;                    // partial rows: token-resident [P][2][wc] FP64 (bins A, B),
                                 //   streaming [rows][wc] FP32; du at absolute columns
                                 //   [lo, D), dow at [D, 2D)
  int64_t wc;                    // columns of a partial row (D, or 2D with dow)
  int64_t tpt;                   // tokens per batch
  int64_t nbatch;                // ceil(N / tpt)
  int64_t hb_end;                // first tail batch
  uint32_t* ctr;                 // counter words (kCtr*)
  int out_norm;
};

// Finaliser of the single-query backward: sums every column's partial rows in a fixed order in
// FP64 and writes dq = du * w (du without w), dw = du * q and dow; zeroes the ticket counter.
struct FinRowsArgs {
  const void* part;              // as BwdArgs::part
  int64_t wc;
  int rows, binned;              // binned: [rows][2][wc] FP64, else [rows][wc] FP32
  int lo, D, R, cols;            // cols = R (+ D with dow): column c < R is du at lo + c, else
                                 //   dow at c - R
  const void* query;
  const void* norm_w;            // nullptr: dq = du and no dw
  void* dq;
  void* dw;
  void* dow;
  uint32_t* ctr;
};

struct FinArgs {
  const float* part_du;          // [P, R]
  const float* part_dow;         // [P, D] or nullptr
  int P, R, D, cols;             // cols = R (+ D when dow is wanted)
  const void* query;
  const void* norm_w;            // nullptr: dq = du and no dw
  void* dq;
  void* dw;
  void* dow;
};

// Multi-query read: queries per launch group (the largest instantiated MQ).
constexpr int kMaxGroupQueries = 4;

// Selected-query read: per-token queries bank[ids[n * K + m0 + m]] (m0 = the group's first
// query slot); ids outside [0, E) read a zero query and drop their bank gradient.
struct SelArgs {
  const void* bank;              // [E, R]
  const int64_t* ids;            // [N, K]
  int E, K, m0;
  int first;                     // backward: the first query group (its partial rows start at 0)
  int lds_bank;                  // backward: the partial bank rows live in LDS
  uint32_t* id_flag;             // forward: word set to 1 on an id outside [0, E), or null
};

struct MultiFwdArgs {
  const void* src[kMaxSources];
  int64_t row_stride;
  int64_t N;
  int S, D, R, lo, M;            // M <= MQ: queries of this group
  float eps, scale, inv_R;
  const void* query;             // [M, R] rows of this group (row stride R)
  void* y;                       // output of query 0 of the group, token 0
  int64_t y_sm, y_sn;            // element strides between queries / tokens
  float* lse;
  int64_t l_sm, l_sn;
  uint32_t* ticket;              // dynamic token counter, zero at launch (nullptr: static split)
  int64_t tpt;                   // tokens per ticket
  SelArgs sel;                   // selected-query kernels only
};

// Multi-query forward through matrix cores (all M <= 16 queries of a call in one pass; bf16).
struct MfmaFwdArgs {
  const void* src[kMaxSources];
  int64_t row_stride;
  int64_t N;
  int S, D, R, lo, M;
  float eps, scale, inv_R;
  const void* query;             // [M, R]
  void* y;                       // output of query 0, token 0
  int64_t y_sm, y_sn;            // element strides between queries / tokens
  float* lse;
  int64_t l_sm, l_sn;
  const int64_t* ids;            // selected-query read: [N, M] bank rows per token (query = bank)
  int E;                         //   bank rows; ids outside [0, E) read a zero query
  uint32_t* id_flag;             //   word set to 1 when such an id is read, or null
  uint32_t* ticket;              // token batch counter (zeroed before the launch), or null: static
  int64_t tpt;                   //   tokens per ticket
};

// Multi-query backward through matrix cores (all M <= 16 queries in one pass; bf16).
struct MfmaBwdArgs {
  const void* src[kMaxSources];
  void* dsrc[kMaxSources];
  int64_t row_stride, drow_stride;
  int64_t N;
  int S, D, R, lo, M;
  float eps, scale, inv_R;
  const void* query;             // [M, R]
  const float* lse;              // query m, token n at m * l_sm + n * l_sn
  int64_t l_sm, l_sn;
  const void* dout;              // dY rows: query m, token n at (m * g_sm + n * g_sn) elements
  int64_t g_sm, g_sn;
  float* coef;                   // [N][16][16] a_{m,s} per token when the dq kernel forms dq
                                 //   (selected read: summed per bank row, rows e < E)
  float* part;                   // [grid][M * R] dq partial rows when the kernel sums dq itself
  const int64_t* ids;            // selected read: [N, M] bank rows of the slots (query = bank)
  int E;                         //   bank rows (<= 16); ids outside [0, E) read a zero query
};

// Its dq kernel: partial rows [ranges][M * R] over static token ranges of tpr tokens.
struct MfmaDqArgs {
  const void* src[kMaxSources];
  int64_t row_stride;
  int64_t N;
  int S, D, R, lo, M;
  int chunk0;                    // first 16-byte chunk of the key slice (lo / 8)
  int64_t tpr;                   // tokens per range
  const float* coef;             // [N][16][16]
  float* part;                   // [ranges][M * R]
};

// Streaming probe (measurement aid): n_in input and n_out output streams of n_rows rows of
// row_chunks 16-byte chunks each.
constexpr int kProbeMaxStreams = 128;
struct ProbeArgs {
  const void* in[kProbeMaxStreams];
  void* out[kProbeMaxStreams];
  int n_in, n_out;
  int64_t n_rows, row_chunks;
};

struct MultiBwdArgs {
  const void* src[kMaxSources];
  void* dsrc[kMaxSources];
  int64_t row_stride, drow_stride;
  int64_t N;
  int S, D, R, lo, M;
  float eps, scale, inv_R;
  const void* query;             // [M, R]
  const float* lse;              // of query 0 of the group
  int64_t l_sm, l_sn;
  const void* dout;              // dY of query 0 of the group, token 0
  int64_t g_sm, g_sn;
  float* part;                   // [gridDim.x, Mtot * R] partial du rows; this group's columns
  int64_t part_stride;           //   start at part, row stride part_stride floats
                                 // (selected-query: [gridDim.x, E * R] partial bank rows)
  uint32_t* ticket;
  int64_t tpt;
  SelArgs sel;
};

}  // namespace attnres
