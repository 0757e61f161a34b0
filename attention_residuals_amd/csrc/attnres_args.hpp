// attnres_args.hpp -- kernel argument blocks, shared by the kernels and the host dispatcher.
#pragma once

#include <stdint.h>

namespace attnres {

constexpr int kMaxSources = 64;

// Finaliser workgroup: 64 columns x 16 row phases.
constexpr int kFinCols = 64;
constexpr int kFinPhases = 16;

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
  uint32_t* ticket;              // dynamic token counter, zero at launch (nullptr: static split)
  int64_t tpt;                   // tokens per ticket (batch size of the dynamic schedule)
  int out_norm;
};

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
  float* part_du;                // [gridDim.x, R]
  float* part_dow;               // [gridDim.x, D] or nullptr
  uint32_t* ticket;              // dynamic token counter, zero at launch (nullptr: static split)
  int64_t tpt;                   // tokens per ticket (batch size of the dynamic schedule)
  int out_norm;
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
  uint32_t* ticket;              // token batch counter (zeroed before the launch), or null: static
  int64_t tpt;                   //   tokens per ticket
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
