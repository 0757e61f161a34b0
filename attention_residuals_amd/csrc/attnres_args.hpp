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

}  // namespace attnres
