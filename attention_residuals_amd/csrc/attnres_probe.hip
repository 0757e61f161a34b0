// attnres_probe.hip -- streaming probe: the practical HBM ceiling of a read's traffic pattern.
//
// Not part of the AttnRes computation: a measurement aid. Each of n_rows rows is read from every
// input stream and written to every output stream, 16 bytes per thread and step, with no arithmetic
// beyond folding the inputs together (bitwise XOR, so every load is used): output j (1 <= j < n_in)
// copies input j, output 0 and outputs j >= n_in receive the fold. The streams go in unrolled
// groups of eight (loads of a group in flight together). Timing it beside a read's kernels, with
// the same streams and rows, gives the rate this device reaches on that access pattern with
// nothing else to do. Each thread handles cpt (1, 2 or 4) chunks per step, all their loads of a
// group in flight together, over a grid of blocks_per_cu blocks per CU (the caller tries shapes
// and keeps the fastest).
#include "attnres_internal.hpp"
#include "attnres_kernels.hpp"

namespace attnres {
namespace {

typedef uint32_t pr_u32x4 __attribute__((ext_vector_type(4)));

}  // namespace

// CPT chunks per thread and step, their loads of a group of streams issued together.
template <int CPT>
__global__ __launch_bounds__(256) void stream_probe_kernel(const ProbeArgs a) {
  constexpr int G = 8;
  const int64_t chunks = a.n_rows * a.row_chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < chunks;
       i0 += stride * CPT) {
    pr_u32x4 fold[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) fold[u] = pr_u32x4{0u, 0u, 0u, 0u};
    for (int j0 = 0; j0 < a.n_in; j0 += G) {
      pr_u32x4 x[CPT][G];
#pragma unroll
      for (int u = 0; u < CPT; ++u)
#pragma unroll
        for (int k = 0; k < G; ++k)
          if (j0 + k < a.n_in && i0 + u * stride < chunks)
            x[u][k] = __builtin_nontemporal_load(reinterpret_cast<const pr_u32x4*>(
                static_cast<const char*>(a.in[j0 + k]) + (i0 + u * stride) * 16));
#pragma unroll
      for (int u = 0; u < CPT; ++u)
#pragma unroll
        for (int k = 0; k < G; ++k) {
          const int j = j0 + k;
          if (j < a.n_in && i0 + u * stride < chunks) {
            fold[u] ^= x[u][k];
            if (j >= 1 && j < a.n_out)
              __builtin_nontemporal_store(x[u][k], reinterpret_cast<pr_u32x4*>(
                  static_cast<char*>(a.out[j]) + (i0 + u * stride) * 16));
          }
        }
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      if (i0 + u * stride >= chunks) break;
      const int64_t off = (i0 + u * stride) * 16;
      __builtin_nontemporal_store(fold[u],
                                  reinterpret_cast<pr_u32x4*>(static_cast<char*>(a.out[0]) + off));
      for (int j = a.n_in; j < a.n_out; ++j)
        __builtin_nontemporal_store(fold[u],
                                    reinterpret_cast<pr_u32x4*>(static_cast<char*>(a.out[j]) + off));
    }
  }
}

const void* stream_probe_kernel_ptr(int cpt) {
  switch (cpt) {
    case 1: return (const void*)&stream_probe_kernel<1>;
    case 2: return (const void*)&stream_probe_kernel<2>;
    case 4: return (const void*)&stream_probe_kernel<4>;
    default: return nullptr;
  }
}

}  // namespace attnres
