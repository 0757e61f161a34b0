// attnres_kernels.hpp -- gfx950 HIP kernels of the Attention Residuals (AttnRes) read.
//
// Operation ("Fast Attention Residuals" PyPI page, section "Equation"), per token n:
//   t_s = v_s[n, D-R..D-1]; rho_s = (mean(t_s^2) + eps)^(-1/2); z_s = scale * rho_s * <t_s, w*q>;
//   p = softmax_s(z); o = sum_s p_s v_s[n, :]; optional output RMSNorm y = o * rho_o * ow
//   (rho_o saved per row, FLA PR "[Perf] Parallelize AttnRes long-sequence reduction", Summary).
// Backward, with do = dL/do (through the output norm when on) and delta = sum_s p_s <do, v_s>:
//   dz_s = p_s (<do, v_s> - delta);  A_s = scale * dz_s * rho_s;  B_s = -A_s rho_s^2 c_s / R
//   dv_s = p_s do + [slice] (A_s * (w*q) + B_s * t_s);  du += A_s t_s;  dq = du*w, dw = du*q.
//
// Layout and mapping (MI355X, wave64):
//   * One workgroup of W waves owns one token at a time (persistent grid, tokens strided by the
//     grid size). The D columns of a row are cut into 16-byte chunks (8 bf16 or 4 f32); thread
//     `tid` owns chunks tid + j*blockDim for j < CH, so every load instruction of the workgroup
//     reads one contiguous, fully coalesced span of the row.
//   * A token's rows for a block of SB sources are held in VGPRs as packed 16-byte chunks.
//     Per-source partial sums (sum t^2, <t, w*q>, <do, v_s>) are reduced across a 16-lane row
//     with DPP, across rows and waves through a small double-buffered LDS exchange (one barrier
//     per source block), and finished on lane s of every wave, which then computes source s's
//     coefficients; v_readlane broadcasts them into SGPRs for the per-element FMAs.
//   * The resident backward keeps all S rows of a token on chip, so delta is exact in FP32 and
//     the output y is never re-read. The streaming backward (output norm on, or S*D too large)
//     reads the forward's FP32 mixture o instead and walks the sources in blocks.
//   * q/w/ow gradients: every backward workgroup keeps its own FP32 partial in registers for the
//     columns it owns and writes one row at the end; the finaliser sums the rows of each column
//     in a fixed order (deterministic), 64 columns x 16 row phases per workgroup.
// No MFMA: per token this is a GEMV with a softmax over a handful of sources, bound by HBM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attnres_args.hpp"

namespace attnres {

// ------------------------------------------------------------------ element access

struct alignas(16) Chunk {
  uint32_t w[4];
};

template <bool BF16>
struct Fmt {
  static constexpr int VEC = BF16 ? 8 : 4;   // elements per 16-byte chunk
  static constexpr int ESZ = BF16 ? 2 : 4;   // bytes per element
};

__device__ __forceinline__ float bits_f(uint32_t b) { return __builtin_bit_cast(float, b); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Element e of a chunk as FP32 (bf16 widening is exact: the 16 bits are the top half).
template <bool BF16>
__device__ __forceinline__ float elem(const Chunk& c, int e) {
  if constexpr (BF16) {
    const uint32_t w = c.w[e >> 1];
    return bits_f((e & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return bits_f(c.w[e]);
  }
}

// Two FP32 values to a packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <bool BF16>
__device__ __forceinline__ Chunk pack(const float* f) {
  Chunk c;
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = f_bits(f[i]);
  }
  return c;
}

// One scalar element of a small parameter vector (q, w, ow).
template <bool BF16>
__device__ __forceinline__ float load_param(const void* p, int i) {
  if constexpr (BF16) {
    return bits_f(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_param(void* p, int i, float v) {
  if constexpr (BF16) {
    typedef __bf16 bf16x1;
    static_cast<bf16x1*>(p)[i] = (bf16x1)v;
  } else {
    static_cast<float*>(p)[i] = v;
  }
}

__device__ __forceinline__ Chunk ld_chunk(const void* base, int64_t byte_off) {
  return *reinterpret_cast<const Chunk*>(static_cast<const char*>(base) + byte_off);
}

// Streaming store: the rows written here are not read again by this kernel.
__device__ __forceinline__ void st_chunk(void* base, int64_t byte_off, const Chunk& c) {
  uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<char*>(base) + byte_off);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = {c.w[0], c.w[1], c.w[2], c.w[3]};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ------------------------------------------------------------------ cross-lane reductions

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return bits_f(static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(f_bits(x)), CTRL, 0xF, 0xF, false)));
}

// Sum over the 16 lanes of a DPP row, result in every lane of the row (fixed order).
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0x128>(x);  // row_ror:8
  x += dpp<0x124>(x);  // row_ror:4
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  return x;
}

// Sum over the 64 lanes of the wave, result in every lane.
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum(x);
  auto a = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  x = bits_f(a[0]) + bits_f(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return bits_f(b[0]) + bits_f(b[1]);
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0xB1>(x));
  auto a = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  x = fmaxf(bits_f(a[0]), bits_f(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return fmaxf(bits_f(b[0]), bits_f(b[1]));
}

__device__ __forceinline__ float bcast(float x, int lane) {
  return bits_f(static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(f_bits(x)), lane)));
}

// Workgroup exchange of per-lane partials: every 16-lane row reduces value k with DPP and its
// first lane writes the row sum to xb[k * R4 + row], R4 = 4 * waves = rows in the workgroup.
__device__ __forceinline__ void xchg_put(float v, float* xb, int k, int R4, int tid) {
  const float r = row_sum(v);
  if ((tid & 15) == 0) xb[k * R4 + (tid >> 4)] = r;
}

// Total of value k after the barrier that follows the xchg_put calls (fixed summation order).
__device__ __forceinline__ float xchg_total(const float* xb, int k, int R4) {
  const float* p = xb + k * R4;
  float s = 0.f;
  for (int i = 0; i < R4; i += 4) {
    const float4 q = *reinterpret_cast<const float4*>(p + i);
    s += (q.x + q.y) + (q.z + q.w);
  }
  return s;
}

// LDS floats one exchange buffer needs for K values and W waves (R4 = 4W, padded to 4).
__host__ __device__ constexpr int xchg_floats(int K, int W) { return K * 4 * W; }

// ------------------------------------------------------------------ per-lane column setup

// For the CH chunks this thread owns: start column, validity, u = w*q (0 off the slice) and
// whether each element lies in the key slice.
template <bool BF16, int CH>
struct Cols {
  static constexpr int VEC = Fmt<BF16>::VEC;
  int col0[CH];
  bool valid[CH];
  float u[CH][VEC];

  __device__ __forceinline__ void init(int tid, int nthr, int D, int lo, const void* query,
                                       const void* norm_w) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      col0[j] = (tid + j * nthr) * VEC;
      valid[j] = col0[j] < D;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int idx = col0[j] + e - lo;
        float uv = 0.f;
        if (valid[j] && idx >= 0) {
          uv = load_param<BF16>(query, idx);
          if (norm_w) uv *= load_param<BF16>(norm_w, idx);
        }
        u[j][e] = uv;
      }
    }
  }
  __device__ __forceinline__ bool in_slice(int j, int e, int lo) const {
    return col0[j] + e >= lo;
  }
};

// ------------------------------------------------------------------ forward

// Forward. SB = sources held per block; S <= SB runs as one block (no rescaling).
template <bool BF16, int CH, int SB, bool FULL>
__global__ __launch_bounds__(512) void fwd_kernel(const FwdArgs a) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int K = 2 * SB;
  extern __shared__ float lds[];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
  const int R4 = nthr >> 4;
  const int xfl = K * R4;

  Cols<BF16, CH> cs;
  cs.init(tid, nthr, a.D, a.lo, a.query, a.norm_w);
  float ow[CH][VEC];
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      ow[j][e] = (a.out_norm && a.out_w && cs.valid[j]) ? load_param<BF16>(a.out_w, cs.col0[j] + e)
                                                         : 1.f;
  int buf = 0;

  for (int64_t n = blockIdx.x; n < a.N; n += gridDim.x) {
    const int64_t row_off = n * a.row_stride * ESZ;
    float acc[CH][VEC];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[j][e] = 0.f;
    float m = -INFINITY, l = 0.f;

    for (int s0 = 0; s0 < a.S; s0 += SB) {
      const int nb = min(SB, a.S - s0);
      Chunk rows[SB][CH];
#pragma unroll
      for (int i = 0; i < SB; ++i)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          if (i < nb && cs.valid[j]) {
            rows[i][j] = ld_chunk(a.src[s0 + i], row_off + (int64_t)cs.col0[j] * ESZ);
          } else {
            rows[i][j] = Chunk{{0u, 0u, 0u, 0u}};
          }
        }
      float* xb = lds + buf * xfl;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        if (i < nb) {
          float ss = 0.f, c = 0.f;
#pragma unroll
          for (int j = 0; j < CH; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const float t = elem<BF16>(rows[i][j], e);
              const float tm = (FULL || cs.in_slice(j, e, a.lo)) ? t : 0.f;
              ss = fmaf(tm, tm, ss);
              c = fmaf(t, cs.u[j][e], c);
            }
          xchg_put(ss, xb, i, R4, tid);
          xchg_put(c, xb, SB + i, R4, tid);
        }
      }
      __syncthreads();
      buf ^= 1;
      float z = -INFINITY;
      if (lane < nb) {
        const float ss = xchg_total(xb, lane, R4);
        const float c = xchg_total(xb, SB + lane, R4);
        z = a.scale * c / sqrtf(ss * a.inv_R + a.eps);
      }
      const float m_new = fmaxf(m, wave_max(z));
      const float ez = (lane < nb) ? expf(z - m_new) : 0.f;
      const float lb = wave_sum(ez);
      if (s0 > 0) {
        const float alpha = expf(m - m_new);
        l = l * alpha + lb;
        if (alpha != 1.f) {
#pragma unroll
          for (int j = 0; j < CH; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[j][e] *= alpha;
        }
      } else {
        l = lb;
      }
      m = m_new;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        if (i < nb) {
          const float pi = bcast(ez, i);
#pragma unroll
          for (int j = 0; j < CH; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[j][e] = fmaf(pi, elem<BF16>(rows[i][j], e), acc[j][e]);
        }
      }
    }

    const float inv_l = 1.f / l;
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[j][e] *= inv_l;  // acc now holds o

    float rho_o = 1.f;
    if (a.out_norm) {
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) sq = fmaf(acc[j][e], acc[j][e], sq);
      float* xb = lds + buf * xfl;
      xchg_put(sq, xb, 0, R4, tid);
      __syncthreads();
      buf ^= 1;
      rho_o = 1.f / sqrtf(xchg_total(xb, 0, R4) * a.inv_D + a.eps);
      if (a.o32) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          if (!cs.valid[j]) continue;
          float* dst = a.o32 + n * a.D + cs.col0[j];
#pragma unroll
          for (int h = 0; h < VEC; h += 4) {
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            f32x4 v = {acc[j][h], acc[j][h + 1], acc[j][h + 2], acc[j][h + 3]};
            *reinterpret_cast<f32x4*>(dst + h) = v;
          }
        }
      }
    } else if (a.o32) {
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        if (!cs.valid[j]) continue;
        float* dst = a.o32 + n * a.D + cs.col0[j];
#pragma unroll
        for (int h = 0; h < VEC; h += 4) {
          typedef float f32x4 __attribute__((ext_vector_type(4)));
          f32x4 v = {acc[j][h], acc[j][h + 1], acc[j][h + 2], acc[j][h + 3]};
          *reinterpret_cast<f32x4*>(dst + h) = v;
        }
      }
    }

#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (!cs.valid[j]) continue;
      float yv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) yv[e] = a.out_norm ? acc[j][e] * rho_o * ow[j][e] : acc[j][e];
      st_chunk(a.y, (n * a.D + cs.col0[j]) * ESZ, pack<BF16>(yv));
    }
    if (tid == 0) {
      a.lse[n] = m + logf(l);
      if (a.out_norm && a.o_rstd) a.o_rstd[n] = rho_o;
    }
  }
}

// ------------------------------------------------------------------ backward, shared tail

// Writes this workgroup's partial sums of du (slice columns) and dow (all columns).
template <bool BF16, int CH>
__device__ __forceinline__ void write_partials(const BwdArgs& a, const Cols<BF16, CH>& cs,
                                               const float (&du)[CH][Fmt<BF16>::VEC],
                                               const float (&dow)[CH][Fmt<BF16>::VEC]) {
  constexpr int VEC = Fmt<BF16>::VEC;
  float* pdu = a.part_du + (int64_t)blockIdx.x * a.R;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    if (!cs.valid[j]) continue;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int idx = cs.col0[j] + e - a.lo;
      if (idx >= 0) pdu[idx] = du[j][e];
    }
  }
  if (a.part_dow) {
    float* pdw = a.part_dow + (int64_t)blockIdx.x * a.D;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (!cs.valid[j]) continue;
#pragma unroll
      for (int e = 0; e < VEC; ++e) pdw[cs.col0[j] + e] = dow[j][e];
    }
  }
}

// ------------------------------------------------------------------ backward, token-resident

// All S <= SB rows of a token stay in VGPRs: delta = sum_s p_s <dY, v_s> is exact in FP32.
// No output norm on this path (dL/do = dY).
template <bool BF16, int CH, int SB, bool FULL>
__global__ __launch_bounds__(512) void bwd_resident_kernel(const BwdArgs a) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int K = 3 * SB;
  extern __shared__ float lds[];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
  const int R4 = nthr >> 4;
  const int xfl = K * R4;

  Cols<BF16, CH> cs;
  cs.init(tid, nthr, a.D, a.lo, a.query, a.norm_w);
  float du[CH][VEC], dow[CH][VEC];
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int e = 0; e < VEC; ++e) du[j][e] = dow[j][e] = 0.f;
  const int S = a.S;
  int buf = 0;

  for (int64_t n = blockIdx.x; n < a.N; n += gridDim.x) {
    const int64_t row_off = n * a.row_stride * ESZ;
    Chunk rows[SB][CH];
    Chunk gy[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j)
      gy[j] = cs.valid[j] ? ld_chunk(a.dout, (n * a.dout_stride + cs.col0[j]) * ESZ)
                          : Chunk{{0u, 0u, 0u, 0u}};
#pragma unroll
    for (int i = 0; i < SB; ++i)
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        if (i < S && cs.valid[j]) {
          rows[i][j] = ld_chunk(a.src[i], row_off + (int64_t)cs.col0[j] * ESZ);
        } else {
          rows[i][j] = Chunk{{0u, 0u, 0u, 0u}};
        }
      }
    const float lse = a.lse[n];
    float* xb = lds + buf * xfl;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      if (i < S) {
        float ss = 0.f, c = 0.f, dp = 0.f;
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float t = elem<BF16>(rows[i][j], e);
            const float tm = (FULL || cs.in_slice(j, e, a.lo)) ? t : 0.f;
            ss = fmaf(tm, tm, ss);
            c = fmaf(t, cs.u[j][e], c);
            dp = fmaf(elem<BF16>(gy[j], e), t, dp);
          }
        xchg_put(ss, xb, i, R4, tid);
        xchg_put(c, xb, SB + i, R4, tid);
        xchg_put(dp, xb, 2 * SB + i, R4, tid);
      }
    }
    __syncthreads();
    buf ^= 1;

    // lane s finishes source s
    float p = 0.f, dp = 0.f, rho = 0.f, c = 0.f;
    if (lane < S) {
      const float ss = xchg_total(xb, lane, R4);
      c = xchg_total(xb, SB + lane, R4);
      dp = xchg_total(xb, 2 * SB + lane, R4);
      rho = 1.f / sqrtf(ss * a.inv_R + a.eps);
      p = expf(a.scale * rho * c - lse);
    }
    const float delta = wave_sum(p * dp);
    const float A = a.scale * p * (dp - delta) * rho;
    const float B = -A * rho * rho * c * a.inv_R;

#pragma unroll
    for (int i = 0; i < SB; ++i) {
      if (i < S) {
        const float pi = bcast(p, i), Ai = bcast(A, i), Bi = bcast(B, i);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          float dv[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float t = elem<BF16>(rows[i][j], e);
            const float tm = (FULL || cs.in_slice(j, e, a.lo)) ? t : 0.f;
            float d = pi * elem<BF16>(gy[j], e);
            d = fmaf(Ai, cs.u[j][e], d);
            d = fmaf(Bi, tm, d);
            dv[e] = d;
            du[j][e] = fmaf(Ai, t, du[j][e]);
          }
          if (cs.valid[j])
            st_chunk(a.dsrc[i], (n * a.drow_stride + cs.col0[j]) * ESZ, pack<BF16>(dv));
        }
      }
    }
  }
  write_partials<BF16, CH>(a, cs, du, dow);
}

// ------------------------------------------------------------------ backward, streaming

// Sources walked in blocks of SB using the forward's FP32 mixture o (and rho_o with the output
// norm): do and delta = <do, o> are known before the first source is read.
template <bool BF16, int CH, int SB, bool FULL>
__global__ __launch_bounds__(512) void bwd_stream_kernel(const BwdArgs a) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int K = 3 * SB;
  extern __shared__ float lds[];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
  const int R4 = nthr >> 4;
  const int xfl = K * R4;

  Cols<BF16, CH> cs;
  cs.init(tid, nthr, a.D, a.lo, a.query, a.norm_w);
  float du[CH][VEC], dow[CH][VEC], ow[CH][VEC];
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      du[j][e] = dow[j][e] = 0.f;
      ow[j][e] = (a.out_norm && a.out_w && cs.valid[j]) ? load_param<BF16>(a.out_w, cs.col0[j] + e)
                                                         : 1.f;
    }
  int buf = 0;

  for (int64_t n = blockIdx.x; n < a.N; n += gridDim.x) {
    const int64_t row_off = n * a.row_stride * ESZ;
    float dov[CH][VEC], o[CH][VEC];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      Chunk g = cs.valid[j] ? ld_chunk(a.dout, (n * a.dout_stride + cs.col0[j]) * ESZ)
                            : Chunk{{0u, 0u, 0u, 0u}};
#pragma unroll
      for (int h = 0; h < VEC; h += 4) {
        Chunk oc = cs.valid[j] ? ld_chunk(a.o32, (n * a.D + cs.col0[j] + h) * 4)
                               : Chunk{{0u, 0u, 0u, 0u}};
#pragma unroll
        for (int e = 0; e < 4; ++e) o[j][h + e] = bits_f(oc.w[e]);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) dov[j][e] = elem<BF16>(g, e);
    }
    // do and delta = <do, o>
    float delta;
    {
      float part[2] = {0.f, 0.f};
      if (a.out_norm) {
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float g = dov[j][e] * ow[j][e];
            part[0] = fmaf(g, o[j][e], part[0]);          // <g, o>
            part[1] = fmaf(o[j][e], o[j][e], part[1]);    // <o, o>
          }
      } else {
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) part[0] = fmaf(dov[j][e], o[j][e], part[0]);
      }
      float* xb = lds + buf * xfl;
      xchg_put(part[0], xb, 0, R4, tid);
      xchg_put(part[1], xb, 1, R4, tid);
      __syncthreads();
      buf ^= 1;
      const float t0 = xchg_total(xb, 0, R4);
      if (a.out_norm) {
        const float oo = xchg_total(xb, 1, R4);
        const float ro = a.o_rstd[n];
        const float k3 = ro * ro * ro * a.inv_D * t0;
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float gy = dov[j][e];
            dow[j][e] = fmaf(gy, ro * o[j][e], dow[j][e]);
            dov[j][e] = ro * gy * ow[j][e] - k3 * o[j][e];
          }
        // <do, o> = ro <g, o> - ro^3 <g, o> <o, o> / D
        delta = ro * t0 - k3 * oo;
      } else {
        delta = t0;
      }
    }
    const float lse = a.lse[n];

    for (int s0 = 0; s0 < a.S; s0 += SB) {
      const int nb = min(SB, a.S - s0);
      Chunk rows[SB][CH];
#pragma unroll
      for (int i = 0; i < SB; ++i)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          if (i < nb && cs.valid[j]) {
            rows[i][j] = ld_chunk(a.src[s0 + i], row_off + (int64_t)cs.col0[j] * ESZ);
          } else {
            rows[i][j] = Chunk{{0u, 0u, 0u, 0u}};
          }
        }
      float* xb = lds + buf * xfl;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        if (i < nb) {
          float ss = 0.f, c = 0.f, dp = 0.f;
#pragma unroll
          for (int j = 0; j < CH; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const float t = elem<BF16>(rows[i][j], e);
              const float tm = (FULL || cs.in_slice(j, e, a.lo)) ? t : 0.f;
              ss = fmaf(tm, tm, ss);
              c = fmaf(t, cs.u[j][e], c);
              dp = fmaf(dov[j][e], t, dp);
            }
          xchg_put(ss, xb, i, R4, tid);
          xchg_put(c, xb, SB + i, R4, tid);
          xchg_put(dp, xb, 2 * SB + i, R4, tid);
        }
      }
      __syncthreads();
      buf ^= 1;
      float p = 0.f, dp = 0.f, rho = 0.f, c = 0.f;
      if (lane < nb) {
        const float ss = xchg_total(xb, lane, R4);
        c = xchg_total(xb, SB + lane, R4);
        dp = xchg_total(xb, 2 * SB + lane, R4);
        rho = 1.f / sqrtf(ss * a.inv_R + a.eps);
        p = expf(a.scale * rho * c - lse);
      }
      const float A = a.scale * p * (dp - delta) * rho;
      const float B = -A * rho * rho * c * a.inv_R;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        if (i < nb) {
          const float pi = bcast(p, i), Ai = bcast(A, i), Bi = bcast(B, i);
#pragma unroll
          for (int j = 0; j < CH; ++j) {
            float dv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const float t = elem<BF16>(rows[i][j], e);
              const float tm = (FULL || cs.in_slice(j, e, a.lo)) ? t : 0.f;
              float d = pi * dov[j][e];
              d = fmaf(Ai, cs.u[j][e], d);
              d = fmaf(Bi, tm, d);
              dv[e] = d;
              du[j][e] = fmaf(Ai, t, du[j][e]);
            }
            if (cs.valid[j])
              st_chunk(a.dsrc[s0 + i], (n * a.drow_stride + cs.col0[j]) * ESZ, pack<BF16>(dv));
          }
        }
      }
    }
  }
  write_partials<BF16, CH>(a, cs, du, dow);
}

// ------------------------------------------------------------------ finaliser

// Sums the P partial rows of every column in a fixed order and writes dq = du*w (du without w),
// dw = du*q and dow. Thread (phase r, column c) adds rows r, r+16, r+32, ...; the 16 phase sums
// are then added in phase order through LDS. No atomics and no inter-workgroup traffic.
template <bool BF16>
__global__ __launch_bounds__(kFinCols * kFinPhases) void finalize_kernel(const FinArgs a) {
  __shared__ float red[kFinPhases][kFinCols];
  const int cl = threadIdx.x % kFinCols, ph = threadIdx.x / kFinCols;
  const int c = blockIdx.x * kFinCols + cl;
  const bool has = c < a.cols;
  const bool is_du = c < a.R;
  float s = 0.f;
  if (has) {
    const float* base = is_du ? a.part_du + c : a.part_dow + (c - a.R);
    const int64_t stride = is_du ? a.R : a.D;
#pragma unroll 4
    for (int p = ph; p < a.P; p += kFinPhases) s += base[p * stride];
  }
  red[ph][cl] = s;
  __syncthreads();
  if (ph != 0 || !has) return;
  float total = 0.f;
#pragma unroll
  for (int r = 0; r < kFinPhases; ++r) total += red[r][cl];
  if (is_du) {
    const float wv = a.norm_w ? load_param<BF16>(a.norm_w, c) : 1.f;
    store_param<BF16>(a.dq, c, total * wv);
    if (a.norm_w) store_param<BF16>(a.dw, c, total * load_param<BF16>(a.query, c));
  } else {
    store_param<BF16>(a.dow, c - a.R, total);
  }
}

}  // namespace attnres
