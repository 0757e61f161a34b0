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
//   * Row addresses are a uniform (SGPR) base per source and token plus a loop-invariant 32-bit
//     lane offset, so loads and stores use the scalar-base form with no per-lane address math.
//   * A token's rows for a block of SB sources are held in VGPRs as packed 16-byte chunks.
//     Per-source partial sums (sum t^2, <t, w*q>, <do, v_s>) are reduced across a 16-lane row
//     with DPP, across rows and waves through a small double-buffered LDS exchange (one barrier
//     per source block), and finished on lane s of every wave, which then computes source s's
//     coefficients; v_readlane broadcasts them into SGPRs for the per-element FMAs.
//   * bf16 sums of products use v_dot2_f32_bf16 on packed pairs (exact products, FP32
//     accumulation), so t never needs widening for them. The FP32 vector u = w*q is split exactly
//     into three bf16 terms (u = u1 + u2 + u3), which keeps <t, u> at FP32 accuracy.
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bits_f(uint32_t b) { return __builtin_bit_cast(float, b); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Low / high bf16 of a packed pair, widened exactly to FP32.
__device__ __forceinline__ float lo_f(uint32_t w) { return bits_f(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return bits_f(w & 0xffff0000u); }

// Element e of a chunk as FP32.
template <bool BF16>
__device__ __forceinline__ float elem(const Chunk& c, int e) {
  if constexpr (BF16) {
    return (e & 1) ? hi_f(c.w[e >> 1]) : lo_f(c.w[e >> 1]);
  } else {
    return bits_f(c.w[e]);
  }
}

// a.lo * b.lo + a.hi * b.hi + acc with exact bf16 products and FP32 accumulation.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Two FP32 values to a packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
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
    static_cast<__bf16*>(p)[i] = (__bf16)v;
  } else {
    static_cast<float*>(p)[i] = v;
  }
}

// A row of `bytes` bytes at base + row_byte as a buffer resource: the 64-bit base lives in SGPRs,
// every access adds a 32-bit per-lane offset, and accesses at or past `bytes` read 0 and drop
// their writes (the hardware range check covers the chunks past D of the last waves).
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc row_rsrc(const void* base, int64_t row_byte, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(base) + row_byte), 0, bytes, 0x00020000);
}

// Streaming 16-byte load (non-temporal: every row is read once per kernel).
// Row resource of source i of a block of `count` sources: empty (reads 0, writes dropped, no
// memory traffic) for i >= count, so loops over a block need no per-source branches.
__device__ __forceinline__ Rsrc src_rsrc(const void* base, int i, int count, int64_t row_byte,
                                         uint32_t bytes) {
  const bool live = i < count;
  return row_rsrc(live ? base : nullptr, live ? row_byte : 0, live ? bytes : 0u);
}

__device__ __forceinline__ Chunk ld_row(Rsrc r, uint32_t voff) {
  return __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2));
}

// Streaming 16-byte store (non-temporal: the rows written are not read again by the kernel).
__device__ __forceinline__ void st_row(Rsrc r, uint32_t voff, const Chunk& c) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c), r, voff, 0, 2);
}

// Loads and stores that go to L2 (sc0: no stale vector-L1 line), for rows a thread rewrites.
__device__ __forceinline__ Chunk ld_row_cached(Rsrc r, uint32_t voff) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 1));
}
__device__ __forceinline__ void st_row_cached(Rsrc r, uint32_t voff, const Chunk& c) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c), r, voff, 0, 1);
}

// (the 4-byte forms move integer words: FP32 values go through bit casts)
__device__ __forceinline__ float ld_f32_cached(Rsrc r, uint32_t voff) {
  return bits_f(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 1)));
}
__device__ __forceinline__ void st_f32_cached(Rsrc r, uint32_t voff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(f_bits(v), r, voff, 0, 1);
}

__device__ __forceinline__ void st_f32x4(float* p, float a, float b, float c, float d) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
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

// Sources per exchange group: a group's partials are reduced and written before the next group is
// computed, which bounds the live partial registers to NV * kGroup.
constexpr int kGroup = 4;

// Workgroup exchange of per-lane partials. Each 16-lane row reduces value v of group source g
// with DPP (the NV * kGroup chains are independent, so their hazards overlap), then the row's
// first lane writes it to xb[(v * SB + i0 + g) * R4 + row], R4 = 4 * waves = rows in the
// workgroup (slots of sources past the block's count hold zeros and are never read).
template <int NV, int SB>
__device__ __forceinline__ void xchg_group(float (&v)[NV][kGroup], int i0, float* xb, int R4,
                                           int tid) {
#pragma unroll
  for (int t = 0; t < NV; ++t)
#pragma unroll
    for (int g = 0; g < kGroup; ++g) v[t][g] = row_sum(v[t][g]);
  if ((tid & 15) == 0) {
    float* dst = xb + (tid >> 4);
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
      if (i0 + g < SB)
#pragma unroll
        for (int t = 0; t < NV; ++t) dst[(t * SB + i0 + g) * R4] = v[t][g];
  }
}

// Total of value k after the barrier that follows xchg_put (fixed summation order).
__device__ __forceinline__ float xchg_total(const float* xb, int k, int R4) {
  const float* p = xb + k * R4;
  float s = 0.f;
  for (int i = 0; i < R4; i += 4) {
    const float4 q = *reinterpret_cast<const float4*>(p + i);
    s += (q.x + q.y) + (q.z + q.w);
  }
  return s;
}

// ------------------------------------------------------------------ per-source scalars

// Reciprocal key RMS and score of one source from its slice sums, each operation rounded on its
// own: with contraction off here, no product below can be fused into an FMA with its neighbours or
// with the caller's subtraction of lse, so the forward and both backwards compute bitwise-identical
// scores and the backward's exp(score - lse) reproduces the forward's routing weights (exactly 1
// for a single source). Division and square root are the correctly rounded HIP defaults.
struct Score {
  float rho, z;
};
__device__ __forceinline__ Score source_score(float ss, float c, float inv_R, float eps,
                                              float scale) {
#pragma clang fp contract(off)
  Score r;
  r.rho = 1.f / sqrtf(ss * inv_R + eps);
  r.z = (scale * r.rho) * c;
  return r;
}

// Routing weight of a source from its score and the token's log-sum-exp (no contraction).
__device__ __forceinline__ float routing_weight(float z, float lse) {
#pragma clang fp contract(off)
  const float x = z - lse;
  return expf(x);
}

// ------------------------------------------------------------------ per-lane column setup

// Columns of the CH chunks a thread owns: byte offset inside a row, validity and, for R < D with
// bf16, a per-half mask of the key slice. The loop-invariant parameter vectors are u = w*q on the
// slice (0 elsewhere) in FP32 and, for bf16, its exact three-term split u = u1 + u2 + u3 in packed
// bf16 pairs. With CH <= 2 they live in LDS rather than VGPRs (each thread's slots are 16 bytes,
// lane-contiguous; 10 bytes per column for bf16) and kernels fetch them per token through a
// laundered offset, so the compiler cannot hoist them back into registers. With CH == 4 (the
// widest rows) the region would not fit a workgroup's LDS, and they stay in registers.
template <bool BF16, int CH, bool FULL>
struct Cols {
  static constexpr int VEC = Fmt<BF16>::VEC;
  static constexpr int ESZ = Fmt<BF16>::ESZ;
  static constexpr bool IN_LDS = CH <= 2;
  static constexpr int U_SLOTS = CH * VEC / 4;          // float4 slots of u
  static constexpr int S_SLOTS = BF16 ? 3 * CH : 0;     // uint4 slots of the split
  static constexpr int SLOTS = IN_LDS ? U_SLOTS + S_SLOTS : 0;
  int col0[CH];
  uint32_t voff[CH];
  bool valid[CH];
  uint32_t mk[CH][4];
  char* params;  // this workgroup's parameter region in LDS (IN_LDS)
  int nthr;
  float ureg[IN_LDS ? 1 : CH][VEC];       // registers otherwise
  uint32_t usreg[IN_LDS ? 1 : 3][IN_LDS ? 1 : CH][4];

  // LDS bytes of the parameter region for a workgroup of `threads` threads.
  static constexpr uint32_t param_bytes(int threads) { return SLOTS * threads * 16u; }

  __device__ __forceinline__ void init(int tid, int nthr_, int D, int lo, const void* query,
                                       const void* norm_w, float* lds_params) {
    nthr = nthr_;
    params = reinterpret_cast<char*>(lds_params);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      col0[j] = (tid + j * nthr) * VEC;
      voff[j] = static_cast<uint32_t>(col0[j] * ESZ);
      valid[j] = col0[j] < D;
      float u[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int idx = col0[j] + e - lo;
        float uv = 0.f;
        if (valid[j] && idx >= 0) {
          uv = load_param<BF16>(query, idx);
          if (norm_w) uv *= load_param<BF16>(norm_w, idx);
        }
        u[e] = uv;
      }
      if constexpr (IN_LDS) {
#pragma unroll
        for (int h = 0; h < VEC / 4; ++h)
          *reinterpret_cast<float4*>(params + ((j * (VEC / 4) + h) * nthr + tid) * 16) =
              make_float4(u[4 * h], u[4 * h + 1], u[4 * h + 2], u[4 * h + 3]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) ureg[IN_LDS ? 0 : j][e] = u[e];
      }
      if constexpr (BF16) {
        uint32_t us[3][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float r0 = u[2 * k], r1 = u[2 * k + 1];
#pragma unroll
          for (int t = 0; t < 3; ++t) {  // u = u1 + u2 + u3; each remainder is exact in FP32
            const __bf16 b0 = (__bf16)r0, b1 = (__bf16)r1;
            us[t][k] = pack_bf16x2(b0, b1);
            r0 -= (float)b0;
            r1 -= (float)b1;
          }
          const bool in0 = col0[j] + 2 * k >= lo, in1 = col0[j] + 2 * k + 1 >= lo;
          mk[j][k] = (in0 ? 0x0000ffffu : 0u) | (in1 ? 0xffff0000u : 0u);
        }
        if constexpr (IN_LDS) {
#pragma unroll
          for (int t = 0; t < 3; ++t)
            *reinterpret_cast<uint4*>(params + ((U_SLOTS + t * CH + j) * nthr + tid) * 16) =
                make_uint4(us[t][0], us[t][1], us[t][2], us[t][3]);
        } else {
#pragma unroll
          for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int k = 0; k < 4; ++k) usreg[IN_LDS ? 0 : t][IN_LDS ? 0 : j][k] = us[t][k];
        }
      }
    }
  }

  // Per-token fetches (after the barrier that follows init). `lane_off` = tid * 16, laundered by
  // the caller once per token.
  __device__ __forceinline__ void fetch_u(uint32_t lane_off, float (&u)[CH][VEC]) const {
    if constexpr (!IN_LDS) {
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) u[j][e] = ureg[IN_LDS ? 0 : j][e];
      return;
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int h = 0; h < VEC / 4; ++h) {
        const float4 v = *reinterpret_cast<const float4*>(
            params + (j * (VEC / 4) + h) * nthr * 16 + lane_off);
        u[j][4 * h] = v.x;
        u[j][4 * h + 1] = v.y;
        u[j][4 * h + 2] = v.z;
        u[j][4 * h + 3] = v.w;
      }
  }
  __device__ __forceinline__ void fetch_us(uint32_t lane_off, uint32_t (&us)[3][CH][4]) const {
    if constexpr (BF16 && !IN_LDS) {
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int k = 0; k < 4; ++k) us[t][j][k] = usreg[IN_LDS ? 0 : t][IN_LDS ? 0 : j][k];
      return;
    }
    if constexpr (BF16) {
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const uint4 v = *reinterpret_cast<const uint4*>(
              params + (U_SLOTS + t * CH + j) * nthr * 16 + lane_off);
          us[t][j][0] = v.x;
          us[t][j][1] = v.y;
          us[t][j][2] = v.z;
          us[t][j][3] = v.w;
        }
    }
  }

  __device__ __forceinline__ bool in_slice(int j, int e, int lo) const {
    return FULL || col0[j] + e >= lo;
  }
};

// Per-token per-lane LDS offset that the compiler cannot prove loop-invariant.
__device__ __forceinline__ uint32_t laundered_lane_off(int tid) {
  uint32_t off = static_cast<uint32_t>(tid) * 16u;
  asm volatile("" : "+v"(off));
  return off;
}

// sum over the slice of t^2 and <t, u> for one row (this thread's chunks).
template <bool BF16, int CH, bool FULL>
__device__ __forceinline__ void key_sums(const Chunk (&r)[CH], const Cols<BF16, CH, FULL>& cs,
                                         const uint32_t (&us)[3][CH][4],
                                         const float (&u)[CH][Fmt<BF16>::VEC], int lo, float& ss,
                                         float& c) {
  ss = 0.f;
  c = 0.f;
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t p = r[j].w[k];
        const uint32_t pm = FULL ? p : (p & cs.mk[j][k]);
        ss = dot2(pm, pm, ss);
        c = dot2(p, us[0][j][k], c);
        c = dot2(p, us[1][j][k], c);
        c = dot2(p, us[2][j][k], c);
      }
  } else {
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = elem<false>(r[j], e);
        const float tm = cs.in_slice(j, e, lo) ? t : 0.f;
        ss = fmaf(tm, tm, ss);
        c = fmaf(t, u[j][e], c);
      }
  }
}

// <g, v> over this thread's chunks, g and v both in storage format.
template <bool BF16, int CH>
__device__ __forceinline__ float dot_rows(const Chunk (&v)[CH], const Chunk (&g)[CH]) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (BF16) {
        acc = dot2(g[j].w[k], v[j].w[k], acc);
      } else {
        acc = fmaf(bits_f(g[j].w[k]), bits_f(v[j].w[k]), acc);
      }
    }
  return acc;
}

// <g, v> with g in FP32.
template <bool BF16, int CH>
__device__ __forceinline__ float dot_f32(const Chunk (&v)[CH], const float (&g)[CH][Fmt<BF16>::VEC]) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int e = 0; e < Fmt<BF16>::VEC; ++e) acc = fmaf(g[j][e], elem<BF16>(v[j], e), acc);
  return acc;
}

// dv = p*do + A*u + B*t (t masked to the slice) and du += A*t for one source row. With ACC the
// row's existing gradient `old` is added in FP32 before the single rounding to storage.
template <bool BF16, int CH, bool FULL, bool ACC = false>
__device__ __forceinline__ void grad_row(const Chunk (&r)[CH], const Cols<BF16, CH, FULL>& cs,
                                         const float (&u)[CH][Fmt<BF16>::VEC],
                                         const float (&dof)[CH][Fmt<BF16>::VEC], float p,
                                         float A, float B, int lo,
                                         float (&du)[CH][Fmt<BF16>::VEC], Chunk (&out)[CH],
                                         const Chunk (&old)[CH]) {
  constexpr int VEC = Fmt<BF16>::VEC;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    float dv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float tm;
      if constexpr (BF16) {
        const uint32_t w = FULL ? r[j].w[e >> 1] : (r[j].w[e >> 1] & cs.mk[j][e >> 1]);
        tm = (e & 1) ? hi_f(w) : lo_f(w);
      } else {
        const float t = elem<false>(r[j], e);
        tm = cs.in_slice(j, e, lo) ? t : 0.f;
      }
      float d = p * dof[j][e];
      d = fmaf(A, u[j][e], d);
      d = fmaf(B, tm, d);
      if constexpr (ACC) d += elem<BF16>(old[j], e);
      dv[e] = d;
      du[j][e] = fmaf(A, tm, du[j][e]);
    }
    out[j] = pack<BF16>(dv);
  }
}

// ------------------------------------------------------------------ occupancy

// Waves per SIMD the register allocator is asked to allow: three workgroups of a 4-wave token
// (3 waves per SIMD, <= 168 VGPRs) keep more tokens' loads in flight per CU than two, and the
// register budget allows it while a token's rows take at most 20 chunks per thread (12 with the
// slice masks of R < D); larger slabs keep the default.
constexpr int occupancy_hint(int ch, int sb, bool full) {
  return ch * sb <= (full ? 20 : 12) ? 3 : 1;
}

// The forward's counters return to zero once every workgroup has taken its last ticket.
__device__ __forceinline__ void fwd_release_counters(uint32_t* ctr, int tid) {
  if (tid == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(ctr + kCtrArrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == gridDim.x) {
      __hip_atomic_store(ctr + kCtrTicket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctr + kCtrArrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ forward

// Output row: o (= acc / l already applied) to y, with the optional output RMSNorm, plus lse,
// rho_o and the FP32 mixture when requested.
template <bool BF16, int CH, bool FULL>
__device__ __forceinline__ void fwd_emit(const FwdArgs& a, const Cols<BF16, CH, FULL>& cs,
                                         float (&acc)[CH][Fmt<BF16>::VEC],
                                         const float (&ow)[CH][Fmt<BF16>::VEC], int64_t n,
                                         float lse, float* lds, int& buf, int xfl, int R4,
                                         int tid, uint32_t row_bytes) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  float rho_o = 1.f;
  if (a.out_norm) {
    float sq[1][kGroup] = {{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) sq[0][0] = fmaf(acc[j][e], acc[j][e], sq[0][0]);
    float* xb = lds + buf * xfl;
    xchg_group<1, 1>(sq, 0, xb, R4, tid);
    __syncthreads();
    buf ^= 1;
    rho_o = 1.f / sqrtf(xchg_total(xb, 0, R4) * a.inv_D + a.eps);
  }
  if (a.o32) {
    const Rsrc ro = row_rsrc(a.o32, n * a.D * 4, static_cast<uint32_t>(a.D * 4));
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int h = 0; h < VEC; h += 4) {
        Chunk c;
#pragma unroll
        for (int e = 0; e < 4; ++e) c.w[e] = f_bits(acc[j][h + e]);
        st_row(ro, static_cast<uint32_t>((cs.col0[j] + h) * 4), c);
      }
  }
  const Rsrc ry = row_rsrc(a.y, n * a.D * ESZ, row_bytes);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    float yv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) yv[e] = a.out_norm ? acc[j][e] * rho_o * ow[j][e] : acc[j][e];
    st_row(ry, cs.voff[j], pack<BF16>(yv));
  }
  if (tid == 0) {
    a.lse[n] = lse;
    if (a.out_norm && a.o_rstd) a.o_rstd[n] = rho_o;
  }
}

// Forward. ONE: all S <= SB sources in one block, software-pipelined over tokens (the next
// token's row i is loaded as soon as row i has been folded into the output, so the load overlaps
// this token's remaining math and stores, and the next token's first wait covers only what was
// issued before it; the vector-memory counter retires loads and stores in order).
// !ONE: blocks of SB sources with an online softmax (running max and sum, rescaled output).
template <bool BF16, int CH, int SB, bool FULL, bool ONE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(occupancy_hint(CH, ONE ? SB : 2 * SB, FULL), 8)))
void fwd_kernel(const FwdArgs a) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int K = 2 * SB;
  extern __shared__ float lds_all[];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
  const int R4 = nthr >> 4;
  const int xfl = K * R4;
  const uint32_t row_bytes = static_cast<uint32_t>(a.D * ESZ);

  Cols<BF16, CH, FULL> cs;
  cs.init(tid, nthr, a.D, a.lo, a.query, a.norm_w, lds_all);
  float* lds = lds_all + Cols<BF16, CH, FULL>::param_bytes(nthr) / 4;  // exchange buffers
  float ow[CH][VEC];
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      ow[j][e] = (a.out_norm && a.out_w && cs.valid[j]) ? load_param<BF16>(a.out_w, cs.col0[j] + e)
                                                         : 1.f;
  int buf = 0;
  // Every loop below runs over all SB slots of a block; slots past the block's source count use
  // an empty resource (zero rows, dropped stores) and get routing weight 0, so there are no
  // per-source branches and the wait counts stay exact across the token loop.
  Chunk rows[SB][CH];

  // Token schedule (single-block path with a counter): tokens go out in batches of B = a.tpt
  // consecutive tokens. Workgroup g starts with batch g; each later batch is grid + a ticket from
  // the device-wide counter, so workgroups that run faster take more batches and all finish
  // together (B > 1 divides the counter's traffic, which is served one atomic at a time). Thread
  // 0 takes the ticket at the top of a batch's last token and publishes it through LDS at the
  // barrier that ends that token's exchange. Otherwise tokens are strided by the grid.
  const bool dyn = ONE && a.ticket != nullptr;
  const int64_t B = dyn ? a.tpt : 1;
  const int64_t n0 = (int64_t)blockIdx.x * B;
  // multi-block path: the following block's rows, loaded while the current block is processed
  Chunk nxt[ONE ? 1 : SB][CH];
  if constexpr (!ONE) {
    const int nb0 = n0 < a.N ? min(SB, a.S) : 0;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const Rsrc r = src_rsrc(a.src[i], i, nb0, n0 * a.row_stride * ESZ, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) rows[i][j] = ld_row(r, cs.voff[j]);
    }
  }

  if constexpr (ONE) {
    // issued in the loop body's order (rows 0..SB-1) so the wait counts at the loop head stay
    // tight over both entry paths
    const int live = n0 < a.N ? a.S : 0;
    const int64_t row_byte = n0 * a.row_stride * ESZ;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const Rsrc r = src_rsrc(a.src[i], i, live, row_byte, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) rows[i][j] = ld_row(r, cs.voff[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // as many dropped stores (empty resource) as the output row the loop body stores after its
    // last row load: the wait for the last row at the loop head then lets the previous token's
    // output stores stay in flight (the wait is the minimum over both entry paths)
    const Rsrc none = row_rsrc(nullptr, 0, 0u);
    const Chunk zero = {};
#pragma unroll
    for (int j = 0; j < CH; ++j) st_row(none, cs.voff[j], zero);
  }

  uint32_t* tslot = reinterpret_cast<uint32_t*>(lds + 2 * xfl);
  int64_t n = n0, batch_end = n0 + B;
  while (n < a.N) {
    const bool take = dyn && n + 1 >= batch_end;  // last token of its batch
    uint32_t tk = 0;
    if (take && tid == 0) tk = atomicAdd(a.ticket + kCtrTicket, 1u);
    int64_t next = dyn ? n + 1 : n + gridDim.x;
    float acc[CH][VEC];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[j][e] = 0.f;
    float m = -INFINITY, l = 0.f;

    for (int s0 = 0; s0 < (ONE ? 1 : a.S); s0 += SB) {
      const int nb = ONE ? a.S : min(SB, a.S - s0);
      if constexpr (!ONE) {
        // the following block: this token's next one, or the next token's first (static split:
        // the next token is known); the same loads on every path (empty past the last token)
        const bool last = s0 + SB >= a.S;
        const int64_t tok = last ? next : n;
        const int f0 = last ? 0 : s0 + SB;
        const int nbf = (tok < a.N) ? min(SB, a.S - f0) : 0;
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          const Rsrc r = src_rsrc(a.src[min(f0 + i, kMaxSources - 1)], i, nbf,
                                  tok * a.row_stride * ESZ, row_bytes);
#pragma unroll
          for (int j = 0; j < CH; ++j) nxt[i][j] = ld_row(r, cs.voff[j]);
        }
      }
      float* xb = lds + buf * xfl;
      uint32_t us[3][CH][4];
      float u[CH][VEC];
      if constexpr (BF16) cs.fetch_us(laundered_lane_off(tid), us);
      else cs.fetch_u(laundered_lane_off(tid), u);
#pragma unroll
      for (int i0 = 0; i0 < SB; i0 += kGroup) {
        float part[2][kGroup];
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
          part[0][g] = part[1][g] = 0.f;
          if (i0 + g < SB)
            key_sums<BF16, CH, FULL>(rows[i0 + g], cs, us, u, a.lo, part[0][g], part[1][g]);
        }
        xchg_group<2, SB>(part, i0, xb, R4, tid);
      }
      if (take && tid == 0) tslot[buf] = tk;
      __syncthreads();
      if (take) {
        next = ((int64_t)gridDim.x + (int64_t)__builtin_amdgcn_readfirstlane(tslot[buf])) * B;
        batch_end = next + B;
      }
      buf ^= 1;
      float z = -INFINITY;
      if (lane < nb) {
        const float ss = xchg_total(xb, lane, R4);
        const float c = xchg_total(xb, SB + lane, R4);
        z = source_score(ss, c, a.inv_R, a.eps, a.scale).z;
      }
      const float m_new = fmaxf(m, wave_max(z));
      float ez = (lane < nb) ? expf(z - m_new) : 0.f;
      const float lb = wave_sum(ez);
      if constexpr (ONE) {
        l = lb;
        ez = ez / lb;  // the routing weight itself: acc becomes o directly
      } else {
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
      }
      m = m_new;
      // raised wave priority while the mixture is folded in and the next token's rows and this
      // token's output go out: waves issuing memory operations go ahead of waves in the
      // exchange (measured 0.8% on the forward at S = 10, D = 4096)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const float pi = bcast(ez, i);
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[j][e] = fmaf(pi, elem<BF16>(rows[i][j], e), acc[j][e]);
        if constexpr (ONE) {
          // the next token's row i (an empty resource past the last token)
          const Rsrc r = src_rsrc(a.src[i], i, next < a.N ? a.S : 0, next * a.row_stride * ESZ,
                                  row_bytes);
#pragma unroll
          for (int j = 0; j < CH; ++j) rows[i][j] = ld_row(r, cs.voff[j]);
        }
      }
      if constexpr (!ONE) {
#pragma unroll
        for (int i = 0; i < SB; ++i)
#pragma unroll
          for (int j = 0; j < CH; ++j) rows[i][j] = nxt[i][j];
      }
    }
    if constexpr (!ONE) {
      const float inv_l = 1.f / l;
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[j][e] *= inv_l;  // acc now holds o
    }
    fwd_emit<BF16, CH, FULL>(a, cs, acc, ow, n, m + logf(l), lds, buf, xfl, R4, tid, row_bytes);
    __builtin_amdgcn_s_setprio(0);
    n = next;
  }
  if (dyn) fwd_release_counters(a.ticket, tid);
}

// ------------------------------------------------------------------ backward, shared tail

// Writes this thread's columns of one FP32 partial row (du at absolute columns [lo, D), dow at
// [D, 2D) when `with_dow`) with 16-byte stores, then clears the sums. Chunks that start below the
// key slice carry zeros there (du only accumulates slice columns), so whole chunks are written.
template <bool BF16, int CH, bool FULL>
__device__ __forceinline__ void store_row(const BwdArgs& a, const Cols<BF16, CH, FULL>& cs,
                                          float (&du)[CH][Fmt<BF16>::VEC],
                                          float (&dow)[CH][Fmt<BF16>::VEC], int64_t row,
                                          bool with_dow) {
  constexpr int VEC = Fmt<BF16>::VEC;
  float* pr = static_cast<float*>(a.part) + row * a.wc;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    if (!cs.valid[j]) continue;
    if (FULL || cs.col0[j] + VEC > a.lo)
#pragma unroll
      for (int h = 0; h < VEC; h += 4)
        st_f32x4(pr + cs.col0[j] + h, du[j][h], du[j][h + 1], du[j][h + 2], du[j][h + 3]);
    if (with_dow)
#pragma unroll
      for (int h = 0; h < VEC; h += 4)
        st_f32x4(pr + a.D + cs.col0[j] + h, dow[j][h], dow[j][h + 1], dow[j][h + 2],
                 dow[j][h + 3]);
  }
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int e = 0; e < VEC; ++e) du[j][e] = dow[j][e] = 0.f;
}

// Adds one batch's FP32 contribution of every column to the exact bins (kBinMagicA/B) and clears
// it. With contraction off no step is fused: each rounding below is the one the bins rely on.
template <int CH, int VEC>
__device__ __forceinline__ void bin_token(float (&c)[CH][VEC], double (&ba)[CH][VEC],
                                          double (&bb)[CH][VEC]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const double x = static_cast<double>(c[j][e]);
      const double xa = (x + kBinMagicA) - kBinMagicA;  // multiple of 2^-20 (|x| < 2^31)
      const double xb = ((x - xa) + kBinMagicB) - kBinMagicB;  // remainder to 2^-53
      ba[j][e] += xa;
      bb[j][e] += xb;
      c[j][e] = 0.f;
    }
}

// Writes this thread's columns of the workgroup's binned partial row (bin A at [row][0][col], bin
// B at [row][1][col]) with 16-byte stores.
template <bool BF16, int CH, bool FULL>
__device__ __forceinline__ void store_bins(const BwdArgs& a, const Cols<BF16, CH, FULL>& cs,
                                           const double (&ba)[CH][Fmt<BF16>::VEC],
                                           const double (&bb)[CH][Fmt<BF16>::VEC], int64_t row) {
  constexpr int VEC = Fmt<BF16>::VEC;
  typedef double f64x2 __attribute__((ext_vector_type(2)));
  double* pa = static_cast<double*>(a.part) + row * 2 * a.wc;
  double* pb = pa + a.wc;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    if (!cs.valid[j] || !(FULL || cs.col0[j] + VEC > a.lo)) continue;
#pragma unroll
    for (int h = 0; h < VEC; h += 2) {
      const f64x2 va = {ba[j][h], ba[j][h + 1]};
      const f64x2 vb = {bb[j][h], bb[j][h + 1]};
      *reinterpret_cast<f64x2*>(pa + cs.col0[j] + h) = va;
      *reinterpret_cast<f64x2*>(pb + cs.col0[j] + h) = vb;
    }
  }
}

// ------------------------------------------------------------------ backward, token-resident

// All S <= SB rows of a token stay in VGPRs: delta = sum_s p_s <dY, v_s> is exact in FP32.
// No output norm on this path (dL/do = dY). ACC: dvalues accumulate (the existing gradient rows
// are prefetched one token ahead like the source rows and added before the store).
// Two waves per SIMD: the grid holds two 4-wave workgroups per CU (more measured slower), and the
// row slab, the exact FP64 bins and the pipelined loads need the registers of that occupancy.
// BIN: the q/w gradient sums go through exact FP64 bins per batch (the same bits whatever tokens
// the counter hands out); without it the workgroup keeps one FP32 running sum over all its tokens
// and writes it as an FP32 row (faster; bitwise reproducible only under a static split).
template <bool BF16, int CH, int SB, bool FULL, bool ACC, bool BIN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 8)))
void bwd_resident_kernel(const BwdArgs a) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int K = 3 * SB;
  extern __shared__ float lds_all[];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
  const int R4 = nthr >> 4;
  const int xfl = K * R4;
  const uint32_t row_bytes = static_cast<uint32_t>(a.D * ESZ);

  Cols<BF16, CH, FULL> cs;
  cs.init(tid, nthr, a.D, a.lo, a.query, a.norm_w, lds_all);
  float* lds = lds_all + Cols<BF16, CH, FULL>::param_bytes(nthr) / 4;  // exchange buffers
  float du[CH][VEC], dow[CH][VEC];
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int e = 0; e < VEC; ++e) du[j][e] = dow[j][e] = 0.f;
  const int S = a.S;
  int buf = 0;

  // Software pipeline over tokens: the next token's dY row is loaded once this token's has been
  // widened, and its source row i once row i's gradient has been stored, so the loads overlap
  // this token's math and stores, and the next token's first wait covers only what was issued
  // before its own loads (the vector-memory counter retires loads and stores in order).
  // Loops run over all SB slots; slots i >= S use an empty resource (zero rows, dropped stores)
  // and get routing weight 0, so there are no per-source branches and the wait counts stay exact.
  Chunk rows[SB][CH];
  Chunk odv[ACC ? SB : 1][CH];  // ACC: the existing dvalues rows of the current token
  Chunk gy[CH];
  // Token schedule (BwdArgs): head batches g, g + P, ... below hb_end, then batches from the
  // ticket counter as this workgroup finishes, so faster workgroups take more of them and all
  // finish together (the two workgroups that share a CU run at unequal speeds, so a static split
  // leaves one of them working alone at the end). Thread 0 takes the ticket at the top of a
  // batch's last token; its latency hides behind pass 1, and it is published through LDS at the
  // barrier pass 1 ends with.
  const int64_t P = gridDim.x;
  const bool dyn = a.hb_end < a.nbatch;
  int64_t b = blockIdx.x;
  const int64_t n0 = b < a.nbatch ? b * a.tpt : a.N;
  // exact bins of this workgroup's q/w gradient sums (kBinMagicA/B): whatever tokens the counter
  // hands this workgroup, the merged sums are the same
  double ba[CH][VEC], bb[CH][VEC];
  if constexpr (BIN) {
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) ba[j][e] = bb[j][e] = 0.0;
  }
  // lse of the current token; the next one is loaded with the next token's rows (a vector load
  // waited for at its use would otherwise also drain every store issued before it)
  float lse = n0 < a.N ? a.lse[n0] : 0.f;
  {
    // issued in the order the loop body issues the next token's loads (dY, then rows 0..SB-1):
    // the wait counts at the loop head are the minimum over both entry paths
    const int live = n0 < a.N ? S : 0;
    const Rsrc rg = src_rsrc(a.dout, 0, live, n0 * a.dout_stride * ESZ, row_bytes);
#pragma unroll
    for (int j = 0; j < CH; ++j) gy[j] = ld_row(rg, cs.voff[j]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const Rsrc r = src_rsrc(a.src[i], i, live, n0 * a.row_stride * ESZ, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) rows[i][j] = ld_row(r, cs.voff[j]);
      if constexpr (ACC) {
        const Rsrc rd = src_rsrc(a.dsrc[i], i, live, n0 * a.drow_stride * ESZ, row_bytes);
#pragma unroll
        for (int j = 0; j < CH; ++j) odv[i][j] = ld_row(rd, cs.voff[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  uint32_t* tslot = reinterpret_cast<uint32_t*>(lds + 2 * xfl);
  int64_t n = n0, batch_end = min(n0 + a.tpt, a.N);
  while (n < a.N) {
    const bool last_tok = n + 1 >= batch_end;
    const bool in_tail = b >= a.hb_end;
    const bool head_more = !in_tail && b + P < a.hb_end;  // another head batch follows
    const bool take = dyn && last_tok && !head_more;
    uint32_t tk = 0;
    if (take && tid == 0) tk = atomicAdd(a.ctr + kCtrTicket, 1u);
    float* xb = lds + buf * xfl;
    uint32_t us[3][CH][4];
    float u[CH][VEC];
    if constexpr (BF16) cs.fetch_us(laundered_lane_off(tid), us);
    else cs.fetch_u(laundered_lane_off(tid), u);
#pragma unroll
    for (int i0 = 0; i0 < SB; i0 += kGroup) {
      float part[3][kGroup];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        part[0][g] = part[1][g] = part[2][g] = 0.f;
        if (i0 + g < SB) {
          key_sums<BF16, CH, FULL>(rows[i0 + g], cs, us, u, a.lo, part[0][g], part[1][g]);
          part[2][g] = dot_rows<BF16, CH>(rows[i0 + g], gy);
        }
      }
      xchg_group<3, SB>(part, i0, xb, R4, tid);
    }
    if (take && tid == 0) tslot[buf] = tk;
    __syncthreads();
    int64_t next = n + 1, b_next = b;
    if (last_tok) {
      if (head_more) b_next = b + P;
      else if (take) b_next = a.hb_end + (int64_t)__builtin_amdgcn_readfirstlane(tslot[buf]);
      else b_next = a.nbatch;
      next = b_next < a.nbatch ? b_next * a.tpt : a.N;
    }
    const bool has_next = next < a.N;
    buf ^= 1;

    // lane s finishes source s
    float p = 0.f, dp = 0.f, rho = 0.f, c = 0.f;
    if (lane < S) {
      const float ss = xchg_total(xb, lane, R4);
      c = xchg_total(xb, SB + lane, R4);
      dp = xchg_total(xb, 2 * SB + lane, R4);
      const Score sc = source_score(ss, c, a.inv_R, a.eps, a.scale);
      rho = sc.rho;
      p = routing_weight(sc.z, lse);
    }
    const float delta = wave_sum(p * dp);
    const float A = a.scale * p * (dp - delta) * rho;
    const float B = -A * rho * rho * c * a.inv_R;

    float dof[CH][VEC];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) dof[j][e] = elem<BF16>(gy[j], e);
    const int live_next = has_next ? S : 0;
    const float lse_next = a.lse[has_next ? next : n];
    {
      // the next token's dY row (an empty resource past the last token)
      const Rsrc rg = src_rsrc(a.dout, 0, live_next, next * a.dout_stride * ESZ, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) gy[j] = ld_row(rg, cs.voff[j]);
    }
    const int64_t drow_byte = n * a.drow_stride * ESZ;
    const int64_t next_byte = next * a.row_stride * ESZ;
    const int64_t next_dbyte = next * a.drow_stride * ESZ;
    cs.fetch_u(laundered_lane_off(tid), u);
    // raised wave priority while the gradient rows are stored and the next token's rows loaded:
    // waves issuing memory operations go ahead of waves in the exchange (measured 1.4% on the
    // backward at S = 10, D = 4096, 1.1% accumulating; priority 3 measured the same as 1). Not
    // when accumulating with a sliced key: that kernel then spilled more (+2.2% time).
    constexpr bool kPrio = FULL || !ACC;
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      Chunk out[CH];
      grad_row<BF16, CH, FULL, ACC>(rows[i], cs, u, dof, bcast(p, i), bcast(A, i), bcast(B, i),
                                    a.lo, du, out, odv[ACC ? i : 0]);
      const Rsrc rd = src_rsrc(a.dsrc[i], i, S, drow_byte, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) st_row(rd, cs.voff[j], out[j]);
      const Rsrc r = src_rsrc(a.src[i], i, live_next, next_byte, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) rows[i][j] = ld_row(r, cs.voff[j]);
      if constexpr (ACC) {
        // the next token's existing gradient row i (issued after this token's row i is stored)
        const Rsrc rn = src_rsrc(a.dsrc[i], i, live_next, next_dbyte, row_bytes);
#pragma unroll
        for (int j = 0; j < CH; ++j) odv[i][j] = ld_row(rn, cs.voff[j]);
      }
    }
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
    // a batch is a fixed token set summed in token order, so its FP32 sum is binned once
    if constexpr (BIN) {
      if (last_tok) bin_token<CH, VEC>(du, ba, bb);
    }
    if (last_tok) {
      b = b_next;
      batch_end = min(next + a.tpt, a.N);
    }
    lse = lse_next;
    n = next;
  }
  if constexpr (BIN) store_bins<BF16, CH, FULL>(a, cs, ba, bb, blockIdx.x);
  else store_row<BF16, CH, FULL>(a, cs, du, dow, blockIdx.x, false);
}

// ------------------------------------------------------------------ backward, streaming

// Sources walked in blocks of SB using the forward's FP32 mixture o (and rho_o with the output
// norm): do and delta = <do, o> are known before the first source is read. Blocks are
// double-buffered: block b+1's rows (and, during a token's last block, the next token's dY, o and
// block 0) are loaded while block b is reduced and its gradients stored; every block issues the
// same loads (empty resources where there is nothing to load), so the wait counts are the same
// on every path. Tokens come in batches from the device-wide counter like the resident kernels.
// ACC: dvalues accumulate (a block's existing gradient rows are loaded with its source rows).
template <bool BF16, int CH, int SB, bool FULL, bool ACC>
__global__ __launch_bounds__(512) void bwd_stream_kernel(const BwdArgs a) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int K = 3 * SB;
  constexpr int OC = VEC / 4;  // 16-byte chunks of the FP32 mixture per row chunk
  extern __shared__ float lds_all[];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
  const int R4 = nthr >> 4;
  const int xfl = K * R4;
  const uint32_t row_bytes = static_cast<uint32_t>(a.D * ESZ);
  const uint32_t o_bytes = static_cast<uint32_t>(a.D * 4);

  Cols<BF16, CH, FULL> cs;
  cs.init(tid, nthr, a.D, a.lo, a.query, a.norm_w, lds_all);
  float* lds = lds_all + Cols<BF16, CH, FULL>::param_bytes(nthr) / 4;  // exchange buffers
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
  const int nblk = (a.S + SB - 1) / SB;

  // token schedule (BwdArgs): head batches summed into row g, each tail batch into its own row
  const int64_t P = gridDim.x;
  const bool dyn = a.hb_end < a.nbatch;
  int64_t b = blockIdx.x;
  const int64_t n0 = b < a.nbatch ? b * a.tpt : a.N;
  bool head_open = true;

  // a token's head (dY row and FP32 mixture row) and one source block's rows (+ existing grads)
  Chunk g[CH], oc[CH][OC];
  Chunk cur[SB][CH], nxt[SB][CH];
  Chunk odc[ACC ? SB : 1][CH], odn[ACC ? SB : 1][CH];
  auto load_head = [&](int64_t tok, bool live) {
    const Rsrc rg = row_rsrc(live ? a.dout : nullptr, live ? tok * a.dout_stride * ESZ : 0,
                             live ? row_bytes : 0u);
    const Rsrc ro = row_rsrc(live ? a.o32 : nullptr, live ? tok * a.D * 4 : 0, live ? o_bytes : 0u);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      g[j] = ld_row(rg, cs.voff[j]);
#pragma unroll
      for (int h = 0; h < OC; ++h)
        oc[j][h] = ld_row(ro, static_cast<uint32_t>((cs.col0[j] + 4 * h) * 4));
    }
  };
  auto load_block = [&](Chunk (&rows)[SB][CH], Chunk (&od)[ACC ? SB : 1][CH], int64_t tok,
                        int s0, bool live) {
    const int nb = live ? min(SB, a.S - s0) : 0;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int s = min(s0 + i, kMaxSources - 1);
      const Rsrc r = src_rsrc(a.src[s], i, nb, tok * a.row_stride * ESZ, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) rows[i][j] = ld_row(r, cs.voff[j]);
      if constexpr (ACC) {
        const Rsrc rd = src_rsrc(a.dsrc[s], i, nb, tok * a.drow_stride * ESZ, row_bytes);
#pragma unroll
        for (int j = 0; j < CH; ++j) od[i][j] = ld_row(rd, cs.voff[j]);
      }
    }
  };
  load_head(n0, n0 < a.N);
  load_block(cur, odc, n0, 0, n0 < a.N);

  uint32_t* tslot = reinterpret_cast<uint32_t*>(lds + 2 * xfl);
  int64_t n = n0, batch_end = min(n0 + a.tpt, a.N);
  while (n < a.N) {
    const bool last_tok = n + 1 >= batch_end;
    const bool in_tail = b >= a.hb_end;
    const bool head_more = !in_tail && b + P < a.hb_end;
    const bool take = dyn && last_tok && !head_more;
    uint32_t tk = 0;
    if (take && tid == 0) tk = atomicAdd(a.ctr + kCtrTicket, 1u);
    int64_t next = n + 1, b_next = b;

    float dov[CH][VEC], o[CH][VEC];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
#pragma unroll
      for (int h = 0; h < OC; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[j][4 * h + e] = bits_f(oc[j][h].w[e]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) dov[j][e] = elem<BF16>(g[j], e);
    }
    // do and delta = <do, o>; the ticket rides on this exchange's barrier
    float delta;
    {
      float part[2][kGroup] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      if (a.out_norm) {
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            part[0][0] = fmaf(dov[j][e] * ow[j][e], o[j][e], part[0][0]);  // <g, o>
            part[1][0] = fmaf(o[j][e], o[j][e], part[1][0]);                // <o, o>
          }
      } else {
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) part[0][0] = fmaf(dov[j][e], o[j][e], part[0][0]);
      }
      float* xb = lds + buf * xfl;
      xchg_group<2, 1>(part, 0, xb, R4, tid);
      if (take && tid == 0) tslot[buf] = tk;
      __syncthreads();
      if (last_tok) {
        if (head_more) b_next = b + P;
        else if (take) b_next = a.hb_end + (int64_t)__builtin_amdgcn_readfirstlane(tslot[buf]);
        else b_next = a.nbatch;
        next = b_next < a.nbatch ? b_next * a.tpt : a.N;
      }
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
    const int64_t drow_byte = n * a.drow_stride * ESZ;
    const bool live_next = next < a.N;

    for (int b = 0; b < nblk; ++b) {
      const int s0 = b * SB;
      const int nb = min(SB, a.S - s0);
      const bool last = b + 1 == nblk;
      // the following block: this token's next one, or the next token's first (with its head)
      load_head(next, last && live_next);
      load_block(nxt, odn, last ? next : n, last ? 0 : s0 + SB, last ? live_next : true);

      float* xb = lds + buf * xfl;
      uint32_t us[3][CH][4];
      float u[CH][VEC];
      if constexpr (BF16) cs.fetch_us(laundered_lane_off(tid), us);
      else cs.fetch_u(laundered_lane_off(tid), u);
#pragma unroll
      for (int i0 = 0; i0 < SB; i0 += kGroup) {
        float part[3][kGroup];
#pragma unroll
        for (int gi = 0; gi < kGroup; ++gi) {
          part[0][gi] = part[1][gi] = part[2][gi] = 0.f;
          if (i0 + gi < SB) {
            key_sums<BF16, CH, FULL>(cur[i0 + gi], cs, us, u, a.lo, part[0][gi], part[1][gi]);
            part[2][gi] = dot_f32<BF16, CH>(cur[i0 + gi], dov);
          }
        }
        xchg_group<3, SB>(part, i0, xb, R4, tid);
      }
      __syncthreads();
      buf ^= 1;
      float p = 0.f, dp = 0.f, rho = 0.f, c = 0.f;
      if (lane < nb) {
        const float ss = xchg_total(xb, lane, R4);
        c = xchg_total(xb, SB + lane, R4);
        dp = xchg_total(xb, 2 * SB + lane, R4);
        const Score sc = source_score(ss, c, a.inv_R, a.eps, a.scale);
        rho = sc.rho;
        p = routing_weight(sc.z, lse);
      }
      const float A = a.scale * p * (dp - delta) * rho;
      const float Bc = -A * rho * rho * c * a.inv_R;
      cs.fetch_u(laundered_lane_off(tid), u);
      // raised wave priority while the block's gradient rows are stored (measured 0.8% on the
      // S = 64, D = 8192 output-norm backward; raising it around the block loads was slower)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        Chunk out[CH];
        grad_row<BF16, CH, FULL, ACC>(cur[i], cs, u, dov, bcast(p, i), bcast(A, i), bcast(Bc, i),
                                      a.lo, du, out, odc[ACC ? i : 0]);
        const Rsrc rd =
            src_rsrc(a.dsrc[min(s0 + i, kMaxSources - 1)], i, nb, drow_byte, row_bytes);
#pragma unroll
        for (int j = 0; j < CH; ++j) st_row(rd, cs.voff[j], out[j]);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int i = 0; i < SB; ++i)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          cur[i][j] = nxt[i][j];
          if constexpr (ACC) odc[i][j] = odn[i][j];
        }
    }
    if (last_tok && !head_more) {
      store_row<BF16, CH, FULL>(a, cs, du, dow, in_tail ? P + (b - a.hb_end) : (int64_t)blockIdx.x,
                                a.out_w != nullptr);
      head_open = head_open && in_tail;
    }
    if (last_tok) {
      b = b_next;
      batch_end = min(next + a.tpt, a.N);
    }
    n = next;
  }
  if (head_open) store_row<BF16, CH, FULL>(a, cs, du, dow, blockIdx.x, a.out_w != nullptr);
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

// Single-query finaliser: a workgroup owns kFinRowsCols columns; thread (phase r, column c) adds
// rows r, r + kFinRowsPhases, ... in FP64 (for binned rows bins A and B separately), the phase sums
// are added in phase order through LDS, then dq = du * w (du without w), dw = du * q and dow are
// written. Binned sums are exact, so the result does not depend on the order; FP32 rows are summed
// in the same fixed order every call. Block 0 returns the backward's ticket counter to zero (this
// kernel runs after the backward).
template <bool BF16>
__global__ __launch_bounds__(kFinRowsCols * kFinRowsPhases) void finalize_rows_kernel(
    const FinRowsArgs a) {
  __shared__ double red[2][kFinRowsPhases][kFinRowsCols];
  const int cl = threadIdx.x % kFinRowsCols, ph = threadIdx.x / kFinRowsCols;
  const int c = blockIdx.x * kFinRowsCols + cl;
  const bool has = c < a.cols;
  const int col = c < a.R ? a.lo + c : a.D + (c - a.R);  // partial-row column
  double sa = 0.0, sb = 0.0;
  if (has) {
    if (a.binned) {
      const double* pa = static_cast<const double*>(a.part) + col;
#pragma unroll 4
      for (int r = ph; r < a.rows; r += kFinRowsPhases) {
        sa += pa[(int64_t)r * 2 * a.wc];
        sb += pa[(int64_t)r * 2 * a.wc + a.wc];
      }
    } else {
      const float* pf = static_cast<const float*>(a.part) + col;
#pragma unroll 4
      for (int r = ph; r < a.rows; r += kFinRowsPhases)
        sa += static_cast<double>(pf[(int64_t)r * a.wc]);
    }
  }
  red[0][ph][cl] = sa;
  red[1][ph][cl] = sb;
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.ctr[kCtrTicket] = 0u;
    a.ctr[kCtrArrive] = 0u;
  }
  if (ph != 0 || !has) return;
  double ta = 0.0, tb = 0.0;
#pragma unroll
  for (int r = 0; r < kFinRowsPhases; ++r) {
    ta += red[0][r][cl];
    tb += red[1][r][cl];
  }
  const float total = static_cast<float>(ta + tb);
  if (c < a.R) {
    const float wv = a.norm_w ? load_param<BF16>(a.norm_w, c) : 1.f;
    store_param<BF16>(a.dq, c, total * wv);
    if (a.norm_w) store_param<BF16>(a.dw, c, total * load_param<BF16>(a.query, c));
  } else {
    store_param<BF16>(a.dow, c - a.R, total);
  }
}

}  // namespace attnres
