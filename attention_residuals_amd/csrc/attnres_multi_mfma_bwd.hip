// attnres_multi_mfma_bwd.hip -- multi-query backward through matrix cores (gfx950, bf16 storage).
//
// Operation ("Fast Attention Residuals" PyPI page, section "Multi-query AttnRes"): M queries read
// the same S sources, p_{m,s} = softmax_s(scale * rho_s * <t_s, q_m>), y_m = sum_s p_{m,s} v_s.
// With dY_m = dL/dy_m, c_{m,s} = <t_s, q_m>, dp_{m,s} = <dY_m, v_s>:
//   delta_m = sum_s p_{m,s} dp_{m,s};  a_{m,s} = scale * p_{m,s} (dp_{m,s} - delta_m) * rho_s
//   dv_s = sum_m p_{m,s} dY_m + [key slice] (sum_m a_{m,s} q_m + B_s t_s),
//   B_s = -rho_s^2 / R * sum_m a_{m,s} c_{m,s};   dq_m = sum_{n,s} a_{m,s} t_s.
// All M <= 16 queries in one pass over the sources: dvalues are written (and rounded) once.
//
// Kernel 1 (multi_bwd_mfma_kernel): one 8-wave workgroup per CU owns one token at a time. Rows sit
// in the matrix-core forward's layout: lane (g, c) of a wave holds, per 128-column group, the
// 16-byte chunk c of sources 4g .. 4g+3 and of the dY rows of queries 4g .. 4g+3.
//   * The contractions over columns (c, dp and the key sums of squares) run on matrix cores too:
//     each wave copies one 32-column block of its source and dY rows to a small LDS staging area
//     and reads it back with row = lane % 16, columns 4 * (lane / 16) .. + 3, which is the operand
//     layout of a 16x16x16 MFMA whose contraction index is the column; the staged queries come
//     from LDS in the same way. Per block: scores = Q V^T, dp = dY V^T, sum t^2 = diag(V V^T).
//   * One LDS exchange sums the 8 waves' 16 x 16 tiles; 256 threads then finish one (m, s) pair
//     each (routing weight from the saved lse, delta by a 16-lane row sum, a, and the B terms),
//     write a_{m,s} to the coefficient array and p, a to LDS.
//   * dv = P^T dY + A^T Q (two MFMA contractions over the queries, weights as two bf16 terms) plus
//     B_s t_s on the vector ALU, rounded once to bf16 (with accumulate: added to the existing row
//     first); the next token's rows of a column group load as soon as its dv is done.
// Kernel 2 (multi_dq_mfma_kernel): dq_m[j] = sum_n sum_s a_{m,s,n} t_{s,n}[j] over a static token
// range per workgroup (16x16x16 MFMAs with the sources as the contraction index), one FP32 partial
// row per range; the finaliser sums the ranges in a fixed order.
#include "attnres_internal.hpp"
#include "attnres_kernels.hpp"

namespace attnres {
namespace {

typedef short mb_short4 __attribute__((ext_vector_type(4)));
typedef float mb_float4 __attribute__((ext_vector_type(4)));
typedef uint32_t mb_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t mb_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Chunk bnt_load16(const char* p) {
  return __builtin_bit_cast(Chunk,
                            __builtin_nontemporal_load(reinterpret_cast<const mb_u32x4*>(p)));
}
__device__ __forceinline__ void bnt_store16(char* p, const Chunk& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(mb_u32x4, v), reinterpret_cast<mb_u32x4*>(p));
}

// {a.low, b.low} / {a.high, b.high} of two words (v_perm_b32)
__device__ __forceinline__ uint32_t bpair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t bpair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// B operand of element e of a chunk from four rows (k = row, 4 bf16 per lane)
__device__ __forceinline__ mb_short4 gather_e(const Chunk (&r)[4], int e) {
  const int wi = e >> 1;
  const uint32_t b0 = (e & 1) ? bpair_hi(r[0].w[wi], r[1].w[wi]) : bpair_lo(r[0].w[wi], r[1].w[wi]);
  const uint32_t b1 = (e & 1) ? bpair_hi(r[2].w[wi], r[3].w[wi]) : bpair_lo(r[2].w[wi], r[3].w[wi]);
  return __builtin_bit_cast(mb_short4, mb_u32x2{b0, b1});
}

// Four FP32 weights as an A operand in two bf16 terms (w = hi + lo, ~16 bits kept)
__device__ __forceinline__ void split_a(const float (&w)[4], mb_short4& hi, mb_short4& lo) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    h[i] = pack_bf16x2(w[2 * i], w[2 * i + 1]);
    l[i] = pack_bf16x2(w[2 * i] - lo_f(h[i]), w[2 * i + 1] - hi_f(h[i]));
  }
  hi = __builtin_bit_cast(mb_short4, mb_u32x2{h[0], h[1]});
  lo = __builtin_bit_cast(mb_short4, mb_u32x2{l[0], l[1]});
}

__device__ __forceinline__ mb_short4 ld8(const char* p) {
  return __builtin_bit_cast(mb_short4, *reinterpret_cast<const mb_u32x2*>(p));
}

// Sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the same lane of the wave's four DPP rows).
__device__ __forceinline__ float rows4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  x = bits_f(a[0]) + bits_f(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return bits_f(b[0]) + bits_f(b[1]);
}

// Lanes of one wave pass data through LDS here with no workgroup barrier between the write and
// the read. The hardware completes a wave's LDS operations in issue order, but the compiler sees
// only one lane: without a fence it may reuse a value it loaded earlier from the same address (a
// lane that did not store assumes the memory unchanged) or move a store above another lane's read.
// A wavefront-scope fence orders them for the compiler and emits no instruction.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

constexpr int kStageRow = 80;                    // bytes per staged row (64 + pad: no conflicts)
constexpr int kWaveRegion = 32 * kStageRow;      // 16 source + 16 dY rows of one 32-column block
constexpr int kXchFloats = 2 * 256 + 16;         // scores, dp tiles and the 16 sums of squares

}  // namespace

size_t multi_bwd_mfma_lds(int cgw, int M) {
  return (size_t)M * kMfmaWaves * cgw * 16 * 16 + (size_t)kMfmaWaves * kWaveRegion +
         (2 * 256 + 4 * 16) * sizeof(float);
}

template <int CGW, bool FULL, bool ACC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 8)))
void multi_bwd_mfma_kernel(const MfmaBwdArgs a) {
  constexpr int W = kMfmaWaves;
  constexpr int NQ = W * CGW * 16;  // 16-byte chunks of a row the workgroup covers
  extern __shared__ float lds[];
  Chunk* qlds = reinterpret_cast<Chunk*>(lds);  // [M][NQ] staged queries
  char* regions = reinterpret_cast<char*>(lds) + (size_t)a.M * NQ * 16;
  float* pa = reinterpret_cast<float*>(regions + W * kWaveRegion);  // p[16][16], a[16][16]
  float* bpart = pa + 512;                                           // [4][16] partial B sums
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  char* stage = regions + wave * kWaveRegion;
  float* xw = reinterpret_cast<float*>(stage);  // the wave's exchange (after its blocks)

  // queries as bf16 chunks of full-width rows, zero outside the key slice [lo, D)
  const uint16_t* qsrc = static_cast<const uint16_t*>(a.query);
  for (int idx = tid; idx < a.M * NQ; idx += W * 64) {
    const int m = idx / NQ, q = idx - m * NQ;
    Chunk v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int col = q * 8 + 2 * i + k;
        h[k] = (col >= a.lo && col < a.D) ? static_cast<uint32_t>(qsrc[(int64_t)m * a.R + (col - a.lo)])
                                          : 0u;
      }
      v.w[i] = h[0] | (h[1] << 16);
    }
    qlds[idx] = v;
  }

  // this lane's sources 4g + j and dY rows of queries 4g + j
  const char* vbase[4];
  bool vlive[4], glive[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vlive[j] = 4 * g + j < a.S;
    glive[j] = 4 * g + j < a.M;
    vbase[j] = static_cast<const char*>(vlive[j] ? a.src[4 * g + j] : nullptr);
  }
  const char* gbase = static_cast<const char*>(a.dout);
  int qidx[CGW];
  bool qok[CGW];
#pragma unroll
  for (int cg = 0; cg < CGW; ++cg) {
    qidx[cg] = (wave * CGW + cg) * 16 + c;
    qok[cg] = qidx[cg] * 8 < a.D;
  }
  // key-slice masks of the chunks' bf16 halves (columns >= lo) for the B t terms
  uint32_t gm[FULL ? 1 : CGW][4];
  if constexpr (!FULL) {
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col0 = qidx[cg] * 8 + 2 * i;
        gm[cg][i] = (col0 >= a.lo ? 0x0000ffffu : 0u) | (col0 + 1 >= a.lo ? 0xffff0000u : 0u);
      }
  }
  __syncthreads();

  auto load_v = [&](Chunk (&r)[4], int cg, int64_t tok) {
    const int64_t off = tok * a.row_stride * 2 + (int64_t)qidx[cg] * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = (tok < a.N && vlive[j] && qok[cg]) ? bnt_load16(vbase[j] + off) : Chunk{};
  };
  auto load_g = [&](Chunk (&r)[4], int cg, int64_t tok) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = (tok < a.N && glive[j] && qok[cg])
                 ? bnt_load16(gbase + ((4 * g + j) * a.g_sm + tok * a.g_sn + (int64_t)qidx[cg] * 8) * 2)
                 : Chunk{};
  };
  auto load_old = [&](Chunk (&r)[4], int cg, int64_t tok) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = (vlive[j] && qok[cg])
                 ? bnt_load16(static_cast<const char*>(a.dsrc[4 * g + j]) + tok * a.drow_stride * 2 +
                              (int64_t)qidx[cg] * 16)
                 : Chunk{};
  };

  Chunk rows[CGW][4], gy[CGW][4];
  int64_t n = blockIdx.x;
#pragma unroll
  for (int cg = 0; cg < CGW; ++cg) {
    load_v(rows[cg], cg, n);
    load_g(gy[cg], cg, n);
  }
  const int pm = tid >> 4, ps = tid & 15;  // (query, source) finished by thread tid < 256
  while (n < a.N) {
    const int64_t next = n + gridDim.x;
    float lse_t = 0.f;
    if (tid < 256 && pm < a.M) lse_t = a.lse[pm * a.l_sm + n * a.l_sn];

    // ---- contractions over the columns: 32-column blocks through the staging area
    mb_float4 tsc = {0.f, 0.f, 0.f, 0.f}, tdp = tsc, tss = tsc;
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        wave_lds_order();  // the previous block's reads precede these writes
        if ((c >> 2) == blk) {
          char* dst = stage + (c & 3) * 16;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<Chunk*>(dst + (4 * g + j) * kStageRow) = rows[cg][j];
            *reinterpret_cast<Chunk*>(dst + (16 + 4 * g + j) * kStageRow) = gy[cg][j];
          }
        }
        wave_lds_order();  // the reads below see the other lanes' writes above
        const int chunk0 = (wave * CGW + cg) * 16 + 4 * blk;  // first chunk of the block
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int off = 32 * kb + 8 * g;  // byte offset of this lane's 4 columns in a row
          const mb_short4 vop = ld8(stage + c * kStageRow + off);
          const mb_short4 gop = ld8(stage + (16 + c) * kStageRow + off);
          const mb_short4 qop = (c < a.M)
              ? ld8(reinterpret_cast<const char*>(qlds + c * NQ + chunk0 + 2 * kb + (g >> 1)) +
                    (g & 1) * 8)
              : mb_short4{0, 0, 0, 0};
          mb_short4 vm = vop;
          if constexpr (!FULL) {
            const int col0 = chunk0 * 8 + 16 * kb + 4 * g;
            uint32_t w2[2];
            const mb_u32x2 raw = __builtin_bit_cast(mb_u32x2, vop);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const uint32_t mk = (col0 + 2 * i >= a.lo ? 0x0000ffffu : 0u) |
                                  (col0 + 2 * i + 1 >= a.lo ? 0xffff0000u : 0u);
              w2[i] = raw[i] & mk;
            }
            vm = __builtin_bit_cast(mb_short4, mb_u32x2{w2[0], w2[1]});
          }
          tsc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qop, vop, tsc, 0, 0, 0);
          tdp = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(gop, vop, tdp, 0, 0, 0);
          tss = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vm, vm, tss, 0, 0, 0);
        }
      }
    }
    // the wave's tiles into its exchange (over its staging area): lane (g, c) holds rows 4g + i,
    // column c
    wave_lds_order();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xw[(4 * g + i) * 16 + c] = tsc[i];
      xw[256 + (4 * g + i) * 16 + c] = tdp[i];
      if (4 * g + i == c) xw[512 + c] = tss[i];
    }
    __syncthreads();

    // ---- (query, source) pairs: routing weight, delta, a and the B terms
    if (tid < 256) {
      float sc = 0.f, dpv = 0.f, ss = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {  // wave order: a fixed summation order
        const float* x = reinterpret_cast<const float*>(regions + w * kWaveRegion);
        sc += x[pm * 16 + ps];
        dpv += x[256 + pm * 16 + ps];
        ss += x[512 + ps];
      }
      const bool valid = pm < a.M && ps < a.S;
      const Score scv = source_score(ss, sc, a.inv_R, a.eps, a.scale);
      const float p = valid ? routing_weight(scv.z, lse_t) : 0.f;
      const float delta = row_sum(p * dpv);
      const float av = a.scale * p * (dpv - delta) * scv.rho;
      const float bt = valid ? -av * scv.rho * scv.rho * sc * a.inv_R : 0.f;
      pa[pm * 16 + ps] = p;
      pa[256 + pm * 16 + ps] = av;
      a.coef[n * 256 + tid] = av;
      const float bs = rows4_sum(bt);  // over this wave's four queries
      if (lane < 16) bpart[wave * 16 + ps] = bs;
    }
    __syncthreads();

    // ---- dv = P^T dY + A^T Q + B t (one rounding to bf16)
    float pt[4], at[4], bsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pt[i] = pa[(4 * g + i) * 16 + c];
      at[i] = pa[256 + (4 * g + i) * 16 + c];
      bsrc[i] = ((bpart[4 * g + i] + bpart[16 + 4 * g + i]) + bpart[32 + 4 * g + i]) +
                bpart[48 + 4 * g + i];
    }
    mb_short4 p_hi, p_lo, a_hi, a_lo;
    split_a(pt, p_hi, p_lo);
    split_a(at, a_hi, a_lo);
    Chunk old[ACC ? 2 : 1][4];
    if constexpr (ACC) load_old(old[0], 0, n);
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) {
      if constexpr (ACC) {
        if (cg + 1 < CGW) load_old(old[(cg + 1) & 1], cg + 1, n);
      }
      Chunk qv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qv[i] = (4 * g + i < a.M) ? qlds[(4 * g + i) * NQ + qidx[cg]] : Chunk{};
      mb_float4 acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const mb_short4 bdy = gather_e(gy[cg], e);
        const mb_short4 bq = gather_e(qv, e);
        mb_float4 o = {0.f, 0.f, 0.f, 0.f};
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_hi, bdy, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_lo, bdy, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, bq, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, bq, o, 0, 0, 0);
        acc[e] = o;
      }
      load_g(gy[cg], cg, next);  // the MFMAs have read this column group's dY rows
      // lane (g, c) holds dv of source 4g + j at chunk qidx[cg], element e, in acc[e][j]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = FULL ? rows[cg][j].w[e >> 1] : (rows[cg][j].w[e >> 1] & gm[FULL ? 0 : cg][e >> 1]);
          const float t = (e & 1) ? hi_f(w) : lo_f(w);
          float d = fmaf(bsrc[j], t, acc[e][j]);
          if constexpr (ACC) d += elem<true>(old[cg & 1][j], e);
          f[e] = d;
        }
        if (vlive[j] && qok[cg])
          bnt_store16(static_cast<char*>(a.dsrc[4 * g + j]) + n * a.drow_stride * 2 +
                          (int64_t)qidx[cg] * 16,
                      pack<true>(f));
      }
      load_v(rows[cg], cg, next);
    }
    n = next;
  }
}

// dq partial rows: workgroup (tile x, range y) covers 1024 key columns from chunk a.chunk0 and the
// tokens [y * tpr, (y + 1) * tpr); wave w owns 128 of the columns. Lane (g, c) holds chunk c of
// sources 4g .. 4g+3 (B operand, sources as the contraction index) and a_{m = c, s = 4g..4g+3} of
// the token (A operand, two bf16 terms); the 16 x 16 results land as query 4g + i at column
// 8c + e. The next token's rows and coefficients load while the current token's MFMAs run.
__global__ __launch_bounds__(512) void multi_dq_mfma_kernel(const MfmaDqArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int q = a.chunk0 + (blockIdx.x * kMfmaWaves + wave) * 16 + c;  // this lane's chunk
  const bool qok = q * 8 < a.D;
  const char* vbase[4];
  bool vlive[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vlive[j] = 4 * g + j < a.S && qok;
    vbase[j] = static_cast<const char*>(vlive[j] ? a.src[4 * g + j] : nullptr);
  }
  const int64_t t0 = (int64_t)blockIdx.y * a.tpr;
  const int64_t t1 = t0 + a.tpr < a.N ? t0 + a.tpr : a.N;
  auto load = [&](Chunk (&r)[4], float4& co, int64_t tok) {
    const bool ok = tok < t1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = (ok && vlive[j]) ? bnt_load16(vbase[j] + tok * a.row_stride * 2 + (int64_t)q * 16)
                              : Chunk{};
    co = ok ? *reinterpret_cast<const float4*>(a.coef + tok * 256 + c * 16 + 4 * g)
            : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  mb_float4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = mb_float4{0.f, 0.f, 0.f, 0.f};
  Chunk rows[4];
  float4 co;
  load(rows, co, t0);
  for (int64_t n = t0; n < t1; ++n) {
    const Chunk cur[4] = {rows[0], rows[1], rows[2], rows[3]};
    const float cw[4] = {co.x, co.y, co.z, co.w};
    load(rows, co, n + 1);
    mb_short4 a_hi, a_lo;
    split_a(cw, a_hi, a_lo);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const mb_short4 b = gather_e(cur, e);
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, b, acc[e], 0, 0, 0);
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, b, acc[e], 0, 0, 0);
    }
  }
  // lane (g, c): query 4g + i at column 8q + e, slice columns only
  float* prow = a.part + (int64_t)blockIdx.y * a.M * a.R;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * g + i;
    if (m >= a.M || !qok) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = q * 8 + e;
      if (col >= a.lo && col < a.D) prow[(int64_t)m * a.R + (col - a.lo)] = acc[e][i];
    }
  }
}

#define ATTNRES_MFMA_BWD_CASE(CGW)                                                    \
  case CGW:                                                                           \
    return acc ? (full ? (const void*)&multi_bwd_mfma_kernel<CGW, true, true>         \
                       : (const void*)&multi_bwd_mfma_kernel<CGW, false, true>)       \
               : (full ? (const void*)&multi_bwd_mfma_kernel<CGW, true, false>        \
                       : (const void*)&multi_bwd_mfma_kernel<CGW, false, false>);

const void* multi_bwd_mfma_kernel_ptr(int cgw, bool full, bool acc) {
  switch (cgw) {
    ATTNRES_MFMA_BWD_CASE(1) ATTNRES_MFMA_BWD_CASE(2) ATTNRES_MFMA_BWD_CASE(3)
    ATTNRES_MFMA_BWD_CASE(4)
    default: break;
  }
  return nullptr;
}

const void* multi_dq_mfma_kernel_ptr() { return (const void*)&multi_dq_mfma_kernel; }

}  // namespace attnres
