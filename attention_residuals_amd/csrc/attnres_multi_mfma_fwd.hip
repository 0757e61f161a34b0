// attnres_multi_mfma_fwd.hip -- multi- and selected-query forward in the operand layout of the
// matrix-core backward (gfx950, bf16 storage, D = 256 nt).
//
// Operation ("Fast Attention Residuals" PyPI page, section "Multi-query AttnRes"): M queries read
// the same S sources; p_{m,s} = softmax_s(scale * rho_s * <t_s, q_m>), y_m = sum_s p_{m,s} v_s,
// lse_m saved for the backward. Selected read: query m of token n is bank row ids[n, m].
//
// One 8-wave workgroup per CU over a static token stride; wave w owns columns
// [w * nt * 32, (w + 1) * nt * 32) as nt tiles of 32. Lane (g, c) loads, per tile, the 16 bytes at
// columns 8g .. 8g+7 of source c: the operand layout of a 16x16x32 MFMA whose contraction index is
// the column, so per tile one MFMA gives the scores Q V^T (queries, or the bank, staged as full
// rows in LDS) and one the key sums of squares diag(V V^T). The 8 waves' tiles meet in LDS and 256
// threads finish one (query, source) pair each: routing weight, row maximum and sum over the
// sources by DPP, lse. The mixture runs transposed, y^T = V^T P^T: each 16-column half of a tile
// takes one identity MFMA (the sources into the k slots) and one 16x16x32 MFMA with the weights as
// two bf16 terms (hi in slots 0-3, lo in 4-7); the two halves leave lane (g, c) with query c's
// output at eight consecutive columns, half of a 128-byte line. With five or more rows two tiles'
// outputs pass through LDS instead and go out as whole lines (8 rows x 128 bytes per store) with
// the streaming hint: up to 8 rows (STG = 8) through the wave's own exchange block, idle during
// the mixture; more (STG = 16) through a 2 KiB block per wave of their own. STG = 0 stores from
// the operand layout (fewer rows, where the staging costs more than it saves).
// Two tokens in flight: each token's rows are loaded into a second register set at the start of
// the previous token, so they arrive while that token's mixture is computed and stored.
#include "attnres_internal.hpp"
#include "attnres_kernels.hpp"
#include "attnres_mfma_tiles.hpp"

namespace attnres {
namespace {

using namespace tiles;

constexpr int kFwdXch = 256 + 16;  // a wave's score tile and its 16 sums of squares
constexpr int kFwdStage = 2048;     // a wave's output staging block: 16 rows x 128 bytes

}  // namespace

// LDS of the tile forward: the staged rows (padded; the selected read adds a zero row), the waves'
// exchange, the routing weights and, with stg = 16, the waves' output staging blocks.
size_t multi_fwd_tile_lds(int nt, int rows, bool sel, int stg) {
  const size_t D = (size_t)nt * kMfmaWaves * 32;
  return (size_t)(rows + (sel ? 1 : 0)) * (D + tiles::kRowPad) * 2 +
         ((size_t)kMfmaWaves * kFwdXch + 256) * sizeof(float) +
         (stg == 16 ? (size_t)kMfmaWaves * kFwdStage : 0);
}

template <int NT, bool FULL, bool SEL, int STG>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 8)))
void multi_fwd_tile_kernel(const MfmaFwdArgs a) {
  constexpr int W = kMfmaWaves;
  constexpr int D = NT * W * 32;
  extern __shared__ float lds[];
  static_assert(!(SEL && STG == 16), "the selected read has no staging blocks of its own");
  const int QR = SEL ? a.E : a.M;  // staged rows (queries or bank rows)
  const int QA = SEL ? QR + 1 : QR;  // allocated rows: the selected read's last one zero
  constexpr int QP = D + kRowPad;                                   // staged row pitch
  char* qrows = reinterpret_cast<char*>(lds);                      // [QA][QP] bf16
  float* xch = reinterpret_cast<float*>(qrows + (size_t)QA * QP * 2);  // [W][kFwdXch]
  float* pa = xch + W * kFwdXch;                                   // p[16][16]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // this wave's staging block (STG = 8: its exchange block, 1088 bytes)
  char* stg = STG == 16 ? reinterpret_cast<char*>(pa + 256) + wave * kFwdStage
                        : reinterpret_cast<char*>(xch + wave * kFwdXch);
  const int g = lane >> 4, c = lane & 15;
  const mb_u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int col_w = wave * NT * 32 + 8 * g;
  auto keyok = [&](int t) { return FULL || col_w + 32 * t >= a.lo; };

  // the rows as full-width rows, zero before the key slice (row QR of the selected read zero: ids
  // outside [0, E))
  for (int idx = tid; idx < QA * (D / 8); idx += W * 64) {
    const int e = idx / (D / 8), j = 8 * (idx - e * (D / 8));
    mb_u32x4 v = zero4;
    if (e < QR && j >= a.lo)
      v = *reinterpret_cast<const mb_u32x4*>(static_cast<const char*>(a.query) +
                                              ((int64_t)e * a.R + (j - a.lo)) * 2);
    *reinterpret_cast<mb_u32x4*>(qrows + ((size_t)e * QP + j) * 2) = v;
  }

  // lane (g, c) streams source c; dead lanes read the first row's chunk and discard it
  const bool vlive = c < a.S, qlive = c < a.M;
  const char* vsrc = static_cast<const char*>(a.src[0]);
#pragma unroll
  for (int s = 1; s < 16; ++s)
    if (s == c && vlive) vsrc = static_cast<const char*>(a.src[s]);
  vsrc += col_w * 2;
  char* ybase = static_cast<char*>(a.y) + ((qlive ? c * a.y_sm : 0) + col_w) * 2;
  // STG: the output rows this lane stores from the staging block, queries (slots) yr and, with
  // STG = 16, 8 + yr, 16 bytes at column 8 yb of each 64-column tile pair
  const int yr = lane >> 3, yb = lane & 7;
  const bool ylive0 = yr < a.M, ylive1 = 8 + yr < a.M;
  char* yrow0 =
      static_cast<char*>(a.y) + ((ylive0 ? yr * a.y_sm : 0) + wave * NT * 32 + 8 * yb) * 2;
  char* yrow1 =
      static_cast<char*>(a.y) + ((ylive1 ? (8 + yr) * a.y_sm : 0) + wave * NT * 32 + 8 * yb) * 2;
  auto ld_v = [&](int t, int64_t n) {
    const mb_u32x4 x = ld16(vsrc + n * a.row_stride * 2 + 64 * t);
    return vlive ? x : zero4;
  };
  // the staged row query (slot) c reads for token n: c itself (lanes past M: the last query, whose
  // score rows there are never used), or the bank row its id names (row QR, zero, for absent slots
  // and ids outside [0, E))
  const int fixed_row = qlive ? c : a.M - 1;
  auto slot_row = [&](int64_t n) {
    if constexpr (!SEL) return fixed_row;
    int r = QR;
    if (qlive) {
      const int64_t id = a.ids[n * a.M + c];
      const bool ok = id >= 0 && id < a.E;
      if (!ok && a.id_flag) *a.id_flag = 1u;  // an ordinary vector store from this lane
      r = ok ? (int)id : a.E;
    }
    return r;
  };
  const mb_u32x2 ident = identity_operand(g, c);
  __syncthreads();

  mb_float4 tsc, tss;
  auto contract = [&](const mb_u32x4 (&V)[NT], int qrow) {
    tsc = tss = mb_float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const mb_u32x4 q =
          *reinterpret_cast<const mb_u32x4*>(qrows + ((size_t)qrow * QP + col_w + 32 * t) * 2);
      tsc = mfma_k32(q, V[t], tsc);
      const mb_u32x4 vm = keyok(t) ? V[t] : zero4;
      tss = mfma_k32(vm, vm, tss);
    }
    float* xw = xch + wave * kFwdXch;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xw[(4 * g + i) * 16 + c] = tsc[i];  // score of query 4g + i with source c
      if (4 * g + i == c) xw[256 + c] = tss[i];
    }
  };
  const int pm = tid >> 4, ps = tid & 15;  // (query, source) finished by thread tid < 256
  // routing weights and lse of token n (after the exchange barrier)
  auto softmax = [&](int64_t n) {
    if (tid < 256) {
      float sc = 0.f, ss = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {  // wave order: a fixed summation order
        sc += xch[w * kFwdXch + pm * 16 + ps];
        ss += xch[w * kFwdXch + 256 + ps];
      }
      const bool valid = pm < a.M && ps < a.S;
      const float z = valid ? source_score(ss, sc, a.inv_R, a.eps, a.scale).z : -INFINITY;
      const float mx = row_max(z);
      const float e = valid ? expf(z - mx) : 0.f;
      const float l = row_sum(e);
      pa[pm * 16 + ps] = valid ? e / l : 0.f;
      if (ps == 0 && pm < a.M) a.lse[pm * a.l_sm + n * a.l_sn] = mx + logf(l);
    }
  };
  // y of token n from the rows V: per half-tile, the transposed sources against the weights
  auto mixture = [&](const mb_u32x4 (&V)[NT], int64_t n) {
    mb_u32x4 bp;  // lane (g, c): p of query c with sources 4g .. 4g+3, hi then lo terms
    {
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = pa[c * 16 + 4 * g + i];
      mb_u32x2 hi, lo;
      split4(pv, hi, lo);
      bp = mb_u32x4{hi[0], hi[1], lo[0], lo[1]};
    }
    if constexpr (STG == 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float f[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const mb_u32x2 vt = tr_half(V[t], h, ident);  // sources 4g .. 4g+3 at one column
          const mb_float4 d = mfma_k32(mb_u32x4{vt[0], vt[1], vt[0], vt[1]}, bp,
                                       mb_float4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) f[4 * h + i] = d[i];  // query c, column 8g + 4h + i
        }
        if (qlive)
          st16(ybase + n * a.y_sn * 2 + 64 * t,
               mb_u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                        pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])});
      }
      return;
    }
    const int64_t yoff = n * a.y_sn * 2;
#pragma unroll
    for (int u = 0; u < NT / 2; ++u) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int t = 2 * u + k;
        float f[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const mb_u32x2 vt = tr_half(V[t], h, ident);  // sources 4g .. 4g+3 at one column
          const mb_float4 d = mfma_k32(mb_u32x4{vt[0], vt[1], vt[0], vt[1]}, bp,
                                       mb_float4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) f[4 * h + i] = d[i];  // query c, column 8g + 4h + i
        }
        // row c, chunk 4k + g of the tile pair (zeros for lanes past M; STG = 8: rows 0 .. 7)
        if (STG == 16 || c < 8)
          *reinterpret_cast<mb_u32x4*>(stg + stage_off(c, 4 * k + g)) =
              mb_u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                       pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
      }
      // the other lanes' chunks: LDS operations of one wave complete in order, the fences keep the
      // compiler from reusing an earlier read of the block or moving the next pair's writes ahead
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const mb_u32x4 r0 = *reinterpret_cast<const mb_u32x4*>(stg + stage_off(yr, yb));
      mb_u32x4 r1 = zero4;
      if constexpr (STG == 16) r1 = *reinterpret_cast<const mb_u32x4*>(stg + stage_off(8 + yr, yb));
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (ylive0)
        __builtin_nontemporal_store(r0, reinterpret_cast<mb_u32x4*>(yrow0 + yoff + 128 * u));
      if (STG == 16 && ylive1)
        __builtin_nontemporal_store(r1, reinterpret_cast<mb_u32x4*>(yrow1 + yoff + 128 * u));
    }
  };

  mb_u32x4 VA[NT], VB[NT];
  int64_t n = blockIdx.x;
  int qrow = slot_row(n);
#pragma unroll
  for (int t = 0; t < NT; ++t) VA[t] = ld_v(t, n);
  contract(VA, qrow);
  __syncthreads();
  softmax(n);
  __syncthreads();
  // one token: the next token's rows go into the other set first, then this token's mixture, then
  // the next token's scores and routing weights; false when there is no next token
  auto step = [&](const mb_u32x4 (&Vc)[NT], mb_u32x4 (&Vn)[NT]) {
    const int64_t next = n + gridDim.x;
    const bool more = next < a.N;
    if (more) {
#pragma unroll
      for (int t = 0; t < NT; ++t) Vn[t] = ld_v(t, next);
      qrow = slot_row(next);
    }
    mixture(Vc, n);
    if (!more) return false;
    contract(Vn, qrow);
    __syncthreads();
    softmax(next);
    __syncthreads();
    n = next;
    return true;
  };
  while (step(VA, VB) && step(VB, VA)) {
  }
}

#define ATTNRES_FWD_TILE_S(NT, SEL, STG)                                                     \
  (full ? (const void*)&multi_fwd_tile_kernel<NT, true, SEL, STG>                            \
        : (const void*)&multi_fwd_tile_kernel<NT, false, SEL, STG>)
#define ATTNRES_FWD_TILE(NT)                                                                 \
  case NT:                                                                                   \
    return sel ? (stg == 8 ? ATTNRES_FWD_TILE_S(NT, true, 8) : ATTNRES_FWD_TILE_S(NT, true, 0)) \
               : (stg == 16 ? ATTNRES_FWD_TILE_S(NT, false, 16)                              \
                            : stg == 8 ? ATTNRES_FWD_TILE_S(NT, false, 8)                    \
                                       : ATTNRES_FWD_TILE_S(NT, false, 0));

// nt = 32-column tiles per wave (D = 256 nt: 4, 8, 12 or 16); stg: outputs stored from the
// operand layout (0) or staged through LDS, up to 8 rows in the exchange block (8) or 16 in blocks
// of their own (16, not with sel)
const void* multi_fwd_tile_kernel_ptr(int nt, bool full, bool sel, int stg) {
  if ((sel && stg == 16) || (stg != 0 && stg != 8 && stg != 16)) return nullptr;
  switch (nt) {
    ATTNRES_FWD_TILE(4) ATTNRES_FWD_TILE(8) ATTNRES_FWD_TILE(12) ATTNRES_FWD_TILE(16)
    default: break;
  }
  return nullptr;
}

}  // namespace attnres
