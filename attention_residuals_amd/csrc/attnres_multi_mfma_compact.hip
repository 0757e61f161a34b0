// attnres_multi_mfma_compact.hip -- multi-query backward through matrix cores when a token's
// sources and dY rows fit one 16-row tile together (S + M <= 16; gfx950, bf16 storage, D = 256 nt).
//
// Operation ("Fast Attention Residuals" PyPI page, section "Multi-query AttnRes") as in
// attnres_multi_mfma_bwd.hip: p_{m,s} from the saved lse, dp_{m,s} = <dY_m, v_s>,
// a_{m,s} = scale p_{m,s} (dp_{m,s} - delta_m) rho_s, B_s = -rho_s^2 / R sum_m a_{m,s} c_{m,s},
// dv_s = sum_m p_{m,s} dY_m + [key slice] (sum_m a_{m,s} q_m + B_s t_s), dq_m = sum_{n,s} a_{m,s} t_s.
//
// Lane (g, c) of an 8-wave workgroup holds, per 32-column tile, the 16 bytes at columns
// 8g .. 8g+7 of row c of X: the token's sources in rows 0 .. S-1, its dY rows in rows
// S .. S+M-1. That is half the registers of separate source and dY tiles, so the next token's rows
// load into a second register set while the current token's dv is formed (two tokens in flight).
//   * Column contractions, one 16x16x32 MFMA each per tile: the Gram matrix X X^T, whose dY-by-
//     source block is dp and whose diagonal over the source rows holds the sums of squares (from a
//     second MFMA on the key-masked rows when R < D), and the scores Q X^T against the queries
//     staged as rows in LDS.
//   * dv^T per 16-column half: an identity MFMA transposes X (its rows into the k slots) for two
//     16x16x16 MFMAs with p as two bf16 terms (zero for the source rows); another transposes the
//     query rows for two with a; B_s t_s is added on the vector ALU and each dv chunk rounded once
//     (without the dq sums in LDS, each tile pair's chunks then go out as whole 128-byte row
//     segments through the wave's exchange block).
//   * dq with M <= 8 where the sums fit the LDS: summed per workgroup in LDS from the same
//     transposed X (a is zero past the source rows) and written as one partial row; otherwise the
//     token's a_{m,s} go to the workspace and the dq kernel forms dq.
#include "attnres_internal.hpp"
#include "attnres_kernels.hpp"
#include "attnres_mfma_tiles.hpp"

namespace attnres {
namespace {

using namespace tiles;

// a wave's exchange (FP32): the score rows of up to QX queries (slots), the dY-by-source rows of
// its Gram tile for those queries and 16 sums of squares; QX = 8 with dq summed in LDS (M <= 8),
// else 16
constexpr int compact_qx(bool dq) { return dq ? 8 : 16; }
constexpr int compact_xch(bool dq) { return 2 * compact_qx(dq) * 16 + 16; }

}  // namespace

// LDS: the dq sums ([M][D + 8] FP32, with dq) and a scratch row for the rows past M of a lane's
// group of four ([32 nt + 32] FP32), the queries (selected read: the bank) as padded rows, the
// waves' exchange, p and a, the B partial sums and the slots' bank rows.
size_t multi_bwd_compact_lds(int nt, bool dq, int rows, int M) {
  const size_t D = (size_t)nt * kMfmaWaves * 32;
  return (dq ? ((size_t)M * (D + 8) + 32 * nt + 32) * sizeof(float) : 0) +
         (size_t)rows * (D + tiles::kRowPad) * 2 +
         ((size_t)kMfmaWaves * compact_xch(dq) + 512 + 64 + 16) * sizeof(float);
}

// SEL: the selected read (M = slots per token; slot m of token n reads bank row ids[n, m], a zero
// row for ids outside [0, E)); the dq kernel then forms dbank from a summed per bank row.
template <int NT, bool FULL, bool ACC, bool DQ, bool SEL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 8)))
void multi_bwd_compact_kernel(const MfmaBwdArgs a) {
  static_assert(!SEL || !DQ, "the selected read forms dbank in the dq kernel");
  constexpr int W = kMfmaWaves;
  constexpr int D = NT * W * 32;
  constexpr int QP = D + kRowPad;  // staged row pitch (bf16 elements)
  constexpr int DQS = D + 8;       // dq row stride (floats)
  extern __shared__ float lds[];
  const int M = a.M, S = a.S;
  const int QR = SEL ? a.E : M;  // staged rows
  constexpr int QX = compact_qx(DQ), XS = compact_xch(DQ);
  float* dql = lds;                                                    // DQ: [M][DQS]
  float* dqx = dql + M * DQS;                                          // DQ: [32 NT + 32]
  char* qrows = reinterpret_cast<char*>(lds + (DQ ? M * DQS + 32 * NT + 32 : 0));  // [QR][QP]
  float* xch = reinterpret_cast<float*>(qrows + (size_t)QR * QP * 2);         // [W][XS]
  float* pa = xch + W * XS;                                                   // p, a [16][16]
  float* bpart = pa + 512;                                                     // [4][16]
  int* sid = reinterpret_cast<int*>(bpart + 64);                               // SEL: [16]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const mb_u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int col_w = wave * NT * 32 + 8 * g;
  auto keyok = [&](int t) { return FULL || col_w + 32 * t >= a.lo; };

  // the queries (the bank) as full-width rows, zero before the key slice
  for (int idx = tid; idx < QR * (D / 8); idx += W * 64) {
    const int e = idx / (D / 8), j = 8 * (idx - e * (D / 8));
    mb_u32x4 v = zero4;
    if (j >= a.lo)
      v = *reinterpret_cast<const mb_u32x4*>(static_cast<const char*>(a.query) +
                                              ((int64_t)e * a.R + (j - a.lo)) * 2);
    *reinterpret_cast<mb_u32x4*>(qrows + ((size_t)e * QP + j) * 2) = v;
  }
  if constexpr (DQ) {
    for (int i = tid; i < M * DQS; i += W * 64) dql[i] = 0.f;
  }

  // lane (g, c) streams row c of X: source c, or the dY row of query c - S; lanes past S + M read
  // the first source's chunk and keep zeros
  const bool vrow = c < S, yrow = c >= S && c < S + M, live = vrow || yrow;
  const char* xsrc = static_cast<const char*>(a.src[0]);
  char* vdst = static_cast<char*>(a.dsrc[0]);
#pragma unroll
  for (int s = 1; s < 16; ++s)
    if (s == c && vrow) {
      xsrc = static_cast<const char*>(a.src[s]);
      vdst = static_cast<char*>(a.dsrc[s]);
    }
  int64_t xstride = a.row_stride;
  if (yrow) {
    xsrc = static_cast<const char*>(a.dout) + (int64_t)(c - S) * a.g_sm * 2;
    xstride = a.g_sn;
  }
  xsrc += col_w * 2;
  vdst += col_w * 2;
  // without dq sums in LDS (a 2 KiB exchange block per wave) dv goes out as whole 128-byte row
  // segments: each tile pair's outputs pass through this wave's exchange block (free during dv:
  // every wave read it before the barrier that precedes dv, and this wave writes it again only
  // after), then lane l stores 16 bytes of sources dr and 8 + dr at column 8 db of the pair, with
  // the streaming hint. With dq sums the block is too small and the register file too full (the
  // staging spilled at D = 4096): dv is stored from the operand layout.
  constexpr bool STG = !DQ;
  char* stg = reinterpret_cast<char*>(xch + wave * XS);
  const int dr = lane >> 3, db = lane & 7;
  const bool dlive0 = dr < S, dlive1 = 8 + dr < S;
  char* dvr0 = static_cast<char*>(a.dsrc[0]);
  char* dvr1 = static_cast<char*>(a.dsrc[0]);
  if constexpr (STG) {
#pragma unroll
    for (int s = 1; s < 8; ++s)
      if (s == dr && dlive0) dvr0 = static_cast<char*>(a.dsrc[s]);
#pragma unroll
    for (int s = 8; s < 16; ++s)
      if (s == 8 + dr && dlive1) dvr1 = static_cast<char*>(a.dsrc[s]);
    dvr0 += (wave * NT * 32 + 8 * db) * 2;
    dvr1 += (wave * NT * 32 + 8 * db) * 2;
  }
  auto ld_x = [&](int t, int64_t n) {
    const mb_u32x4 x = ld16(xsrc + n * xstride * 2 + 64 * t);
    return live ? x : zero4;
  };
  auto ld_old = [&](int t, int64_t n) {
    const mb_u32x4 x = ld16(vdst + n * a.drow_stride * 2 + 64 * t);
    return vrow ? x : zero4;
  };
  // the staged row query (slot) c reads for token n: c itself (lanes past M: the last query, since
  // their score rows are never used and their weights a are zero), or the bank row its id names
  // (QR, read as zeros, for lanes past M and ids outside [0, E))
  const int fixed_row = c < M ? c : M - 1;
  auto slot_row = [&](int64_t n) {
    if constexpr (!SEL) return fixed_row;
    int r = QR;
    if (c < M) {
      const int64_t id = a.ids[n * M + c];
      r = (id >= 0 && id < a.E) ? (int)id : a.E;
    }
    return r;
  };
  // that row at the lane's eight columns of tile t (row QR of the selected read: zeros)
  auto ld_q = [&](int t, int qrow) {
    const int r = (SEL && qrow >= QR) ? 0 : qrow;
    const mb_u32x4 v =
        *reinterpret_cast<const mb_u32x4*>(qrows + ((size_t)r * QP + col_w + 32 * t) * 2);
    if constexpr (SEL) return qrow < QR ? v : zero4;
    return v;
  };
  const mb_u32x2 ident = identity_operand(g, c);
  // the dq sums of this lane, rows m0 + i = 4(g % 2) + i at its column of tile 0 (tile t adds 32 t
  // floats); rows past M go to the scratch row, whose contents are never used
  const int m0 = 4 * (g & 1), dcol = 8 * (c >> 2) + (c & 3) + 4 * (g >> 1);
  float* dqp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dqp[i] = (m0 + i < M) ? dql + (m0 + i) * DQS + wave * NT * 32 + dcol : dqx + dcol;
  __syncthreads();

  mb_float4 tsc, tg, tk;
  // scores, Gram matrix and key sums of squares of a token's rows X (after the exchange barrier
  // the 8 waves' tiles sit in LDS)
  auto contract = [&](const mb_u32x4 (&X)[NT], int qrow) {
    tsc = tg = tk = mb_float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      tsc = mfma_k32(ld_q(t, qrow), X[t], tsc);
      tg = mfma_k32(X[t], X[t], tg);
      if constexpr (!FULL) {
        const mb_u32x4 xm = keyok(t) ? X[t] : zero4;
        tk = mfma_k32(xm, xm, tk);
      }
    }
    float* xw = xch + wave * XS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      if (r < QX) xw[r * 16 + c] = tsc[i];  // score of query r with row c
      if (r >= S && r < S + M) xw[(QX + r - S) * 16 + c] = tg[i];  // <dY row of query r - S, row c>
      if (r == c) xw[2 * QX * 16 + c] = FULL ? tg[i] : tk[i];
    }
  };
  const int pm = tid >> 4, ps = tid & 15;  // (query, source) finished by thread tid < 256
  // the pairs of token n: routing weight, delta, a and the B terms into LDS
  auto pairs = [&](int64_t n, float lse_t, int qrow) {
    if (SEL && tid < 16) sid[tid] = qrow;  // lanes 0 .. 15 of wave 0 hold slots 0 .. 15
    if (tid < 256) {
      const int qm = pm < M ? pm : 0;  // exchange row read (queries past M are masked below)
      float sc = 0.f, dpv = 0.f, ss = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {  // wave order: a fixed summation order
        const float* x = xch + w * XS;
        sc += x[qm * 16 + ps];
        dpv += x[(QX + qm) * 16 + ps];
        ss += x[2 * QX * 16 + ps];
      }
      const bool valid = pm < M && ps < S;
      const Score scv = source_score(ss, sc, a.inv_R, a.eps, a.scale);
      const float p = valid ? routing_weight(scv.z, lse_t) : 0.f;
      const float delta = row_sum(p * dpv);
      const float av = valid ? a.scale * p * (dpv - delta) * scv.rho : 0.f;
      const float bt = valid ? -av * scv.rho * scv.rho * sc * a.inv_R : 0.f;
      pa[pm * 16 + ps] = p;
      pa[256 + pm * 16 + ps] = av;
      if constexpr (!DQ && !SEL) a.coef[n * 256 + tid] = av;
      const float bs = rows4_sum(bt);  // over this wave's four queries
      if (lane < 16) bpart[wave * 16 + ps] = bs;
    }
  };
  auto load_lse = [&](int64_t n) {
    return (tid < 256 && pm < M) ? a.lse[pm * a.l_sm + n * a.l_sn] : 0.f;
  };

  // dv of token n from its rows X (weights in LDS)
  auto dv = [&](const mb_u32x4 (&X)[NT], int64_t n, int qrow) {
    // B operands (k = rows of X, then queries): lane (g, c) holds the weights of rows 4g .. 4g+3
    // for output source c, p of the dY rows (zero for the source rows) and a of the queries
    mb_u32x2 py_hi, py_lo, aq_hi, aq_lo;
    {
      float pv[4], av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i - S;
        pv[i] = (m >= 0 && m < M) ? pa[m * 16 + c] : 0.f;
        av[i] = pa[256 + (4 * g + i) * 16 + c];
      }
      split4(pv, py_hi, py_lo);
      split4(av, aq_hi, aq_lo);
    }
    if constexpr (SEL) {
      // the dq kernel's coefficients: a of bank rows 4g .. 4g+3 with source c, the token's slots
      // summed per bank row in slot order (slots reading no bank row add to none)
      float ab[4] = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < M; ++k) {
        const int e = sid[k] - 4 * g;
        const float ak = pa[256 + k * 16 + c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (e == i && sid[k] < a.E) ab[i] += ak;
      }
      if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a.coef[n * 256 + (4 * g + i) * 16 + c] = ab[i];
      }
    }
    const float bsrc = ((bpart[c] + bpart[16 + c]) + bpart[32 + c]) + bpart[48 + c];
    // dq A operands: output row r = m + 8h (m = r % 8) takes a[m][4g + i] in slots 4h .. 4h+3
    mb_u32x4 dqa_hi = zero4, dqa_lo = zero4;
    if constexpr (DQ) {
      const int m = c & 7;
      float av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = pa[256 + m * 16 + 4 * g + i];
      mb_u32x2 ah, al;
      split4(av, ah, al);
      if (c >> 3) {
        dqa_hi = mb_u32x4{0u, 0u, ah[0], ah[1]};
        dqa_lo = mb_u32x4{0u, 0u, al[0], al[1]};
      } else {
        dqa_hi = mb_u32x4{ah[0], ah[1], 0u, 0u};
        dqa_lo = mb_u32x4{al[0], al[1], 0u, 0u};
      }
    }
    mb_u32x4 old[NT];
    if constexpr (ACC) {
      old[0] = ld_old(0, n);
      if (NT > 1) old[1] = ld_old(1, n);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (ACC) {
        if (t + 2 < NT) old[t + 2] = ld_old(t + 2, n);
      }
      const mb_u32x4 qop = ld_q(t, qrow);
      float f[8];
      mb_u32x2 xt[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        xt[h] = tr_half(X[t], h, ident);  // rows 4g .. 4g+3 of X at one column
        const mb_u32x2 qt = tr_half(qop, h, ident);  // queries 4g .. 4g+3 at that column
        mb_float4 d = mfma_k16(xt[h], py_hi, mb_float4{0.f, 0.f, 0.f, 0.f});
        d = mfma_k16(xt[h], py_lo, d);
        d = mfma_k16(qt, aq_hi, d);
        d = mfma_k16(qt, aq_lo, d);
        // lane (g, c): dv of source c at column 8g + 4h + i of the tile
#pragma unroll
        for (int i = 0; i < 4; ++i) f[4 * h + i] = d[i];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = X[t][e >> 1];
        const float tv = keyok(t) ? ((e & 1) ? hi_f(w) : lo_f(w)) : 0.f;
        float d = fmaf(bsrc, tv, f[e]);
        if constexpr (ACC) d += (e & 1) ? hi_f(old[t][e >> 1]) : lo_f(old[t][e >> 1]);
        f[e] = d;
      }
      if constexpr (DQ) {
        // the sources in the k slots (a is zero past them); output row 4g + i is query
        // m0 + i = 4(g % 2) + i of half g / 2 (queries past M have zero rows; lanes whose four
        // queries are all past M skip the sums)
        const mb_u32x4 b = {xt[0][0], xt[0][1], xt[1][0], xt[1][1]};
        mb_float4 acc = {0.f, 0.f, 0.f, 0.f};
        if (m0 < M) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = dqp[i][32 * t];
        }
        acc = mfma_k32(dqa_hi, b, acc);
        acc = mfma_k32(dqa_lo, b, acc);
        if (m0 < M) {
#pragma unroll
          for (int i = 0; i < 4; ++i) dqp[i][32 * t] = acc[i];
        }
      }
      const mb_u32x4 out = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                            pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
      if constexpr (STG) {
        // row c, chunk 4(t % 2) + g of the tile pair (zeros for lanes past S)
        *reinterpret_cast<mb_u32x4*>(stg + stage_off(c, 4 * (t & 1) + g)) = out;
        if (t & 1) {
          // the other lanes' chunks (a wave's LDS operations complete in order; the fences keep
          // the compiler from reusing an earlier read or moving the next pair's writes ahead)
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          const mb_u32x4 r0 = *reinterpret_cast<const mb_u32x4*>(stg + stage_off(dr, db));
          const mb_u32x4 r1 = *reinterpret_cast<const mb_u32x4*>(stg + stage_off(8 + dr, db));
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          const int64_t off = n * a.drow_stride * 2 + 128 * (t >> 1);
          if (dlive0) __builtin_nontemporal_store(r0, reinterpret_cast<mb_u32x4*>(dvr0 + off));
          if (dlive1) __builtin_nontemporal_store(r1, reinterpret_cast<mb_u32x4*>(dvr1 + off));
        }
      } else if (vrow) {
        st16(vdst + n * a.drow_stride * 2 + 64 * t, out);
      }
    }
  };

  mb_u32x4 XA[NT], XB[NT];
  int qa = 0, qb = 0;  // the staged rows the tokens in XA and XB read
  int64_t n = blockIdx.x;
  const float lse0 = load_lse(n);
  qa = slot_row(n);
#pragma unroll
  for (int t = 0; t < NT; ++t) XA[t] = ld_x(t, n);
  contract(XA, qa);
  __syncthreads();
  pairs(n, lse0, qa);
  __syncthreads();
  // one token: the next token's rows go into the other set first, then this token's dv, then the
  // next token's contractions and pairs; false when there is no next token
  auto step = [&](const mb_u32x4 (&Xc)[NT], int qc, mb_u32x4 (&Xn)[NT], int& qn) {
    const int64_t next = n + gridDim.x;
    const bool more = next < a.N;
    float lse_n = 0.f;
    if (more) {
#pragma unroll
      for (int t = 0; t < NT; ++t) Xn[t] = ld_x(t, next);
      lse_n = load_lse(next);
      qn = slot_row(next);
    }
    dv(Xc, n, qc);
    if (!more) return false;
    contract(Xn, qn);
    __syncthreads();
    pairs(next, lse_n, qn);
    __syncthreads();
    n = next;
    return true;
  };
  while (step(XA, qa, XB, qb) && step(XB, qb, XA, qa)) {
  }

  // this workgroup's dq partial row [M][R] (key columns)
  if constexpr (DQ) {
    __syncthreads();
    float* prow = a.part + (int64_t)blockIdx.x * a.M * a.R;
    for (int idx = tid; idx < a.M * a.R; idx += W * 64) {
      const int m = idx / a.R, j = idx - m * a.R;
      prow[idx] = dql[m * DQS + a.lo + j];
    }
  }
}

#define ATTNRES_COMPACT_K(NT, DQ, SEL)                                                           \
  (acc ? (full ? (const void*)&multi_bwd_compact_kernel<NT, true, true, DQ, SEL>                 \
               : (const void*)&multi_bwd_compact_kernel<NT, false, true, DQ, SEL>)               \
       : (full ? (const void*)&multi_bwd_compact_kernel<NT, true, false, DQ, SEL>                \
               : (const void*)&multi_bwd_compact_kernel<NT, false, false, DQ, SEL>))

#define ATTNRES_COMPACT_NT(NT)                                                                   \
  case NT:                                                                                       \
    return sel ? ATTNRES_COMPACT_K(NT, false, true)                                              \
               : (dq ? ATTNRES_COMPACT_K(NT, true, false) : ATTNRES_COMPACT_K(NT, false, false));

// nt = 32-column tiles per wave (D = 256 nt: 4, 8, 12 or 16); dq: dq summed in LDS (M <= 8, not
// with sel); sel: the selected read
const void* multi_bwd_compact_kernel_ptr(int nt, bool dq, bool full, bool acc, bool sel) {
  if (sel && dq) return nullptr;
  switch (nt) {
    ATTNRES_COMPACT_NT(4) ATTNRES_COMPACT_NT(8) ATTNRES_COMPACT_NT(12) ATTNRES_COMPACT_NT(16)
    default: break;
  }
  return nullptr;
}

}  // namespace attnres
