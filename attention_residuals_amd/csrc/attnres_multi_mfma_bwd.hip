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
// Kernel 1 (multi_bwd_mfma_kernel): one 8-wave workgroup per CU owns one token at a time; wave w
// owns the 32-column tiles (t * 8 + w), t < NT, of every row. Rows are held in the layout of a
// matrix-core operand whose contraction index is the column: lane (g, c) keeps, per tile, the 16
// bytes at columns 8g .. 8g+7 of source c and of query c's dY row. So the column contractions run
// on 16x16x32 MFMAs straight from the loaded registers: scores = Q V^T, dp = dY V^T and the key
// sums of squares diag(V V^T). The contractions over queries and sources (dv, dq) need the other
// index in the operand's k slots: a 16x16x16 MFMA against the identity transposes a 16 x 16 block
// (lane (g, c) then holds rows 4g .. 4g+3 of one column), exact for bf16 data.
//   * Per token: the score tiles of the 8 waves meet in LDS; 256 threads finish one (m, s) pair
//     each (routing weight from the saved lse, delta by a 16-lane row sum, a, and the B terms).
//   * dv^T = dY^T P + Q^T A per 16-column half-tile: one K = 32 operand carries four queries' dY
//     and q values, the other the matching p and a values, as two bf16 terms (hi, then lo, in two
//     MFMAs); B_s t_s is added on the vector ALU and each dv row chunk is rounded once to bf16
//     (with accumulate: added to the existing row first). Each tile pair's chunks then pass
//     through the wave's exchange block and go out as whole 128-byte row segments.
//   * As soon as a tile's dv is written, its registers take the next token's rows, and the next
//     token's score contractions run a few tiles behind those loads, so the loads overlap the
//     current token's work.
//   * dq: with M <= 4 the partial sums over the workgroup's tokens sit in LDS ([4][columns] FP32,
//     two half-tiles stacked into one 16x16x32 MFMA per term). Otherwise the per-token a_{m,s} go
//     to the workspace and kernel 2 forms dq. Either way one FP32 partial row per workgroup or
//     range, summed by the finaliser in a fixed order.
// Kernel 2 (multi_dq_mfma_kernel): dq_m[j] = sum_n sum_s a_{m,s,n} t_{s,n}[j] over a static token
// range per workgroup (16x16x16 MFMAs with the sources as the contraction index).
#include "attnres_internal.hpp"
#include "attnres_kernels.hpp"
#include "attnres_mfma_tiles.hpp"

namespace attnres {
namespace {

using namespace tiles;

constexpr int kXchFloats = 2 * 256 + 16;  // a wave's score and dp tiles and its 16 sums of squares

constexpr int dq_rows(int dqm) { return dqm == 1 ? 4 : 0; }
// LDS row stride of the dq sums: the row's columns plus a pad that puts the two halves' lane groups
// of one access on different banks
constexpr int dq_stride(int nt, int dqm) { return dqm ? kMfmaWaves * nt * 32 + 8 : 0; }

}  // namespace

// LDS of the per-token kernel: the dq sums (dqm = 1), the staged queries as four-row groups per
// column (M rows; selected read, qm = 2: the E bank rows), with qm >= 1 also as full-width rows
// plus a zero row and the token's slot ids, the waves' exchange, p and a, and the B partial sums.
size_t multi_bwd_mfma_lds(int nt, int dqm, int M, int qm, int E) {
  const size_t D = (size_t)nt * kMfmaWaves * 32;
  const int rows = qm == 2 ? E : M;
  size_t b = ((size_t)dq_rows(dqm) * dq_stride(nt, dqm) + (size_t)kMfmaWaves * kXchFloats + 512 +
              64) * sizeof(float) + D * ((rows + 3) / 4) * 8;
  if (qm >= 1) b += (size_t)(rows + 1) * (D + tiles::kRowPad) * 2 + 16 * sizeof(int);
  return b;
}

// QM: how the queries are staged. 0: only as four-row groups per column (the score operand is
// their transpose); 1: also as M + 1 full-width rows (the last zero), the score operand read
// directly (M <= 8); 2: the selected-query read: token n's query m is bank row ids[n, m] (M =
// slots per token), the bank staged both ways (E rows), the q term of dv and dq (here dbank)
// taking the token's a_{m,s} summed per bank row; dq is formed by the dq kernel.
template <int NT, bool FULL, bool ACC, int DQM, int QM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 8)))
void multi_bwd_mfma_kernel(const MfmaBwdArgs a) {
  constexpr bool SEL = QM == 2;
  constexpr bool QROWS = QM >= 1;
  static_assert(!SEL || DQM == 0, "the selected read forms dbank in the dq kernel");
  constexpr int W = kMfmaWaves;
  constexpr int D = NT * W * 32;          // the row width this kernel is built for
  // the next token's contractions trail its loads by LAG tiles (2 for the widest rows with the
  // transposed score operand: its registers, else spilled)
  constexpr int LAG = NT >= 8 ? (QM == 0 && NT == 16 ? 2 : 4) : 2;
  constexpr int DQR = dq_rows(DQM);
  constexpr int DQS = dq_stride(NT, DQM);
  extern __shared__ float lds[];
  float* dql = lds;                                          // [DQR][DQS] dq partial sums
  const int QR = SEL ? a.E : a.M;                            // staged query rows
  const int QG = (QR + 3) >> 2;                              // in groups of four
  char* qtl = reinterpret_cast<char*>(lds + DQR * DQS);      // [D][QG][4] bf16 queries
  float* xch = lds + DQR * DQS + D * QG * 2;                 // [W][kXchFloats]
  float* pa = xch + W * kXchFloats;                          // p[16][16], a[16][16]
  float* bpart = pa + 512;                                   // [4][16] partial B sums
  constexpr int QP = D + kRowPad;                            // staged row pitch
  char* bankl = reinterpret_cast<char*>(bpart + 64);         // QROWS: [QR + 1][QP] bf16 rows
  int* sid = reinterpret_cast<int*>(bankl + (QROWS ? (size_t)(QR + 1) * QP * 2 : 0));  // [16]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const mb_u32x4 zero4 = {0u, 0u, 0u, 0u};

  // Wave w owns columns [w * NT * 32, (w + 1) * NT * 32): tile t of lane (g, c) is the 16 bytes
  // at column ccol(t) = (w * NT + t) * 32 + 8g of source c and of query c's dY row, so a tile's
  // addresses are the lane's base plus the immediate 64 t.
  const int col_w = wave * NT * 32 + 8 * g;
  auto keyok = [&](int t) { return FULL || col_w + 32 * t >= a.lo; };

  // lane (g, c) streams source c and query c's dY row; dead lanes read the first row's chunk (the
  // same addresses as lane c = 0, so the loads coalesce) and discard it
  const bool vlive = c < a.S, qlive = c < a.M;
  const char* vsrc = static_cast<const char*>(a.src[0]);
  char* vdst = static_cast<char*>(a.dsrc[0]);
#pragma unroll
  for (int s = 1; s < 16; ++s)
    if (s == c && vlive) {
      vsrc = static_cast<const char*>(a.src[s]);
      vdst = static_cast<char*>(a.dsrc[s]);
    }
  vsrc += col_w * 2;
  vdst += col_w * 2;
  // dv goes out as whole 128-byte row segments: each tile pair's outputs pass through this wave's
  // exchange block (free during the dv loop: every wave read it before the barrier that precedes
  // the loop, and this wave writes it again only after), then lane l stores 16 bytes of sources
  // dr and 8 + dr at column 8 db of the pair, with the streaming hint
  char* stg = reinterpret_cast<char*>(xch + wave * kXchFloats);
  const int dr = lane >> 3, db = lane & 7;
  const bool dlive0 = dr < a.S, dlive1 = 8 + dr < a.S;
  char* dvr0 = static_cast<char*>(a.dsrc[0]);
  char* dvr1 = static_cast<char*>(a.dsrc[0]);
#pragma unroll
  for (int s = 1; s < 8; ++s)
    if (s == dr && dlive0) dvr0 = static_cast<char*>(a.dsrc[s]);
#pragma unroll
  for (int s = 8; s < 16; ++s)
    if (s == 8 + dr && dlive1) dvr1 = static_cast<char*>(a.dsrc[s]);
  dvr0 += (wave * NT * 32 + 8 * db) * 2;
  dvr1 += (wave * NT * 32 + 8 * db) * 2;
  const char* gsrc = static_cast<const char*>(a.dout) + ((qlive ? c * a.g_sm : 0) + col_w) * 2;

  auto ld_v = [&](int t, int64_t n) {
    const mb_u32x4 x = ld16(vsrc + n * a.row_stride * 2 + 64 * t);
    return vlive ? x : zero4;
  };
  auto ld_y = [&](int t, int64_t n) {
    const mb_u32x4 x = ld16(gsrc + n * a.g_sn * 2 + 64 * t);
    return qlive ? x : zero4;
  };
  auto ld_old = [&](int t, int64_t n) {
    const mb_u32x4 x = ld16(vdst + n * a.drow_stride * 2 + 64 * t);
    return vlive ? x : zero4;
  };

  // The queries live in LDS as qtl[column][group][4]: the four queries of a group at one column.
  // The dv contraction reads them as they are (queries 4g .. 4g+3 at the lane's column), and the
  // score contraction takes their transpose (query c at eight consecutive columns). Global loads
  // would wait behind the row loads in flight: the vector-memory counter completes in order.
  for (int idx = tid; idx < D * QG; idx += W * 64) {
    const int j = idx / QG, grp = idx - j * QG;
    uint32_t w2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t h[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int m = 4 * grp + 2 * k + e;
        h[e] = (m < QR && j >= a.lo)
                   ? static_cast<const uint16_t*>(a.query)[(int64_t)m * a.R + (j - a.lo)]
                   : 0u;
      }
      w2[k] = h[0] | (h[1] << 16);
    }
    *reinterpret_cast<mb_u32x2*>(qtl + (size_t)idx * 8) = mb_u32x2{w2[0], w2[1]};
  }
  if constexpr (QROWS) {
    // the queries (the bank) as full-width rows (zero before the key slice); row QR zero, for
    // absent slots and ids out of range
    for (int idx = tid; idx < (QR + 1) * (D / 8); idx += W * 64) {
      const int e = idx / (D / 8), j = 8 * (idx - e * (D / 8));
      mb_u32x4 v = zero4;
      if (e < QR && j >= a.lo)
        v = *reinterpret_cast<const mb_u32x4*>(static_cast<const char*>(a.query) +
                                                ((int64_t)e * a.R + (j - a.lo)) * 2);
      *reinterpret_cast<mb_u32x4*>(bankl + ((size_t)e * QP + j) * 2) = v;
    }
  }
  // QROWS: the staged row of query (slot) c for token n: c itself, or the bank row its id names
  // (row QR, zero, for ids outside [0, E) and for the lanes of absent queries)
  auto slot_row = [&](int64_t n) {
    int r = QR;
    if (qlive) {
      if constexpr (SEL) {
        const int64_t id = a.ids[n * a.M + c];
        r = (id >= 0 && id < a.E) ? (int)id : a.E;
      } else {
        r = c;
      }
    }
    return r;
  };
  // lane (g, c), half h of tile t: queries 4g .. 4g+3 at column (w NT + t) 32 + 8(c/4) + 4h + c%4
  const bool qgl = g < QG;
  const char* qtp = qtl + ((size_t)(wave * NT * 32 + 8 * (c >> 2) + (c & 3)) * QG + (qgl ? g : 0)) * 8;
  auto ld_qt = [&](int t, int h) {
    const mb_u32x2 x = *reinterpret_cast<const mb_u32x2*>(qtp + (32 * t + 4 * h) * QG * 8);
    return qgl ? x : mb_u32x2{0u, 0u};
  };

  // identity B operand of the transposes: lane (g, c) holds I[4g + i][c] (bf16 1.0 in slot c % 4
  // when c / 4 == g)
  const uint32_t one_bf = ((c >> 2) == g) ? ((c & 1) ? 0x3F800000u : 0x00003F80u) : 0u;
  const mb_u32x2 ident = {(c & 2) ? 0u : one_bf, (c & 2) ? one_bf : 0u};

  if constexpr (DQM != 0) {
    for (int i = tid; i < DQR * DQS; i += W * 64) dql[i] = 0.f;
  }
  __syncthreads();

  mb_u32x4 V[NT], Y[NT];
  mb_float4 tsc, tdp, tss;
  // scores, dp and sums of squares of tile t (lane (g, c) ends with rows 4g + i, column c); the
  // score operand is query c at the tile's eight columns 8g .. 8g+7, the transpose of its groups
  int qrow = 0;  // QROWS: the staged row query (slot) c reads for the token being contracted
  auto contract = [&](int t) {
    mb_u32x4 qop;
    if constexpr (QROWS) {
      qop = *reinterpret_cast<const mb_u32x4*>(bankl + ((size_t)qrow * QP + col_w + 32 * t) * 2);
    } else {
      const mb_u32x2 q0 = tr2(ld_qt(t, 0), ident);
      const mb_u32x2 q1 = tr2(ld_qt(t, 1), ident);
      qop = mb_u32x4{q0[0], q0[1], q1[0], q1[1]};
    }
    tsc = mfma_k32(qop, V[t], tsc);
    tdp = mfma_k32(Y[t], V[t], tdp);
    const mb_u32x4 vm = keyok(t) ? V[t] : zero4;
    tss = mfma_k32(vm, vm, tss);
  };
  auto exchange = [&]() {
    float* xw = xch + wave * kXchFloats;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xw[(4 * g + i) * 16 + c] = tsc[i];
      xw[256 + (4 * g + i) * 16 + c] = tdp[i];
      if (4 * g + i == c) xw[512 + c] = tss[i];
    }
  };
  const int pm = tid >> 4, ps = tid & 15;  // (query, source) finished by thread tid < 256
  // the pairs of token n: routing weight, delta, a and the B terms into LDS
  auto pairs = [&](int64_t n, float lse_t) {
    if (SEL && tid < 16) sid[tid] = qrow;  // lanes 0 .. 15 of wave 0 hold slots 0 .. 15
    if (tid < 256) {
      float sc = 0.f, dpv = 0.f, ss = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {  // wave order: a fixed summation order
        const float* x = xch + w * kXchFloats;
        sc += x[pm * 16 + ps];
        dpv += x[256 + pm * 16 + ps];
        ss += x[512 + ps];
      }
      const bool valid = pm < a.M && ps < a.S;
      const Score scv = source_score(ss, sc, a.inv_R, a.eps, a.scale);
      const float p = valid ? routing_weight(scv.z, lse_t) : 0.f;
      const float delta = row_sum(p * dpv);
      const float av = valid ? a.scale * p * (dpv - delta) * scv.rho : 0.f;
      const float bt = valid ? -av * scv.rho * scv.rho * sc * a.inv_R : 0.f;
      pa[pm * 16 + ps] = p;
      pa[256 + pm * 16 + ps] = av;
      if constexpr (DQM == 0 && !SEL) a.coef[n * 256 + tid] = av;
      const float bs = rows4_sum(bt);  // over this wave's four queries
      if (lane < 16) bpart[wave * 16 + ps] = bs;
    }
  };
  auto load_lse = [&](int64_t n) {
    return (tid < 256 && pm < a.M) ? a.lse[pm * a.l_sm + n * a.l_sn] : 0.f;
  };

  // first token: rows, contractions, pairs
  int64_t n = blockIdx.x;
  {
    const float lse_t = load_lse(n);
    if constexpr (SEL) qrow = slot_row(n);
    else if constexpr (QROWS) qrow = qlive ? c : QR;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      V[t] = ld_v(t, n);
      Y[t] = ld_y(t, n);
    }
    tsc = tdp = tss = mb_float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) contract(t);
    exchange();
    __syncthreads();
    pairs(n, lse_t);
    __syncthreads();
  }

  while (n < a.N) {
    const int64_t next = n + gridDim.x;
    const bool more = next < a.N;
    const int64_t ln = more ? next : n;  // rows loaded behind this token (unused after the last)
    const float lse_next = more ? load_lse(next) : 0.f;
    if constexpr (SEL) qrow = slot_row(ln);  // (fixed per lane for the multi-query read)

    // this token's coefficient operands: lane (g, c) pairs p and a of queries 4g .. 4g+3 with
    // source c (hi and lo terms), and B_c
    mb_u32x4 bop_hi, bop_lo;
    {
      float pv[4], av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = pa[(4 * g + i) * 16 + c];
        av[i] = SEL ? 0.f : pa[256 + (4 * g + i) * 16 + c];
      }
      if constexpr (SEL) {
        // a of bank rows 4g .. 4g+3 with source c: the token's slots summed per bank row, in slot
        // order; slots reading no bank row (ids out of range) add to none
        for (int k = 0; k < a.M; ++k) {
          const int e = sid[k] - 4 * g;
          const float ak = pa[256 + k * 16 + c];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (e == i && sid[k] < a.E) av[i] += ak;
        }
        if (wave == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) a.coef[n * 256 + (4 * g + i) * 16 + c] = av[i];
        }
      }
      mb_u32x2 ph, pl, ah, al;
      split4(pv, ph, pl);
      split4(av, ah, al);
      bop_hi = mb_u32x4{ph[0], ph[1], ah[0], ah[1]};
      bop_lo = mb_u32x4{pl[0], pl[1], al[0], al[1]};
    }
    const float bsrc = ((bpart[c] + bpart[16 + c]) + bpart[32 + c]) + bpart[48 + c];
    // dq A operands (M <= 4): output row r = m + 8h (m = r % 8) takes a[m][4g + i] in slots
    // 4h .. 4h+3 and zero in the other four
    mb_u32x4 dqa_hi = zero4, dqa_lo = zero4;
    if constexpr (DQM != 0) {
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

    tsc = tdp = tss = mb_float4{0.f, 0.f, 0.f, 0.f};
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
      // dv^T of tile t, two 16-column halves: k slots 0-3 carry dY of queries 4g .. 4g+3 against
      // p, slots 4-7 their q values against a
      float f[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const mb_u32x2 yt = tr_half(Y[t], h, ident);
        const mb_u32x2 qt = ld_qt(t, h);
        const mb_u32x4 op = {yt[0], yt[1], qt[0], qt[1]};
        mb_float4 d = mfma_k32(op, bop_hi, mb_float4{0.f, 0.f, 0.f, 0.f});
        d = mfma_k32(op, bop_lo, d);
        // lane (g, c): dv of source c at columns ccol(t) + 4h + i
#pragma unroll
        for (int i = 0; i < 4; ++i) f[4 * h + i] = d[i];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = V[t][e >> 1];
        const float tv = keyok(t) ? ((e & 1) ? hi_f(w) : lo_f(w)) : 0.f;
        float d = fmaf(bsrc, tv, f[e]);
        if constexpr (ACC) d += (e & 1) ? hi_f(old[t][e >> 1]) : lo_f(old[t][e >> 1]);
        f[e] = d;
      }
      // dq (M <= 4): the sources in the k slots (their transposed half-tiles); output row 4g + i
      // is query 4(g % 2) + i of half g / 2 (rows of queries 4 .. 7 are zero)
      if constexpr (DQM != 0) {
        const mb_u32x2 v0 = tr_half(V[t], 0, ident);
        const mb_u32x2 v1 = tr_half(V[t], 1, ident);
        const mb_u32x4 b = {v0[0], v0[1], v1[0], v1[1]};
        mb_float4 acc = {0.f, 0.f, 0.f, 0.f};
        float* acc_p = dql + (wave * NT + t) * 32 + 8 * (c >> 2) + (c & 3) + 4 * (g >> 1);
        if (!(g & 1)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = acc_p[i * DQS];
        }
        acc = mfma_k32(dqa_hi, b, acc);
        acc = mfma_k32(dqa_lo, b, acc);
        if (!(g & 1)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_p[i * DQS] = acc[i];
        }
      }
      // the tile's registers take the next token's rows
      V[t] = ld_v(t, ln);
      Y[t] = ld_y(t, ln);
      // row c, chunk 4(t % 2) + g of the tile pair (zeros for lanes past S)
      *reinterpret_cast<mb_u32x4*>(stg + stage_off(c, 4 * (t & 1) + g)) =
          mb_u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                   pack_bf16x2(f[6], f[7])};
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
      if (t >= LAG) contract(t - LAG);
    }
#pragma unroll
    for (int t = NT - LAG; t < NT; ++t) contract(t);
    if (!more) break;
    exchange();
    __syncthreads();
    pairs(next, lse_next);
    __syncthreads();
    n = next;
  }

  // this workgroup's dq partial row [M][R] (key columns)
  if constexpr (DQM != 0) {
    __syncthreads();
    float* prow = a.part + (int64_t)blockIdx.x * a.M * a.R;
    for (int idx = tid; idx < a.M * a.R; idx += W * 64) {
      const int m = idx / a.R, j = idx - m * a.R;
      prow[idx] = dql[m * DQS + a.lo + j];
    }
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

#define ATTNRES_MFMA_BWD_K(NT, DQM, QM)                                                       \
  (acc ? (full ? (const void*)&multi_bwd_mfma_kernel<NT, true, true, DQM, QM>                       \
               : (const void*)&multi_bwd_mfma_kernel<NT, false, true, DQM, QM>)                     \
       : (full ? (const void*)&multi_bwd_mfma_kernel<NT, true, false, DQM, QM>                      \
               : (const void*)&multi_bwd_mfma_kernel<NT, false, false, DQM, QM>))

#define ATTNRES_MFMA_BWD_NT(NT)                                                                   \
  case NT:                                                                                        \
    switch (dqm * 4 + qm) {                                                                       \
      case 1 * 4 + 1: return ATTNRES_MFMA_BWD_K(NT, 1, 1);                                       \
      case 0 * 4 + 1: return ATTNRES_MFMA_BWD_K(NT, 0, 1);                                       \
      case 0 * 4 + 0: return ATTNRES_MFMA_BWD_K(NT, 0, 0);                                       \
      case 0 * 4 + 2: return ATTNRES_MFMA_BWD_K(NT, 0, 2);                                       \
      default: return nullptr;                                                                    \
    }

// nt = 32-column tiles per wave (D = 256 nt: 4, 8, 12 or 16); dqm = 1: dq summed in LDS (M <= 4,
// with qm = 1), 0: coefficients to the workspace for the dq kernel; qm = query staging (0: groups
// only, 1: groups and rows, M <= 8; 2: the selected read)
const void* multi_bwd_mfma_kernel_ptr(int nt, int dqm, bool full, bool acc, int qm) {
  switch (nt) {
    ATTNRES_MFMA_BWD_NT(4) ATTNRES_MFMA_BWD_NT(8) ATTNRES_MFMA_BWD_NT(12) ATTNRES_MFMA_BWD_NT(16)
    default: break;
  }
  return nullptr;
}

const void* multi_dq_mfma_kernel_ptr() { return (const void*)&multi_dq_mfma_kernel; }

}  // namespace attnres
