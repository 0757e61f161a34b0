// attnres_multi_kernels.hpp -- gfx950 kernels of the multi-query AttnRes read.
//
// "Fast Attention Residuals" PyPI page, section "Multi-query AttnRes": M queries q_m read the same
// S sources; each has its own routing weights p_{m,s} = softmax_s(scale * <t_s / r_s, q_m>) and
// its own full-width output y_m = sum_s p_{m,s} v_s. The keys t_s / r_s are shared. No key-norm
// weight and no output norm (the page's operator as written).
//
// One launch serves a group of MQ <= 4 queries (the host runs larger M as several groups). The
// structure is the single-query resident path's: a workgroup holds a token's S rows in VGPRs, one
// exchange per token reduces all per-source sums (1 + MQ in the forward, 1 + 2 MQ in the backward),
// lane s finishes source s, and tokens come from the same batched ticket schedule with the next
// token's rows prefetched as the current ones are consumed. The group's query slices sit in VGPRs
// for the whole kernel (zero outside the key slice, so <t, q> needs no mask).
//
// Backward, per token, with dz_{m,s} = p_{m,s} (<dY_m, v_s> - delta_m), delta_m = sum_s p dp:
//   a_{m,s} = scale dz_{m,s} / r_s,   B_s = -sum_m a_{m,s} c_{m,s} / (R r_s^2)   (c = <t_s, q_m>)
//   dV_s = sum_m p_{m,s} dY_m + sum_m a_{m,s} q_m + B_s t_s   (q, t zero outside the slice)
//   du_m += sum_s a_{m,s} t_s   ->  dq_m (summed over tokens by the finaliser).
//
// Selected-query variant (SEL; same page and section, per-token query selection): token n's slot m
// reads with the bank row ids[n, m0 + m] of an [E, R] bank, so the query slices are reloaded per
// token (the next token's right after the exchange barrier), and the backward adds each token's
// du_m into the FP32 partial row of the bank row it selected (a per-workgroup copy of the whole
// bank's partial rows, in LDS or in a global block) instead of keeping du across tokens.
#pragma once

#include "attnres_kernels.hpp"

namespace attnres {

// A thread's columns and the group's query slices (zero outside the slice and past D).
template <bool BF16, int CH, bool FULL, int MQ>
struct MultiCols {
  static constexpr int VEC = Fmt<BF16>::VEC;
  static constexpr int ESZ = Fmt<BF16>::ESZ;
  int col0[CH];
  uint32_t voff[CH];
  uint32_t mk[CH][4];  // bf16, R < D: per-half mask of the key slice
  Chunk q[MQ][CH];     // storage-format query values at this thread's columns

  __device__ __forceinline__ void init(int tid, int nthr, int D, int lo, int M,
                                       const void* query, int R) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      col0[j] = (tid + j * nthr) * VEC;
      voff[j] = static_cast<uint32_t>(col0[j] * ESZ);
      const bool valid = col0[j] < D;
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        float v[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int idx = col0[j] + e - lo;
          v[e] = (valid && m < M && idx >= 0)
                     ? load_param<BF16>(static_cast<const char*>(query) + (int64_t)m * R * ESZ, idx)
                     : 0.f;
        }
        q[m][j] = pack<BF16>(v);  // exact: the values came from this format
      }
      if constexpr (BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bool in0 = col0[j] + 2 * k >= lo, in1 = col0[j] + 2 * k + 1 >= lo;
          mk[j][k] = (in0 ? 0x0000ffffu : 0u) | (in1 ? 0xffff0000u : 0u);
        }
      }
    }
  }
  __device__ __forceinline__ bool in_slice(int j, int e, int lo) const {
    return FULL || col0[j] + e >= lo;
  }
};

// Selected-query read: the bank rows a token's slots select (ids[tok, m0 + m]); -1 for padded slots,
// dead tokens and ids outside [0, E). An id outside [0, E) read from memory sets the flag word when
// there is one (an ordinary vector store from the lanes that met it).
template <int MQ>
__device__ __forceinline__ void load_sel_ids(const SelArgs& sa, int M, int64_t tok, bool live,
                                             int (&id)[MQ]) {
  bool bad = false;
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    const bool read = live && m < M;
    const int64_t v = read ? sa.ids[tok * sa.K + sa.m0 + m] : -1;
    id[m] = (v >= 0 && v < sa.E) ? static_cast<int>(v) : -1;
    bad |= read && id[m] < 0;
  }
  if (bad && sa.id_flag) *sa.id_flag = 1u;
}

// The query slices of bank rows `id` (zero for id < 0). With R % VEC == 0 a chunk lies wholly
// inside or before the slice; each row is read through a resource of exactly R elements and a
// chunk before the slice is given the offset R (out of range: reads zero). Otherwise the chunks
// straddle the slice start and are gathered element by element.
template <bool BF16, int CH, bool FULL, int MQ>
__device__ __forceinline__ void load_sel_queries(const SelArgs& sa, int R, int lo, int D,
                                                 const int (&id)[MQ],
                                                 const MultiCols<BF16, CH, FULL, MQ>& cs,
                                                 Chunk (&q)[MQ][CH]) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    const bool ok = id[m] >= 0;
    const char* row = static_cast<const char*>(sa.bank) + (ok ? id[m] : 0) * (int64_t)R * ESZ;
    if (R % VEC == 0) {
      const Rsrc rq = row_rsrc(ok ? row : nullptr, 0, ok ? static_cast<uint32_t>(R * ESZ) : 0u);
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int idx = cs.col0[j] - lo;
        q[m][j] = ld_row(rq, static_cast<uint32_t>((idx >= 0 ? idx : R) * ESZ));
      }
    } else {
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        float v[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int idx = cs.col0[j] + e - lo;
          v[e] = (ok && idx >= 0 && cs.col0[j] + e < D) ? load_param<BF16>(row, idx) : 0.f;
        }
        q[m][j] = pack<BF16>(v);
      }
    }
  }
}

// Selected-query backward: a thread's columns [col, col + VEC) of one FP32 partial bank row, at
// byte `row` of the workgroup's global block (a resource) or at float `row` of its LDS block. Only
// columns inside the key slice [lo, D) are touched (global: the others read 0 and drop their
// writes). With the slice start a multiple of 4 the columns go as 16-byte chunks (a chunk is then
// wholly inside or outside the slice), else element by element.
__device__ __forceinline__ uint32_t part_off(uint32_t row, int col, int lo, int D, uint32_t end) {
  return (col >= lo && col < D) ? row + static_cast<uint32_t>((col - lo) * 4) : end;
}

template <int VEC>
__device__ __forceinline__ void part_load(Rsrc rp, uint32_t row, int col, int lo, int D,
                                          uint32_t end, bool al4, float (&v)[VEC]) {
  if (al4) {
#pragma unroll
    for (int h = 0; h < VEC; h += 4) {
      const Chunk c = ld_row_cached(rp, part_off(row, col + h, lo, D, end));
#pragma unroll
      for (int k = 0; k < 4; ++k) v[h + k] = bits_f(c.w[k]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = ld_f32_cached(rp, part_off(row, col + e, lo, D, end));
  }
}

template <int VEC>
__device__ __forceinline__ void part_store(Rsrc rp, uint32_t row, int col, int lo, int D,
                                           uint32_t end, bool al4, const float (&v)[VEC]) {
  if (al4) {
#pragma unroll
    for (int h = 0; h < VEC; h += 4) {
      Chunk c;
#pragma unroll
      for (int k = 0; k < 4; ++k) c.w[k] = f_bits(v[h + k]);
      st_row_cached(rp, part_off(row, col + h, lo, D, end), c);
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) st_f32_cached(rp, part_off(row, col + e, lo, D, end), v[e]);
  }
}

// LDS block: v (+)= row[col - lo ...] over the slice; columns outside it read 0 / are skipped.
template <int VEC>
__device__ __forceinline__ void lds_part_load(const float* blk, int col, int lo, int D, bool al4,
                                              float (&v)[VEC]) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  if (al4) {
#pragma unroll
    for (int h = 0; h < VEC; h += 4) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (col + h >= lo && col + h < D) x = *reinterpret_cast<const f32x4*>(blk + (col + h - lo));
#pragma unroll
      for (int k = 0; k < 4; ++k) v[h + k] = x[k];
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = (col + e >= lo && col + e < D) ? blk[col + e - lo] : 0.f;
  }
}

template <int VEC>
__device__ __forceinline__ void lds_part_store(float* blk, int col, int lo, int D, bool al4,
                                               const float (&v)[VEC]) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  if (al4) {
#pragma unroll
    for (int h = 0; h < VEC; h += 4)
      if (col + h >= lo && col + h < D) {
        const f32x4 x = {v[h], v[h + 1], v[h + 2], v[h + 3]};
        *reinterpret_cast<f32x4*>(blk + (col + h - lo)) = x;
      }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (col + e >= lo && col + e < D) blk[col + e - lo] = v[e];
  }
}

// Sum of t^2 over the slice for one row (this thread's chunks).
template <bool BF16, int CH, bool FULL, int MQ>
__device__ __forceinline__ float slice_sumsq(const Chunk (&r)[CH],
                                             const MultiCols<BF16, CH, FULL, MQ>& cs, int lo) {
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    if constexpr (BF16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t pm = FULL ? r[j].w[k] : (r[j].w[k] & cs.mk[j][k]);
        ss = dot2(pm, pm, ss);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = elem<false>(r[j], e);
        const float tm = cs.in_slice(j, e, lo) ? t : 0.f;
        ss = fmaf(tm, tm, ss);
      }
    }
  }
  return ss;
}

// Multi-query forward: all S <= SB sources of a token in one block. SEL: the selected-query read
// (each token's queries come from the bank; the next token's are loaded once it is known).
template <bool BF16, int CH, int SB, bool FULL, int MQ, bool SEL>
__global__ __launch_bounds__(512) void multi_fwd_kernel(const MultiFwdArgs a) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int NV = 1 + MQ;  // per source: sum t^2, then <t, q_m>
  constexpr int K = NV * SB;
  extern __shared__ float lds[];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
  const int R4 = nthr >> 4;
  const int xfl = K * R4;
  const uint32_t row_bytes = static_cast<uint32_t>(a.D * ESZ);

  MultiCols<BF16, CH, FULL, MQ> cs;
  cs.init(tid, nthr, a.D, a.lo, SEL ? 0 : a.M, a.query, a.R);
  // with two or more chunks per thread the group's fixed query slices (not SEL) wait in LDS after
  // the exchange buffers and the ticket slots (each thread its own chunks; only the exchange reads
  // them), so their registers go to the row slab (measured: the two-query forward at D = 4096 went
  // from 0.592 to 0.521 ms); the compiler cannot hoist the per-token reloads past the exchange's
  // LDS stores. With one chunk per thread registers are not short and the reloads cost time.
  constexpr bool kQLds = !SEL && CH >= 2;
  Chunk* qlds = reinterpret_cast<Chunk*>(lds + 2 * xfl + 4);
  if constexpr (kQLds) {
#pragma unroll
    for (int m = 0; m < MQ; ++m)
#pragma unroll
      for (int j = 0; j < CH; ++j) qlds[(m * CH + j) * nthr + tid] = cs.q[m][j];
  }
  int buf = 0;
  Chunk rows[SB][CH];

  // token schedule: batches of B tokens, later batches from the counter (as the single-query
  // kernels: the ticket is taken at the top of a batch's last token and published through LDS at
  // that token's exchange barrier)
  const bool dyn = a.ticket != nullptr;
  const int64_t B = dyn ? a.tpt : 1;
  const int64_t n0 = (int64_t)blockIdx.x * B;
  if constexpr (SEL) {
    int id[MQ];
    load_sel_ids<MQ>(a.sel, a.M, n0, n0 < a.N, id);
    load_sel_queries<BF16, CH, FULL, MQ>(a.sel, a.R, a.lo, a.D, id, cs, cs.q);
  }
  {
    const int live = n0 < a.N ? a.S : 0;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const Rsrc r = src_rsrc(a.src[i], i, live, n0 * a.row_stride * ESZ, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) rows[i][j] = ld_row(r, cs.voff[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // dropped stores matching the output rows the loop body stores after its last row load
    const Rsrc none = row_rsrc(nullptr, 0, 0u);
    const Chunk zero = {};
#pragma unroll
    for (int m = 0; m < MQ; ++m)
#pragma unroll
      for (int j = 0; j < CH; ++j) st_row(none, cs.voff[j], zero);
  }

  uint32_t* tslot = reinterpret_cast<uint32_t*>(lds + 2 * xfl);
  int64_t n = n0, batch_end = n0 + B;
  while (n < a.N) {
    const bool take = dyn && n + 1 >= batch_end;
    uint32_t tk = 0;
    if (take && tid == 0) tk = atomicAdd(a.ticket, 1u);
    int64_t next = dyn ? n + 1 : n + gridDim.x;

    float* xb = lds + buf * xfl;
#pragma unroll
    for (int i0 = 0; i0 < SB; i0 += kGroup) {
      float part[NV][kGroup];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
#pragma unroll
        for (int v = 0; v < NV; ++v) part[v][g] = 0.f;
        if (i0 + g < SB) {
          part[0][g] = slice_sumsq<BF16, CH, FULL, MQ>(rows[i0 + g], cs, a.lo);
#pragma unroll
          for (int m = 0; m < MQ; ++m) {
            if constexpr (!kQLds) {
              part[1 + m][g] = dot_rows<BF16, CH>(rows[i0 + g], cs.q[m]);
            } else {
              Chunk qv[CH];
#pragma unroll
              for (int j = 0; j < CH; ++j) qv[j] = qlds[(m * CH + j) * nthr + tid];
              part[1 + m][g] = dot_rows<BF16, CH>(rows[i0 + g], qv);
            }
          }
        }
      }
      xchg_group<NV, SB>(part, i0, xb, R4, tid);
    }
    if (take && tid == 0) tslot[buf] = tk;
    __syncthreads();
    if (take) {
      next = ((int64_t)gridDim.x + (int64_t)__builtin_amdgcn_readfirstlane(tslot[buf])) * B;
      batch_end = next + B;
    }
    buf ^= 1;
    // SEL: the queries are not used again for this token: load the next token's in their place
    if constexpr (SEL) {
      int nid[MQ];
      load_sel_ids<MQ>(a.sel, a.M, next, next < a.N, nid);
      load_sel_queries<BF16, CH, FULL, MQ>(a.sel, a.R, a.lo, a.D, nid, cs, cs.q);
    }

    // lane s finishes source s for every query of the group
    float pw[MQ], lse[MQ];
    {
      float ss = 0.f;
      if (lane < a.S) ss = xchg_total(xb, lane, R4);
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        float z = -INFINITY;
        if (lane < a.S) {
          const float c = xchg_total(xb, (1 + m) * SB + lane, R4);
          z = source_score(ss, c, a.inv_R, a.eps, a.scale).z;
        }
        const float mx = wave_max(z);
        const float ez = (lane < a.S) ? expf(z - mx) : 0.f;
        const float l = wave_sum(ez);
        pw[m] = ez / l;
        lse[m] = mx + logf(l);
      }
    }

    float acc[MQ][CH][VEC];
#pragma unroll
    for (int m = 0; m < MQ; ++m)
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[m][j][e] = 0.f;
    // SEL: raised wave priority while the mixture is folded in and the rows and outputs go out
    // (the fixed-query forward ran 1.5% slower with it and keeps the default). Placed here, ahead
    // of the next token's row offsets, the two-chunk kernel allocates without spilling (0.583 ->
    // 0.532 ms for two slots at D = 4096); placed right before the loop below it spilled 68
    // registers (0.877 ms).
    if constexpr (SEL) __builtin_amdgcn_s_setprio(1);
    const int64_t next_byte = next * a.row_stride * ESZ;
    const int live_next = next < a.N ? a.S : 0;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      float pi[MQ];
#pragma unroll
      for (int m = 0; m < MQ; ++m) pi[m] = bcast(pw[m], i);
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float v = elem<BF16>(rows[i][j], e);
#pragma unroll
          for (int m = 0; m < MQ; ++m) acc[m][j][e] = fmaf(pi[m], v, acc[m][j][e]);
        }
      // the next token's row i (an empty resource past the last token)
      const Rsrc r = src_rsrc(a.src[i], i, live_next, next_byte, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) rows[i][j] = ld_row(r, cs.voff[j]);
    }
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      // queries past the group's count store through an empty resource (dropped)
      const Rsrc ry = src_rsrc(a.y, m, a.M, (m * a.y_sm + n * a.y_sn) * ESZ, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) st_row(ry, cs.voff[j], pack<BF16>(acc[m][j]));
    }
    if (tid < MQ && tid < a.M) {
      float v = lse[0];
#pragma unroll
      for (int m = 1; m < MQ; ++m) v = (tid == m) ? lse[m] : v;
      a.lse[tid * a.l_sm + n * a.l_sn] = v;
    }
    if constexpr (SEL) __builtin_amdgcn_s_setprio(0);
    n = next;
  }
}

// Multi-query backward, token-resident. ACC: dvalues accumulate (existing rows prefetched one
// token ahead like the source rows). SEL: the selected-query read; each token's query gradients
// are added into this workgroup's FP32 partial rows of the bank rows it selected (zeroed at the
// start; each thread only touches its own columns, read at the top of the token and written back
// at its end), summed over workgroups by the finaliser.
template <bool BF16, int CH, int SB, bool FULL, int MQ, bool ACC, bool SEL>
__global__ __launch_bounds__(512) void multi_bwd_kernel(const MultiBwdArgs a) {
  constexpr int VEC = Fmt<BF16>::VEC;
  constexpr int ESZ = Fmt<BF16>::ESZ;
  constexpr int NV = 1 + 2 * MQ;  // per source: sum t^2, <t, q_m>, <dY_m, v>
  constexpr int K = NV * SB;
  extern __shared__ float lds[];
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
  const int R4 = nthr >> 4;
  const int xfl = K * R4;
  const uint32_t row_bytes = static_cast<uint32_t>(a.D * ESZ);
  const int S = a.S;

  MultiCols<BF16, CH, FULL, MQ> cs;
  cs.init(tid, nthr, a.D, a.lo, SEL ? 0 : a.M, a.query, a.R);
  // SEL: this workgroup's FP32 partial rows of the whole bank [E, R]: in LDS after the exchange
  // buffers when they fit (a.sel.lds_bank; added into the global block once, at the end), else its
  // global block, read-modify-written per token through L2. Each thread only touches its own
  // columns, so no barrier guards them.
  const uint32_t pend = SEL ? static_cast<uint32_t>(a.sel.E * a.R * 4) : 0u;
  const bool al4 = (a.lo & 3) == 0;
  const Rsrc rpart = row_rsrc(SEL ? a.part + (int64_t)blockIdx.x * a.part_stride : nullptr, 0, pend);
  float* lbank = lds + 2 * xfl + 4;
  if (SEL && (a.sel.lds_bank || a.sel.first)) {
    float zero[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) zero[e] = 0.f;
    for (int e = 0; e < a.sel.E; ++e)
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        if (a.sel.lds_bank)
          lds_part_store<VEC>(lbank + e * a.R, cs.col0[j], a.lo, a.D, al4, zero);
        else
          part_store<VEC>(rpart, static_cast<uint32_t>(e * a.R * 4), cs.col0[j], a.lo, a.D, pend,
                          al4, zero);
      }
  }
  float du[MQ][CH][VEC];
#pragma unroll
  for (int m = 0; m < MQ; ++m)
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) du[m][j][e] = 0.f;
  int buf = 0;

  Chunk rows[SB][CH];
  Chunk odv[ACC ? SB : 1][CH];
  Chunk gy[MQ][CH];
  const bool dyn = a.ticket != nullptr;
  const int64_t B = dyn ? a.tpt : 1;
  const int64_t n0 = (int64_t)blockIdx.x * B;
  // lse of the current token per query (lane m holds query m); the next token's is loaded with
  // its rows
  float lse_l = 0.f;
  if (lane < a.M && n0 < a.N) lse_l = a.lse[lane * a.l_sm + n0 * a.l_sn];
  // SEL: the current token's bank rows, and the next token's rows and query slices (loaded right
  // after the exchange barrier, in flight during the dV loop)
  int bid[SEL ? MQ : 1], nid[SEL ? MQ : 1];
  Chunk qn[SEL ? MQ : 1][CH];
  if constexpr (SEL) {
    load_sel_ids<MQ>(a.sel, a.M, n0, n0 < a.N, bid);
    load_sel_queries<BF16, CH, FULL, MQ>(a.sel, a.R, a.lo, a.D, bid, cs, cs.q);
  }
  {
    const int live = n0 < a.N ? S : 0;
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      const Rsrc rg = src_rsrc(a.dout, m, live ? a.M : 0, (m * a.g_sm + n0 * a.g_sn) * ESZ,
                               row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) gy[m][j] = ld_row(rg, cs.voff[j]);
    }
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
  int64_t n = n0, batch_end = n0 + B;
  while (n < a.N) {
    const bool take = dyn && n + 1 >= batch_end;
    uint32_t tk = 0;
    if (take && tid == 0) tk = atomicAdd(a.ticket, 1u);
    // SEL: this token's query gradients start from zero; with global partial blocks and up to two
    // slots the rows they add into are read now (the thread's own stores of earlier tokens precede
    // these loads); with three slots there are no registers for them and they are read at the end
    constexpr bool kPrefetchPart = SEL && MQ <= 2;
    float pold[kPrefetchPart ? MQ : 1][CH][kPrefetchPart ? VEC : 1];
    if constexpr (SEL) {
#pragma unroll
      for (int m = 0; m < MQ; ++m)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) du[m][j][e] = 0.f;
          if constexpr (kPrefetchPart) {
            if (!a.sel.lds_bank && bid[m] >= 0)
              part_load<VEC>(rpart, static_cast<uint32_t>(bid[m] * a.R * 4), cs.col0[j], a.lo,
                             a.D, pend, al4, pold[m][j]);
          }
        }
    }
    float* xb = lds + buf * xfl;
#pragma unroll
    for (int i0 = 0; i0 < SB; i0 += kGroup) {
      float part[NV][kGroup];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
#pragma unroll
        for (int v = 0; v < NV; ++v) part[v][g] = 0.f;
        if (i0 + g < SB) {
          part[0][g] = slice_sumsq<BF16, CH, FULL, MQ>(rows[i0 + g], cs, a.lo);
#pragma unroll
          for (int m = 0; m < MQ; ++m) {
            part[1 + m][g] = dot_rows<BF16, CH>(rows[i0 + g], cs.q[m]);
            part[1 + MQ + m][g] = dot_rows<BF16, CH>(rows[i0 + g], gy[m]);
          }
        }
      }
      xchg_group<NV, SB>(part, i0, xb, R4, tid);
    }
    if (take && tid == 0) tslot[buf] = tk;
    __syncthreads();
    int64_t next = dyn ? n + 1 : n + gridDim.x;
    if (take) {
      next = ((int64_t)gridDim.x + (int64_t)__builtin_amdgcn_readfirstlane(tslot[buf])) * B;
      batch_end = next + B;
    }
    const bool has_next = next < a.N;
    buf ^= 1;
    if constexpr (SEL) {
      load_sel_ids<MQ>(a.sel, a.M, next, has_next, nid);
      load_sel_queries<BF16, CH, FULL, MQ>(a.sel, a.R, a.lo, a.D, nid, cs, qn);
    }

    // lane s finishes source s
    float pw[MQ], aw[MQ], Bs = 0.f;
    {
      float ss = 0.f, rho = 0.f;
      if (lane < S) ss = xchg_total(xb, lane, R4);
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        const float lse_m = bcast(lse_l, m);
        float p = 0.f, dp = 0.f, c = 0.f;
        if (lane < S) {
          c = xchg_total(xb, (1 + m) * SB + lane, R4);
          dp = xchg_total(xb, (1 + MQ + m) * SB + lane, R4);
          const Score sc = source_score(ss, c, a.inv_R, a.eps, a.scale);
          rho = sc.rho;
          p = routing_weight(sc.z, lse_m);
        }
        const float delta = wave_sum(p * dp);
        const float am = a.scale * p * (dp - delta) * rho;
        Bs -= am * rho * rho * c * a.inv_R;
        pw[m] = p;
        aw[m] = am;
      }
    }
    // queries past the group's count have dY = 0 (empty resource) and q = 0, so p dY, a q and
    // a t all vanish for them: dp = 0 = delta gives a = 0

    float dof[MQ][CH][VEC];
#pragma unroll
    for (int m = 0; m < MQ; ++m)
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) dof[m][j][e] = elem<BF16>(gy[m][j], e);
    const int live_next = has_next ? S : 0;
    if (lane < a.M && has_next) lse_l = a.lse[lane * a.l_sm + next * a.l_sn];
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      // the next token's dY rows (empty resources past the last token or the group's count)
      const Rsrc rg = src_rsrc(a.dout, m, has_next ? a.M : 0,
                               (m * a.g_sm + next * a.g_sn) * ESZ, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) gy[m][j] = ld_row(rg, cs.voff[j]);
    }
    const int64_t drow_byte = n * a.drow_stride * ESZ;
    const int64_t next_byte = next * a.row_stride * ESZ;
    const int64_t next_dbyte = next * a.drow_stride * ESZ;
    // not SEL: raised wave priority while the gradient rows are stored and the next rows loaded
    // (measured: the two- and four-query backwards 2.7% faster; the selected backward ran 1.2%
    // slower with it, so it keeps the default priority)
    if constexpr (!SEL) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      float pi[MQ], ai[MQ];
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        pi[m] = bcast(pw[m], i);
        ai[m] = bcast(aw[m], i);
      }
      const float bi = bcast(Bs, i);
      Chunk out[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        float dv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float tm;
          if constexpr (BF16) {
            const uint32_t w = FULL ? rows[i][j].w[e >> 1] : (rows[i][j].w[e >> 1] & cs.mk[j][e >> 1]);
            tm = (e & 1) ? hi_f(w) : lo_f(w);
          } else {
            const float t = elem<false>(rows[i][j], e);
            tm = cs.in_slice(j, e, a.lo) ? t : 0.f;
          }
          float d = bi * tm;
#pragma unroll
          for (int m = 0; m < MQ; ++m) {
            d = fmaf(pi[m], dof[m][j][e], d);
            d = fmaf(ai[m], elem<BF16>(cs.q[m][j], e), d);
            du[m][j][e] = fmaf(ai[m], tm, du[m][j][e]);
          }
          if constexpr (ACC) d += elem<BF16>(odv[i][j], e);
          dv[e] = d;
        }
        out[j] = pack<BF16>(dv);
      }
      const Rsrc rd = src_rsrc(a.dsrc[i], i, S, drow_byte, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) st_row(rd, cs.voff[j], out[j]);
      const Rsrc r = src_rsrc(a.src[i], i, live_next, next_byte, row_bytes);
#pragma unroll
      for (int j = 0; j < CH; ++j) rows[i][j] = ld_row(r, cs.voff[j]);
      if constexpr (ACC) {
        const Rsrc rn = src_rsrc(a.dsrc[i], i, live_next, next_dbyte, row_bytes);
#pragma unroll
        for (int j = 0; j < CH; ++j) odv[i][j] = ld_row(rn, cs.voff[j]);
      }
    }
    if constexpr (!SEL) __builtin_amdgcn_s_setprio(0);
    if constexpr (SEL) {
      // this token's query gradients into the partial bank rows it selected, slot by slot (a row
      // named by two slots adds both: the later slot starts from the earlier one's result)
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        if (bid[m] < 0) continue;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          float v[VEC];
          if (a.sel.lds_bank) {
            float* blk = lbank + bid[m] * a.R;
            lds_part_load<VEC>(blk, cs.col0[j], a.lo, a.D, al4, v);
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] += du[m][j][e];
            lds_part_store<VEC>(blk, cs.col0[j], a.lo, a.D, al4, v);
          } else if constexpr (kPrefetchPart) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = pold[m][j][e] + du[m][j][e];
            part_store<VEC>(rpart, static_cast<uint32_t>(bid[m] * a.R * 4), cs.col0[j], a.lo, a.D,
                            pend, al4, v);
#pragma unroll
            for (int m2 = m + 1; m2 < MQ; ++m2)
              if (bid[m2] == bid[m])
#pragma unroll
                for (int e = 0; e < VEC; ++e) pold[m2][j][e] = v[e];
          } else {
            const uint32_t row = static_cast<uint32_t>(bid[m] * a.R * 4);
            part_load<VEC>(rpart, row, cs.col0[j], a.lo, a.D, pend, al4, v);
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] += du[m][j][e];
            part_store<VEC>(rpart, row, cs.col0[j], a.lo, a.D, pend, al4, v);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        bid[m] = nid[m];
#pragma unroll
        for (int j = 0; j < CH; ++j) cs.q[m][j] = qn[SEL ? m : 0][j];
      }
    }
    n = next;
  }
  if constexpr (SEL) {
    // LDS partial rows into the global block: stored by the first query group, added by later ones
    if (a.sel.lds_bank) {
      for (int e = 0; e < a.sel.E; ++e)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          float v[VEC];
          lds_part_load<VEC>(lbank + e * a.R, cs.col0[j], a.lo, a.D, al4, v);
          const uint32_t row = static_cast<uint32_t>(e * a.R * 4);
          if (!a.sel.first) {
            float g[VEC];
            part_load<VEC>(rpart, row, cs.col0[j], a.lo, a.D, pend, al4, g);
#pragma unroll
            for (int k = 0; k < VEC; ++k) v[k] += g[k];
          }
          part_store<VEC>(rpart, row, cs.col0[j], a.lo, a.D, pend, al4, v);
        }
    }
    return;
  }

  // this workgroup's partial du rows of the group's queries (slice columns only)
  float* prow = a.part + (int64_t)blockIdx.x * a.part_stride;
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    if (m >= a.M) break;
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int col = cs.col0[j] + e;
        if (col < a.D && col >= a.lo) prow[m * a.R + (col - a.lo)] = du[m][j][e];
      }
  }
}

}  // namespace attnres
