// attnres_multi_mfma.hip -- multi-query forward through matrix cores (gfx950, bf16 storage).
//
// Operation ("Fast Attention Residuals" PyPI page, section "Multi-query AttnRes"): M queries read
// the same S sources; each has its own routing weights p_m = softmax_s(score_{m,s}) and output
// o_m = sum_s p_{m,s} v_s. All M <= 16 queries run in one pass over the sources.
//
// Layout: a workgroup of 8 waves owns one token at a time; wave w covers CGW groups of 128 columns.
// In a wave, lane (g, c) = (lane / 16, lane % 16) holds, for every column group, the 16-byte chunk c
// of the rows of sources 4g .. 4g+3 (S <= 16). That is the B-operand layout of a 16x16x16 bf16
// MFMA with the sources as the contraction index, so the mixture o[m][col] = sum_s p[m][s] v_s[col]
// is eight MFMAs per column group (one per element of the chunk) whose results land with lane
// (g, c) holding outputs of queries 4g .. 4g+3 at chunk c: each is stored as one 16-byte chunk.
// The routing weights enter as the A operand split into two bf16 terms (p = p_hi + p_lo), so the
// mixture keeps ~16 bits of the weights; the products and sums are FP32 inside the MFMA.
// The scores (contractions over the key columns) stay on the vector ALU: each lane dots its four
// rows with the queries' chunks (staged in LDS once per workgroup, zero outside the key slice),
// a DPP row sum reduces over the 16 lanes of the lane group, and one LDS exchange per token sums
// the 8 waves. Lane (g, c) then scores query c on its own four sources; the softmax's maximum and
// sum combine the four lane groups through lane swaps.
#include "attnres_internal.hpp"
#include "attnres_kernels.hpp"

namespace attnres {
namespace {

typedef short mf_short4 __attribute__((ext_vector_type(4)));
typedef float mf_float4 __attribute__((ext_vector_type(4)));
typedef uint32_t mf_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mf_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ Chunk nt_load16(const char* p) {
  return __builtin_bit_cast(Chunk,
                            __builtin_nontemporal_load(reinterpret_cast<const mf_u32x4*>(p)));
}
__device__ __forceinline__ void nt_store16(char* p, const Chunk& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(mf_u32x4, v), reinterpret_cast<mf_u32x4*>(p));
}

// Two bf16 halves gathered from two words: {a.low, b.low} and {a.high, b.high} (v_perm_b32 picks
// bytes 0-3 from its second operand and 4-7 from its first).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Maximum / sum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the same lane of the wave's four DPP
// rows): row pairs are swapped lane by lane, then the two halves of the wave.
__device__ __forceinline__ float group4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  x = fmaxf(bits_f(a[0]), bits_f(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return fmaxf(bits_f(b[0]), bits_f(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  x = bits_f(a[0]) + bits_f(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return bits_f(b[0]) + bits_f(b[1]);
}

// Sum of 8 consecutive floats in LDS (the 8 waves' partial sums of one value), in wave order.
__device__ __forceinline__ float sum8(const float* p) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  const float4 v = *reinterpret_cast<const float4*>(p + 4);
  return ((u.x + u.y) + (u.z + u.w)) + ((v.x + v.y) + (v.z + v.w));
}

}  // namespace

// SEL: the selected-query read: token n's query m is bank row ids[n, m] (M = slots per token); the
// whole bank plus one zero row (for ids outside [0, E)) is staged instead of M fixed queries.
// Up to four queries: four waves per SIMD (two workgroups per CU), measured 2-3% faster than the
// compiler's own allocation even where the widest rows then spill a few registers.
template <int CGW, int MQ, bool FULL, bool SEL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(MQ <= 4 ? 4 : 1, 8)))
void multi_fwd_mfma_kernel(const MfmaFwdArgs a) {
  constexpr int W = kMfmaWaves;
  constexpr int NQ = W * CGW * 16;           // 16-byte chunks of a row the workgroup covers
  constexpr int XF = 16 * (MQ + 1) * W;      // one exchange buffer: [16 sources][MQ + 1][W]
  extern __shared__ float lds[];
  const int QROWS = SEL ? a.E + 1 : MQ;         // staged query rows
  Chunk* qlds = reinterpret_cast<Chunk*>(lds);  // [QROWS][NQ] query chunks
  float* xch = lds + (size_t)QROWS * NQ * 4;    // two exchange buffers
  uint32_t* tslot = reinterpret_cast<uint32_t*>(xch + 2 * XF);  // two ticket slots
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;

  // the queries (SEL: the bank rows) as bf16 chunks of full-width rows: zero outside the key slice
  // [lo, D) and for rows past M (SEL: the extra row E), so <row, query> needs no mask
  const uint16_t* qsrc = static_cast<const uint16_t*>(a.query);
  const int qlive_rows = SEL ? a.E : a.M;
  for (int idx = tid; idx < QROWS * NQ; idx += W * 64) {
    const int m = idx / NQ, q = idx - m * NQ;
    Chunk v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int col = q * 8 + 2 * i + k;
        h[k] = (m < qlive_rows && col >= a.lo && col < a.D)
                   ? static_cast<uint32_t>(qsrc[(int64_t)m * a.R + (col - a.lo)])
                   : 0u;
      }
      v.w[i] = h[0] | (h[1] << 16);
    }
    qlds[idx] = v;
  }

  // this lane's sources 4g + j and its chunk q = (wave * CGW + cg) * 16 + c of every column group
  const char* base[4];
  bool live[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = 4 * g + j;
    live[j] = s < a.S;
    base[j] = static_cast<const char*>(live[j] ? a.src[s] : nullptr);
  }
  int qidx[CGW];
  bool qok[CGW];
#pragma unroll
  for (int cg = 0; cg < CGW; ++cg) {
    qidx[cg] = (wave * CGW + cg) * 16 + c;
    qok[cg] = qidx[cg] * 8 < a.D;
  }
  // key-slice masks of the chunks' bf16 halves for sum t^2 (columns >= lo)
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
  char* ybase = static_cast<char*>(a.y);
  __syncthreads();

  // Tokens are strided over the grid. With 16 query slots (one workgroup per CU, no other latency
  // hiding) a column group's rows for the next token are loaded as soon as this token's mixture has
  // read them, into the same registers, so loads stay in flight through the rest of the token
  // (forward at M = 16: 1.89 -> 1.72 ms); with up to 8 slots (two workgroups per CU up to four) each
  // token loads its rows at its start, which measured faster there (M = 3: 0.74 ms against 1.06;
  // M = 8: 1.04 against 1.14). A one-token-ahead prefetch into a second register set measured 2-3%
  // slower than loading at the start: its per-token register copies cost more than it hid.
  constexpr bool kInPlace = MQ == 16;
  auto load_group = [&](Chunk (&r)[4], int cg, int64_t tok) {
    const int64_t roff = tok * a.row_stride * 2;
    const bool tok_ok = tok < a.N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (tok_ok && live[j] && qok[cg]) {
        r[j] = nt_load16(base[j] + roff + (int64_t)qidx[cg] * 16);
      } else {
        r[j] = Chunk{};
      }
    }
  };
  // Tokens: with a counter, batches of tpt consecutive tokens, the first batch by workgroup index
  // and each later one by a ticket taken during the batch's last token (read after that token's
  // exchange barrier, before the next token's rows are loaded); without one, a static stride.
  // Only the sixteen-slot kernels (one workgroup per CU) take tickets: M = 16, 1.86 -> 1.79 ms.
  // With up to eight slots the counter's registers cost more than it balances (two or more
  // workgroups per CU; M = 4 0.78 -> 0.97 ms, M = 8 1.03 -> 1.15, even on the static stride).
  constexpr bool kTickets = MQ == 16;
  const bool dyn = kTickets && a.ticket != nullptr;
  const int64_t B = dyn ? a.tpt : 1;
  int64_t n = (int64_t)blockIdx.x * B, batch_end = n + B;
  Chunk rows[CGW][4];
  if constexpr (kInPlace) {
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) load_group(rows[cg], cg, n);
  }
  int buf = 0;
  while (n < a.N) {
    const bool take = dyn && n + 1 >= batch_end;
    uint32_t tk = 0;
    if (take && tid == 0) tk = atomicAdd(a.ticket, 1u);
    if constexpr (!kInPlace) {
#pragma unroll
      for (int cg = 0; cg < CGW; ++cg) load_group(rows[cg], cg, n);
    }

    // SEL: the staged row of each slot's query (uniform: the ids are read through the scalar cache)
    int qrow[MQ];
    bool bad_id = false;
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      if constexpr (SEL) {
        const int64_t id = m < a.M ? a.ids[n * a.M + m] : -1;
        qrow[m] = (id >= 0 && id < a.E) ? (int)id : a.E;
        bad_id |= m < a.M && qrow[m] == a.E;
      } else {
        qrow[m] = m;
      }
    }
    // an id outside [0, E): one lane sets the flag word (an ordinary vector store)
    if (SEL && bad_id && tid == 0 && a.id_flag) *a.id_flag = 1u;

    // per source: sum t^2 over the key slice and <row, query_m> (queries zero off the slice)
    float ss[4], acc[4][MQ];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ss[j] = 0.f;
#pragma unroll
      for (int m = 0; m < MQ; ++m) acc[j][m] = 0.f;
    }
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t t = rows[cg][j].w[i];
          ss[j] = dot2(t, FULL ? t : (t & gm[FULL ? 0 : cg][i]), ss[j]);
        }
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        const Chunk qv = qlds[qrow[m] * NQ + qidx[cg]];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][m] = dot2(rows[cg][j].w[i], qv.w[i], acc[j][m]);
      }
    }
    float* xb = xch + buf * XF;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ss[j] = row_sum(ss[j]);
#pragma unroll
      for (int m = 0; m < MQ; ++m) acc[j][m] = row_sum(acc[j][m]);
    }
    if (c == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 4 * g + j;
        xb[(s * (MQ + 1)) * W + wave] = ss[j];
#pragma unroll
        for (int m = 0; m < MQ; ++m) xb[(s * (MQ + 1) + 1 + m) * W + wave] = acc[j][m];
      }
    }
    if (take && tid == 0) tslot[buf] = tk;
    __syncthreads();
    int64_t next = dyn ? n + 1 : n + gridDim.x;
    if (take) {
      next = ((int64_t)gridDim.x + (int64_t)__builtin_amdgcn_readfirstlane(tslot[buf])) * B;
      batch_end = next + B;
    }
    buf ^= 1;

    // lane (g, c) finishes query c on its sources 4g .. 4g+3; the softmax's maximum and sum
    // combine the four lane groups (lanes c, c + 16, c + 32, c + 48), so every lane ends with
    // its routing weights p[c][4g + r] and the query's lse
    const bool qlive = c < a.M;
    float z4[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = 4 * g + r;
      z4[r] = -INFINITY;
      if (qlive && s < a.S) {
        const float gsum = sum8(xb + (s * (MQ + 1)) * W);
        const float csum = sum8(xb + (s * (MQ + 1) + 1 + c) * W);
        z4[r] = source_score(gsum, csum, a.inv_R, a.eps, a.scale).z;
        mx = fmaxf(mx, z4[r]);
      }
    }
    mx = group4_max(qlive ? mx : 0.f);
    float e4[4], l = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e4[r] = (qlive && 4 * g + r < a.S) ? expf(z4[r] - mx) : 0.f;
      l += e4[r];
    }
    l = group4_sum(l);
    float p4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p4[r] = qlive ? e4[r] / l : 0.f;
    if (g == 0 && qlive) a.lse[c * a.l_sm + n * a.l_sn] = mx + logf(l);

    // A operand: row c (query), k = 4g + r (source): p as two bf16 terms
    uint32_t ah[2], al[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float p0 = p4[2 * i], p1 = p4[2 * i + 1];
      ah[i] = pack_bf16x2(p0, p1);
      al[i] = pack_bf16x2(p0 - lo_f(ah[i]), p1 - hi_f(ah[i]));
    }
    const mf_short4 a_hi = __builtin_bit_cast(mf_short4, mf_u32x2{ah[0], ah[1]});
    const mf_short4 a_lo = __builtin_bit_cast(mf_short4, mf_u32x2{al[0], al[1]});

#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) {
      mf_float4 acc_o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        const uint32_t b0 = (e & 1) ? pair_hi(rows[cg][0].w[wi], rows[cg][1].w[wi])
                                    : pair_lo(rows[cg][0].w[wi], rows[cg][1].w[wi]);
        const uint32_t b1 = (e & 1) ? pair_hi(rows[cg][2].w[wi], rows[cg][3].w[wi])
                                    : pair_lo(rows[cg][2].w[wi], rows[cg][3].w[wi]);
        const mf_short4 bv = __builtin_bit_cast(mf_short4, mf_u32x2{b0, b1});
        mf_float4 o = {0.f, 0.f, 0.f, 0.f};
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, bv, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, bv, o, 0, 0, 0);
        acc_o[e] = o;
      }
      // the mixture has read this column group: its registers take the next token's rows
      if constexpr (kInPlace) load_group(rows[cg], cg, next);
      // lane (g, c) holds query 4g + r at chunk qidx[cg], element e, in acc_o[e][r]
      if (qok[cg]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * g + r;
          if (m < a.M) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = acc_o[e][r];
            nt_store16(ybase + ((int64_t)m * a.y_sm + n * a.y_sn + (int64_t)qidx[cg] * 8) * 2,
                       pack<true>(f));
          }
        }
      }
    }
    n = next;
  }
}

// instantiations: 1 to 4 column groups per wave, with or without a key slice
#define ATTNRES_MFMA_CASE(CGW) \
  case CGW: return full ? (const void*)&multi_fwd_mfma_kernel<CGW, MQ, true, SEL> \
                        : (const void*)&multi_fwd_mfma_kernel<CGW, MQ, false, SEL>;

template <int MQ, bool SEL>
static const void* mfma_ptr(int cgw, bool full) {
  switch (cgw) {
    ATTNRES_MFMA_CASE(1) ATTNRES_MFMA_CASE(2) ATTNRES_MFMA_CASE(3) ATTNRES_MFMA_CASE(4)
    default: break;
  }
  return nullptr;
}

const void* multi_fwd_mfma_kernel_ptr(int cgw, int mq, bool full, bool sel) {
  if (sel) {
    if (mq == 4) return mfma_ptr<4, true>(cgw, full);
    if (mq == 8) return mfma_ptr<8, true>(cgw, full);
    if (mq == 16) return mfma_ptr<16, true>(cgw, full);
    return nullptr;
  }
  if (mq == 4) return mfma_ptr<4, false>(cgw, full);
  if (mq == 8) return mfma_ptr<8, false>(cgw, full);
  if (mq == 16) return mfma_ptr<16, false>(cgw, full);
  return nullptr;
}

size_t multi_fwd_mfma_lds(int cgw, int mq, int qrows) {
  return (size_t)qrows * kMfmaWaves * cgw * 16 * 16 +
         2 * sizeof(float) * 16 * (mq + 1) * kMfmaWaves + 2 * sizeof(uint32_t);
}

}  // namespace attnres
