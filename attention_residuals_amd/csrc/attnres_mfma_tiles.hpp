// attnres_mfma_tiles.hpp -- operand helpers of the matrix-core multi-query kernels (gfx950).
//
// Rows are held in the operand layout of a 16x16x32 bf16 MFMA whose contraction index is the
// column: lane (g, c) = (lane / 16, lane % 16) keeps, per 32-column tile, the 16 bytes at columns
// 8g .. 8g+7 of row c. A 16x16x16 MFMA against the identity transposes a 16x16 block of such data
// into the output layout (lane (g, c): rows 4g .. 4g+3 of one column), exactly for bf16 values.
#pragma once
#include "attnres_kernels.hpp"

namespace attnres {
namespace tiles {

// bf16 elements of padding after each row staged in LDS: row r starts 16 r bytes further round the
// 64 banks, so the 16 lanes of one lane group g, which read 16 bytes of rows 0..15 at the same
// column, fall in distinct banks instead of all in the same four
constexpr int kRowPad = 8;


typedef short mb_short4 __attribute__((ext_vector_type(4)));
typedef float mb_float4 __attribute__((ext_vector_type(4)));
typedef uint32_t mb_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t mb_u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 mb_bf16x8 __attribute__((ext_vector_type(8)));

// 16 bytes with the streaming hint: for loads whose 64 lanes cover whole 128-byte lines
__device__ __forceinline__ Chunk bnt_load16(const char* p) {
  return __builtin_bit_cast(Chunk,
                            __builtin_nontemporal_load(reinterpret_cast<const mb_u32x4*>(p)));
}
// 16 bytes with the default cache policy. The operand-layout tiles touch 64 bytes of each of 16
// rows per instruction and the other half of each 128-byte line one tile later; with the
// streaming hint those halves were fetched and written back separately (HBM counters: 1.46x the
// bytes read and 1.45x the bytes written at sixteen queries), with the default policy the line
// stays in L2 until its second half arrives.
__device__ __forceinline__ mb_u32x4 ld16(const char* p) {
  return *reinterpret_cast<const mb_u32x4*>(p);
}
__device__ __forceinline__ void st16(char* p, const mb_u32x4& v) {
  *reinterpret_cast<mb_u32x4*>(p) = v;
}

// Byte offset of 16-byte chunk b (0 .. 7) of row r (0 .. 15) in a 2 KiB staging block that turns
// two operand-layout tiles (lane (g, c): row c, 16 bytes at column 8g of each) into whole 128-byte
// row segments: the XOR spreads both the tile writes (16 rows, one chunk each) and the row reads
// (8 rows of 8 chunks) over all 64 banks per 16 lanes.
__device__ __forceinline__ int stage_off(int r, int b) { return (r * 8 + (b ^ ((r >> 1) & 7))) * 16; }

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

// Four FP32 weights as two bf16 terms (w = hi + lo, ~16 bits kept), each packed as 4 bf16
__device__ __forceinline__ void split4(const float (&w)[4], mb_u32x2& hi, mb_u32x2& lo) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    hi[i] = pack_bf16x2(w[2 * i], w[2 * i + 1]);
    lo[i] = pack_bf16x2(w[2 * i] - lo_f(hi[i]), w[2 * i + 1] - hi_f(hi[i]));
  }
}
__device__ __forceinline__ void split_a(const float (&w)[4], mb_short4& hi, mb_short4& lo) {
  mb_u32x2 h, l;
  split4(w, h, l);
  hi = __builtin_bit_cast(mb_short4, h);
  lo = __builtin_bit_cast(mb_short4, l);
}

__device__ __forceinline__ mb_float4 mfma_k32(const mb_u32x4& a, const mb_u32x4& b,
                                              const mb_float4& acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mb_bf16x8, a),
                                                 __builtin_bit_cast(mb_bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ mb_float4 mfma_k16(const mb_u32x2& a, const mb_u32x2& b,
                                              const mb_float4& acc) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mb_short4, a),
                                                   __builtin_bit_cast(mb_short4, b), acc, 0, 0, 0);
}

// Transpose of half h of a tile held in operand layout (lane (g, c): row c, columns 8g .. 8g+7 in
// x's eight bf16 slots). The 16x16x16 A operand takes slots 4h .. 4h+3 (columns 8g + 4h + i as
// k = 4g + i); against the identity the product is that block itself in the output layout, so
// lane (g, c) receives rows 4g .. 4g+3 at column 8(c/4) + 4h + c%4 of the tile, exact in FP32,
// and the high halves of the FP32 words are those bf16 values again.
__device__ __forceinline__ mb_u32x2 tr_half(const mb_u32x4& x, int h, const mb_u32x2& ident) {
  const mb_u32x2 a = h ? mb_u32x2{x[2], x[3]} : mb_u32x2{x[0], x[1]};
  const mb_float4 t = mfma_k16(a, ident, mb_float4{0.f, 0.f, 0.f, 0.f});
  return mb_u32x2{bpair_hi(f_bits(t[0]), f_bits(t[1])), bpair_hi(f_bits(t[2]), f_bits(t[3]))};
}

// The same transpose of a block already in the 16x16x16 A layout (four bf16 per lane).
__device__ __forceinline__ mb_u32x2 tr2(const mb_u32x2& a, const mb_u32x2& ident) {
  const mb_float4 t = mfma_k16(a, ident, mb_float4{0.f, 0.f, 0.f, 0.f});
  return mb_u32x2{bpair_hi(f_bits(t[0]), f_bits(t[1])), bpair_hi(f_bits(t[2]), f_bits(t[3]))};
}

// Sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the same lane of the wave's four DPP rows).
__device__ __forceinline__ float rows4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  x = bits_f(a[0]) + bits_f(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return bits_f(b[0]) + bits_f(b[1]);
}

// Identity B operand of the transposes: lane (g, c) holds I[4g + i][c] (bf16 1.0 in slot c % 4
// when c / 4 == g), built without a runtime vector index.
__device__ __forceinline__ mb_u32x2 identity_operand(int g, int c) {
  const uint32_t one = ((c >> 2) == g) ? ((c & 1) ? 0x3F800000u : 0x00003F80u) : 0u;
  return mb_u32x2{(c & 2) ? 0u : one, (c & 2) ? one : 0u};
}

// Maximum over the 16 lanes of a DPP row, in every lane of the row.
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp<0x128>(x));  // row_ror:8
  x = fmaxf(x, dpp<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  return x;
}

}  // namespace tiles
}  // namespace attnres
