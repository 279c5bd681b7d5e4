// device_common.hpp -- element types, conversions and MFMA fragment helpers
// for gfx950 (CDNA4, wave64).
//
// MFMA fragment conventions used throughout (16x16 output tiles):
//   lane l = 16*g + c, c = l % 16, g = l / 16 (g = 0..3).
//   A operand (16 x K): lane holds row c; B operand (K x 16): lane holds
//   column c; the K elements a lane holds are indexed by (g, e).  The hardware
//   multiplies A's element (g, e) with B's element (g, e), so any fixed
//   assignment of logical k indices to (g, e) is valid as long as A and B use
//   the same one.
//   D/C accumulator (16 x 16 fp32): lane holds column c, rows 4*g + i for
//   i = 0..3 (one floatx4).
//
// "Accumulator as B operand": a 16x16 fp32 accumulator tile X (rows = the
// contraction index) already holds, in lane (c, g), X[4g + i][c] for i < 4.
// Used as a B operand with the logical k index of element (g, i) = 4g + i it
// needs no data movement, only a conversion; the A operand then loads
// A[row][4g + i].  For the 32-deep bf16 instruction two consecutive 16-row
// tiles X0, X1 are used: element e < 4 is X0[4g + e], element e >= 4 is
// X1[4g + e - 4], i.e. logical k = 4g + e for e < 4 and 16 + 4g + (e - 4)
// otherwise; the A operand then loads two 4-element runs at columns 4g and
// 16 + 4g of the 32-wide block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linattn {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bf16 bit pattern in memory

__device__ __forceinline__ float bf2f(bf16_t x) {
  return __uint_as_float((uint32_t)x << 16);
}
// round to nearest even (hardware conversion; NaN stays NaN)
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Element-type traits: storage type of q/k/v/beta/g/o and of LDS operands.
struct BF16 {
  typedef bf16_t T;
  static constexpr int kVec = 8;  // elements per 16-byte vector
  __device__ static __forceinline__ float ld(const T* p) { return bf2f(*p); }
  __device__ static __forceinline__ T cvt(float f) { return f2bf(f); }
  __device__ static __forceinline__ float tof(T x) { return bf2f(x); }
};
struct F32 {
  typedef float T;
  static constexpr int kVec = 4;
  __device__ static __forceinline__ float ld(const T* p) { return *p; }
  __device__ static __forceinline__ T cvt(float f) { return f; }
  __device__ static __forceinline__ float tof(T x) { return x; }
};

struct alignas(16) Vec16 {
  uint32_t w[4];
};

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// Sum over each row of 16 lanes, returned to every lane of the row, with
// DPP moves (VALU operands) instead of LDS permutes.  quad_perm [1,0,3,2]
// and [2,3,0,1] pair lanes i, i^1 and then i, i^2; row_half_mirror pairs
// every lane of quad 0 with one of quad 1 (and 2 with 3), row_mirror every
// lane of one half-row with one of the other.  These are the pairs of an xor
// butterfly with offsets 1, 2, 4, 8, so the additions are the butterfly's,
// in its order.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  x += dpp_f32<0x140>(x);  // row_mirror
  return x;
}
// Sums of lanes l and l^16 (xsum16) and of lanes l and l^32 (xsum32), by
// v_permlane16_swap / v_permlane32_swap (VALU, no LDS).  Given one value
// twice, the 16-lane swap returns rows (0, 0, 2, 2) and (1, 1, 3, 3) of it,
// the 32-lane swap the lower half twice and the upper half twice (checked on
// the hardware), so the sum of the two results is the pair's sum in every
// lane, the same operands as a shuffle by 16 or 32 would add.
__device__ __forceinline__ float xsum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum over the whole wave in every lane: the butterfly's pairs, in its order.
__device__ __forceinline__ float sum64(float x) { return xsum32(xsum16(sum16(x))); }

// Inclusive scans over each row of 16 lanes by DPP row shifts (a lane with
// no source lane in its row reads 0): scan16_up gives lane c the sum over
// lanes 0..c, scan16_down the sum over lanes c..15.  The additions and their
// order are those of the shuffle scans with offsets 1, 2, 4, 8.
__device__ __forceinline__ float scan16_up(float x) {
  x += dpp_f32<0x111>(x);  // row_shr:1
  x += dpp_f32<0x112>(x);  // row_shr:2
  x += dpp_f32<0x114>(x);  // row_shr:4
  x += dpp_f32<0x118>(x);  // row_shr:8
  return x;
}
__device__ __forceinline__ float scan16_down(float x) {
  x += dpp_f32<0x101>(x);  // row_shl:1
  x += dpp_f32<0x102>(x);  // row_shl:2
  x += dpp_f32<0x104>(x);  // row_shl:4
  x += dpp_f32<0x108>(x);  // row_shl:8
  return x;
}
// Inclusive prefix over the whole wave: the row scans above, then
// row_bcast:15 adds the last lane of rows 0 and 2 to rows 1 and 3, and
// row_bcast:31 adds lane 31 to rows 2 and 3 (rows left out by the row mask
// add 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f32_rows(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float scan64_up(float x) {
  x = scan16_up(x);
  x += dpp_f32_rows<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_f32_rows<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// ---------------------------------------------------------------------------
// Raw MFMA instructions
// ---------------------------------------------------------------------------
__device__ __forceinline__ floatx4 mfma_k32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_k16(shortx4 a, shortx4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Operand packing
// ---------------------------------------------------------------------------
// two floats -> two bf16 (round to nearest even) in one word; written as a
// vector conversion so that it is one two-source convert instruction (a pair
// of scalar conversions became two converts plus a shift and an or)
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float float2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const float2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ bf16x8 words_to_bf16x8(uint32_t w0, uint32_t w1, uint32_t w2,
                                                   uint32_t w3) {
  struct { uint32_t w[4]; } s{{w0, w1, w2, w3}};
  return __builtin_bit_cast(bf16x8, s);
}
__device__ __forceinline__ shortx4 words_to_shortx4(uint32_t w0, uint32_t w1) {
  struct { uint32_t w[2]; } s{{w0, w1}};
  return __builtin_bit_cast(shortx4, s);
}
// two accumulator tiles -> 8 bf16 (B operand of the 32-deep instruction)
__device__ __forceinline__ bf16x8 acc_pair_to_b(floatx4 x0, floatx4 x1) {
  return words_to_bf16x8(pack2(x0[0], x0[1]), pack2(x0[2], x0[3]), pack2(x1[0], x1[1]),
                         pack2(x1[2], x1[3]));
}
__device__ __forceinline__ shortx4 acc_to_b16(floatx4 x) {
  return words_to_shortx4(pack2(x[0], x[1]), pack2(x[2], x[3]));
}

// 4 consecutive elements from LDS as two packed bf16 words
__device__ __forceinline__ void ld4_bf16(const bf16_t* p, uint32_t& w0, uint32_t& w1) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  w0 = v.x;
  w1 = v.y;
}
__device__ __forceinline__ void ld4_bf16(const float* p, uint32_t& w0, uint32_t& w1) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  w0 = pack2(v.x, v.y);
  w1 = pack2(v.z, v.w);
}

// ---------------------------------------------------------------------------
// Tile products.  `lane` is the lane index in the wave.
// ---------------------------------------------------------------------------

// acc += A[r, 0:16*ntiles] * X, with X given as `ntiles` accumulator tiles
// (tile t = contraction rows 16t..16t+15) and A's row r = lane % 16 at `arow`
// (LDS, element type EA: bf16_t or float).  Compute in bf16, fp32 accumulate.
// ntiles must be even, or 1: one accumulation chain must not mix the 32-deep
// and the 16-deep bf16 MFMA opcodes, because the compiler can issue the second
// one back to back on the first one's result without the wait states the
// different pass counts need, and the second then reads a stale accumulator.
template <class EA>
__device__ __forceinline__ floatx4 mm_accB_bf16(floatx4 acc, const EA* arow,
                                                 const floatx4* xt, int ntiles, int lane) {
  const int g = lane >> 4;
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    uint32_t a0, a1, a2, a3;
    ld4_bf16(arow + 16 * t + 4 * g, a0, a1);
    ld4_bf16(arow + 16 * t + 16 + 4 * g, a2, a3);
    acc = mfma_k32(words_to_bf16x8(a0, a1, a2, a3), acc_pair_to_b(xt[t], xt[t + 1]), acc);
  }
  if (t < ntiles) {  // only when ntiles == 1 (see above)
    uint32_t a0, a1;
    ld4_bf16(arow + 16 * t + 4 * g, a0, a1);
    acc = mfma_k16(words_to_shortx4(a0, a1), acc_to_b16(xt[t]), acc);
  }
  return acc;
}

// Same contraction in fp32 (16x16x4 fp32 MFMA; A read from fp32 LDS).
__device__ __forceinline__ floatx4 mm_accB_f32(floatx4 acc, const float* arow,
                                                const floatx4* xt, int ntiles, int lane) {
  const int g = lane >> 4;
  for (int t = 0; t < ntiles; ++t) {
    const float4 a = *reinterpret_cast<const float4*>(arow + 16 * t + 4 * g);
    acc = mfma_f32(a.x, xt[t][0], acc);
    acc = mfma_f32(a.y, xt[t][1], acc);
    acc = mfma_f32(a.z, xt[t][2], acc);
    acc = mfma_f32(a.w, xt[t][3], acc);
  }
  return acc;
}

// acc += A[r, 0:K] * B[c, 0:K]^T with both operands row-major in LDS:
// arow = row r = lane % 16 of A, brow = row c = lane % 16 of B.  K % 16 == 0.
__device__ __forceinline__ floatx4 mm_rowrow_bf16(floatx4 acc, const bf16_t* arow,
                                                   const bf16_t* brow, int K, int lane) {
  const int g = lane >> 4;
  int k0 = 0;
  for (; k0 + 32 <= K; k0 += 32) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + k0 + 8 * g);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(brow + k0 + 8 * g);
    acc = mfma_k32(a, b, acc);
  }
  if (k0 < K) {
    const shortx4 a = *reinterpret_cast<const shortx4*>(arow + k0 + 4 * g);
    const shortx4 b = *reinterpret_cast<const shortx4*>(brow + k0 + 4 * g);
    acc = mfma_k16(a, b, acc);
  }
  return acc;
}
__device__ __forceinline__ floatx4 mm_rowrow_f32(floatx4 acc, const float* arow,
                                                  const float* brow, int K, int lane) {
  const int g = lane >> 4;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const float4 a = *reinterpret_cast<const float4*>(arow + k0 + 4 * g);
    const float4 b = *reinterpret_cast<const float4*>(brow + k0 + 4 * g);
    acc = mfma_f32(a.x, b.x, acc);
    acc = mfma_f32(a.y, b.y, acc);
    acc = mfma_f32(a.z, b.z, acc);
    acc = mfma_f32(a.w, b.w, acc);
  }
  return acc;
}

}  // namespace linattn
