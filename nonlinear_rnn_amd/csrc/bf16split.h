// fp32 products on the bf16 matrix cores.
//
// An fp32 value v splits exactly into three bf16 terms, v = hi + mid + lo:
// hi keeps the sign, the exponent and the top 7 stored mantissa bits of v
// (truncation); v - hi is exact in fp32 and has at most 16 significant
// bits, whose top 8 make mid; the rest, lo = v - hi - mid, has at most 8 and
// is a bf16 exactly.  A product a b is then the sum of the nine products of
// the terms, each exact in fp32; the six with combined weight 2^-16 or more
// (a_u b_v with u + v <= 2, hi = 0) carry it to within 3 * 2^-24 |a b|,
// below the rounding of an fp32 product.  On CDNA4 a 32 x 32 x 16 bf16
// matrix instruction takes half the cycles of eight 32 x 32 x 2 fp32 ones
// over the same 16 k, so six of them cover 16 k in 3/8 of the fp32 time.
// Non-finite inputs give non-finite sums (an infinite term minus itself is
// NaN), not necessarily the ones an fp32 product would give.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prn {

typedef __attribute__((ext_vector_type(8))) __bf16 sp_bf16x8;
typedef __attribute__((ext_vector_type(4))) float sp_f32x4;

// The three terms of eight fp32 values va[0..3], vb[0..3]; term e of each
// bf16x8 belongs to element e of (va, vb).
__device__ __forceinline__ void split3(const sp_f32x4& va, const sp_f32x4& vb, sp_bf16x8& hi, sp_bf16x8& mid,
                                       sp_bf16x8& lo) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  u32x4 h, m, l;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float v0 = p < 2 ? va[2 * p] : vb[2 * p - 4];
    const float v1 = p < 2 ? va[2 * p + 1] : vb[2 * p - 3];
    const uint32_t b0 = __float_as_uint(v0), b1 = __float_as_uint(v1);
    const float r0 = v0 - __uint_as_float(b0 & 0xffff0000u), r1 = v1 - __uint_as_float(b1 & 0xffff0000u);
    const uint32_t c0 = __float_as_uint(r0), c1 = __float_as_uint(r1);
    const float q0 = r0 - __uint_as_float(c0 & 0xffff0000u), q1 = r1 - __uint_as_float(c1 & 0xffff0000u);
    const uint32_t d0 = __float_as_uint(q0), d1 = __float_as_uint(q1);
    h[p] = (b1 & 0xffff0000u) | (b0 >> 16);
    m[p] = (c1 & 0xffff0000u) | (c0 >> 16);
    l[p] = (d1 & 0xffff0000u) | (d0 >> 16);
  }
  hi = __builtin_bit_cast(sp_bf16x8, h);
  mid = __builtin_bit_cast(sp_bf16x8, m);
  lo = __builtin_bit_cast(sp_bf16x8, l);
}

// the six term pairs (u, v) of a product, in the order both the projection
// kernel and the fused Newton tile accumulate them
constexpr int kSplitU[6] = {0, 0, 1, 0, 1, 2};
constexpr int kSplitV[6] = {0, 1, 0, 2, 1, 0};

}  // namespace prn
