// The RMSNorm arithmetic of the q_norm / k_norm node (RMSNorm over each 128-wide head with one
// 128-element weight shared by all heads: "ws1_one_h3_block" page, Bindings table and Results),
// shared by every kernel that norms or back-propagates through the norm.
#pragma once

#include "h3_common.h"

namespace h3 {

// The norm's output is a quantised code (bf16), so the rounding decision is taken in FP64: the
// normalised value is computed in double precision and rounded ONCE, to nearest even, to bf16.
// Every input is a bf16 value, so x^2 is exact in FP64 and the sum of squares is exact for any
// realistic dynamic range; the result is then the correctly rounded bf16 of the FP64 value.
//
// A 128-wide row is 16 chunks of 8 channels (chunk c = channels 8c..8c+7).  The sum of squares is
// evaluated in ONE fixed expression tree, whatever the thread mapping:
//   p_c   = x_{8c}^2, then p_c = fma(x_{8c+i}, x_{8c+i}, p_c) for i = 1..7     (chunk partial)
//   E     = ((p0 + p2) + (p4 + p6)) + ((p8 + p10) + (p12 + p14))              (even chunks)
//   Odd   = ((p1 + p3) + (p5 + p7)) + ((p9 + p11) + (p13 + p15))              (odd chunks)
//   total = E + Odd
// With 16 lanes per row, lane c holding chunk c, butterflies over lane xor 2, 4, 8, then 1 compute
// exactly this tree (IEEE addition is commutative, so both partners of a butterfly hold the same
// bits).
// Then ms = total / 128 (exact), r = 1 / sqrt(ms + eps) with correctly rounded FP64 sqrt and
// division, y_d = (x_d * r) * w_d with both products rounded to FP64, and q_d = bf16_rne(y_d).

__device__ __forceinline__ double chunk_sumsq(const float* x) {
  double p = (double)x[0] * (double)x[0];
#pragma unroll
  for (int i = 1; i < 8; i++) p = __builtin_fma((double)x[i], (double)x[i], p);
  return p;
}

__device__ __forceinline__ double norm_rscale(double total, float eps) {
  const double ms = total * 0.0078125;
  return __ddiv_rn(1.0, __dsqrt_rn(ms + (double)eps));
}

// Sum of squares for the 16-lanes-per-row mapping (lanes of one row: a 16-aligned lane group).
__device__ __forceinline__ double row_total_16lanes(double p) {
  p = p + __shfl_xor(p, 2, 64);
  p = p + __shfl_xor(p, 4, 64);
  p = p + __shfl_xor(p, 8, 64);
  p = p + __shfl_xor(p, 1, 64);
  return p;
}

// FP64 -> bf16 bit pattern, round to nearest even, in one step (no intermediate fp32 rounding).
// |y| is rounded onto the bf16 grid of its binade by one add and one subtract of
// c = 1.5 * 2^(e + 45), e = the binade's exponent clamped to [-126, 128]: the sum lies in c's
// binade, whose spacing 2^(e - 7) is the bf16 spacing at |y| (2^-133 below 2^-126, the bf16
// subnormals), so the IEEE adder rounds |y| to nearest with ties to an even multiple, which is the
// even bf16 mantissa, and the subtraction is exact.  The result converts to fp32 exactly (or to
// infinity past the bf16 range) and its top half is the bf16 pattern; NaN becomes the quiet NaN.
// No branches: every element of a lane takes the same instructions.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double y) {
  const uint64_t b = __builtin_bit_cast(uint64_t, y);
  const uint32_t hi = (uint32_t)(b >> 32);
  const uint32_t sign = (hi >> 16) & 0x8000u;
  const int ed = (int)((hi >> 20) & 0x7FFu);  // biased FP64 exponent
  int e = ed - 1023;
  e = e < -126 ? -126 : (e > 128 ? 128 : e);
  const double c = __builtin_bit_cast(double, ((uint64_t)(e + 1068) << 52) | (1ull << 51));
  const double a = __builtin_bit_cast(double, b & 0x7FFFFFFFFFFFFFFFull);
  const double r = (a + c) - c;
  uint32_t out = __builtin_bit_cast(uint32_t, (float)r) >> 16;
  if (ed == 0x7FF && (b << 12) != 0) out = 0x7FC0u;
  return sign | out;
}

// Normalise one 8-channel chunk with the row's scale r and the chunk's weights; pack to bf16.
__device__ __forceinline__ u32x4 norm_chunk(const float* x, const float* w, double r) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const double y0 = ((double)x[2 * i] * r) * (double)w[2 * i];
    const double y1 = ((double)x[2 * i + 1] * r) * (double)w[2 * i + 1];
    o[i] = f64_to_bf16_rne(y0) | (f64_to_bf16_rne(y1) << 16);
  }
  return o;
}

}  // namespace h3
