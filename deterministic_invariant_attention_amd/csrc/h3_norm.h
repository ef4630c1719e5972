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

// FP64 -> bf16, round to nearest even, correctly rounded (as if rounded once from the FP64 value).
// Two steps: y is first rounded to fp32 "to odd" (toward zero, with the last bit set when the
// conversion is inexact), then that fp32 is rounded to bf16, nearest even, by the hardware
// conversion.  Rounding to odd into a format with at least two more significand bits keeps the
// information a later nearest-even rounding needs (fp32 has 24 bits against bf16's 8, and 16 more
// bits in the subnormal range), so the two roundings give the one correct rounding of y.
// The fp32 step: t = fp32(y) to nearest; r = y - t is exact in FP64 (at most 29 significant bits);
// when r != 0 the conversion was inexact, and when r and y differ in sign t lies farther from zero
// than y, so the value toward zero is the fp32 one step below t in magnitude (t's bit pattern - 1;
// for t = infinity that is the largest finite fp32, which then rounds to bf16 infinity).  Exact
// values (r == 0), infinities and NaN (r unordered) keep t.  No branches.
__device__ __forceinline__ float f64_to_f32_odd(double y) {
  const float t = (float)y;
  const double r = y - (double)t;
  const uint32_t inexact = (r < 0.0 || r > 0.0) ? 1u : 0u;
  const uint32_t away =
      (uint32_t)((__builtin_bit_cast(uint64_t, r) ^ __builtin_bit_cast(uint64_t, y)) >> 63) & inexact;
  return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, t) - away) | inexact);
}

// Two FP64 values -> packed bf16x2 (first value in the low half), each correctly rounded.
__device__ __forceinline__ uint32_t f64x2_to_bf16x2_rne(double y0, double y1) {
  return pack_bf16(f64_to_f32_odd(y0), f64_to_f32_odd(y1));
}

// Normalise one 8-channel chunk with the row's scale r and the chunk's weights; pack to bf16.
__device__ __forceinline__ u32x4 norm_chunk(const float* x, const float* w, double r) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const double y0 = ((double)x[2 * i] * r) * (double)w[2 * i];
    const double y1 = ((double)x[2 * i + 1] * r) * (double)w[2 * i + 1];
    o[i] = f64x2_to_bf16x2_rne(y0, y1);
  }
  return o;
}

// ---------------------------------------------------------------- MM-RoPE (partial)
// The rope node between the norm and the attention rotates 96 of the 128 channels ("ws1_one_h3_block"
// page, Bindings table: rope_q/rope_k; Tests: 96 of 128 channels).  Table-driven: per token, the
// cosine and sine (float32) of each of the 48 rotated pairs; pair i is channels (2i, 2i+1):
//   y_2i = x_2i cos_i - x_2i+1 sin_i,   y_2i+1 = x_2i sin_i + x_2i+1 cos_i,
// channels 96..127 unchanged.  The products of a bf16 and a float32 value are exact in FP64, so each
// output is one FP64 rounding of the exact expression, then one correct rounding to bf16 (the
// node's output dtype): the same bits as any FP64 evaluation in this order.
constexpr int ROPE_PAIRS = 48;
constexpr int ROPE_CHUNKS = ROPE_PAIRS / 4;  // 8-channel chunks touched by the rotation (0..11)

// Rotate one 8-channel chunk (4 pairs) of bf16 values x with the chunk's 4 cosines and sines.
__device__ __forceinline__ u32x4 rope_chunk(const u32x4& x, const f32x4& cs, const f32x4& sn) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const double a = (double)bf16_lo(x[j]), b = (double)bf16_hi(x[j]);
    const double c = (double)cs[j], s = (double)sn[j];
    o[j] = f64x2_to_bf16x2_rne(a * c - b * s, a * s + b * c);
  }
  return o;
}

// The transposed rotation of one chunk of a gradient (FP64 in and out):
//   dx_2i = dy_2i cos_i + dy_2i+1 sin_i,   dx_2i+1 = dy_2i+1 cos_i - dy_2i sin_i.
__device__ __forceinline__ void rope_chunk_transpose(double* dy, const f32x4& cs, const f32x4& sn) {
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const double a = dy[2 * j], b = dy[2 * j + 1];
    const double c = (double)cs[j], s = (double)sn[j];
    dy[2 * j] = a * c + b * s;
    dy[2 * j + 1] = b * c - a * s;
  }
}

}  // namespace h3
