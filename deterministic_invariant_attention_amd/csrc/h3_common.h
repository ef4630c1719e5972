// Shared definitions of libh3attn: tile sizes, workspace layout, vector types, rounding helpers and
// the one RMSNorm arithmetic that both the standalone q/k norm and the attention prologue use.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace h3 {

constexpr int HD = 128;  // head dim (fixed by the H3 node: 128-wide heads)
constexpr int BQ = 256;  // queries per attention work item (8 waves x 32 rows)
constexpr int BK = 64;   // keys per KV tile; the KV walk is in these tiles, ascending from the segment start

// ---------------------------------------------------------------- workspace
// [0, 256)            header: status bits, segment and work-item counts
// segtab              int32 [2*T]: (start, length) of each segment, in packing order
// items               int32 [2*(T + ceil(T/BQ))]: (segment, q-tile) work items
// khat                bf16 [H][T][128]: normed K (head-major, so a KV tile is contiguous)
// v16                 fp16 [H][T][128]: V converted to fp16 (head-major)
// qhat                bf16 [H][T][128]: normed Q (head-major, packed token order), with norm weights
struct WsHeader {
  int32_t status;  // OR of STATUS_* bits; reset by the plan kernel
  int32_t nseg;
  int32_t nitems;
  int32_t nbkt;     // backward plan: cost classes in the work order
  int32_t next[2];  // backward: work counters of the dq and the dk/dv kernel, reset by the plan kernel
  int32_t pad[58];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

constexpr int32_t STATUS_SEG_BIT = 1;    // segment ids decrease
constexpr int32_t STATUS_RANGE_BIT = 2;  // a finite |v| exceeds the fp16 range

struct WsLayout {
  size_t segtab, items, khat, v16, qhat, total;
  int64_t max_items;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline WsLayout ws_layout(int64_t T, int32_t H) {
  WsLayout w;
  w.max_items = T + (T + BQ - 1) / BQ;
  w.segtab = 256;
  w.items = w.segtab + align256((size_t)T * 8);
  w.khat = w.items + align256((size_t)w.max_items * 8);
  w.v16 = w.khat + align256((size_t)T * H * HD * 2);
  w.qhat = w.v16 + align256((size_t)T * H * HD * 2);
  w.total = w.qhat + align256((size_t)T * H * HD * 2);
  return w;
}

// ---------------------------------------------------------------- backward workspace
// [0, 256)   header: status bits, segment and work-item counts
// segtab     int32 [2*T]
// items      int32 [2*(T + ceil(T/BT))]: (segment, tile) work items, BT = 128 queries or keys
// qhat, khat bf16 [H][T][128]: normed q, k (head-major)      qhat16, khat16: the same in fp16
// vh, doh    bf16 [H][T][128]: v and dO (head-major)          do16: dO in fp16
// lse2       fp32 [H][T]: the forward's log-sum-exp in log2 units
// delta      fp32 [H][T]: D_i = sum_j P_ij dP_ij
// dwq, dwk   fp32 [max_items][H][128]: per-item partial sums of the norm-weight gradients
// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- scalar conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Two floats -> packed bf16x2, each rounded to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}
// Two floats -> packed fp16x2, each rounded to nearest even (v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// ---------------------------------------------------------------- the RMSNorm arithmetic
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
// Two mappings compute exactly this tree (IEEE addition is commutative, so both partners of a
// butterfly hold the same bits):
//   * 16 lanes per row, lane c holds chunk c: butterflies over lane xor 2, 4, 8, then 1;
//   * 2 lanes per row, lane half h holds chunks 2m+h (m = 0..7) as its local chunks 0..7: the local
//     tree ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)) is E (h = 0) or Odd (h = 1), then one exchange.
// Then ms = total / 128 (exact), r = 1 / sqrt(ms + eps) with correctly rounded FP64 sqrt and
// division, y_d = (x_d * r) * w_d with both products rounded to FP64, and q_d = bf16_rne(y_d).

__device__ __forceinline__ double chunk_sumsq(const float* x) {
  double p = (double)x[0] * (double)x[0];
#pragma unroll
  for (int i = 1; i < 8; i++) p = __builtin_fma((double)x[i], (double)x[i], p);
  return p;
}

__device__ __forceinline__ double tree8(const double* p) {
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
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

// Sum of squares for the 2-lanes-per-row mapping (partners are lane and lane ^ 32).
__device__ __forceinline__ double row_total_2lanes(const double* local_partials) {
  const double own = tree8(local_partials);
  return own + __shfl_xor(own, 32, 64);
}

// FP64 -> bf16 bit pattern, round to nearest even, in one step (no intermediate fp32 rounding).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double y) {
  const uint64_t b = __builtin_bit_cast(uint64_t, y);
  const uint32_t hi = (uint32_t)(b >> 32), lo = (uint32_t)b;
  const uint32_t sign = (hi >> 16) & 0x8000u;
  const uint32_t ed = (hi >> 20) & 0x7FFu;  // biased FP64 exponent
  if (ed == 0x7FFu) return sign | ((((hi & 0xFFFFFu) | lo) != 0) ? 0x7FC0u : 0x7F80u);
  if ((int)ed - 1023 + 127 >= 1) {
    // keep the exponent and the top 7 mantissa bits (bits 62..45); round on bits 44..0
    const uint32_t keep = (hi & 0x7FFFFFFFu) >> 13;
    const uint32_t guard = (hi >> 12) & 1u;
    const uint32_t sticky = (((hi & 0xFFFu) | lo) != 0) ? 1u : 0u;
    const uint32_t r = keep + (guard & (sticky | (keep & 1u)));  // a carry moves into the exponent
    const int e2 = (int)(r >> 7) - 1023 + 127;
    if (e2 >= 255) return sign | 0x7F80u;
    return sign | ((uint32_t)e2 << 7) | (r & 0x7Fu);
  }
  // |y| < 2^-126: bf16 subnormals are k * 2^-133; the scaling is exact, rint rounds half to even
  const double k = __builtin_rint(__builtin_fabs(y) * 0x1p133);
  return sign | (uint32_t)k;
}

// Unpack 8 bf16 (one 16-byte chunk) to floats (exact).
__device__ __forceinline__ void unpack8_bf16(const u32x4& w, float* x) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
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
