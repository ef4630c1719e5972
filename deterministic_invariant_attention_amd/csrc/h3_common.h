// Shared definitions of libh3attn: tile sizes, workspace layouts, vector types and rounding helpers.
// (The RMSNorm arithmetic is in h3_norm.h.)
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "h3attn.h"

namespace h3 {

constexpr int HD = 128;  // head dim (fixed by the H3 node: 128-wide heads)
constexpr int BQ = 256;  // queries per attention work item (8 waves x 32 rows)
constexpr int BK = 96;   // keys per KV tile; the KV walk is in these tiles, ascending from the segment start

// ---------------------------------------------------------------- workspace
// [0, 256)            header: status bits, segment and work-item counts
// segtab              int32 [2*T]: (start, length) of each segment, in packing order
// items               int32 [4*(T + ceil(T/BQ))]: (segment, q-tile, segment start, length) work items
// khat                bf16 [H][T][128]: normed K (head-major, so a KV tile is contiguous)
// v16                 fp16 [H][T][128]: V converted to fp16 (head-major)
// qhat                bf16 [H][T][128]: normed Q (head-major, packed token order), with norm weights
// tok2seg             int32 [T]: the segment (index into segtab) of every token
// segflag             int32 [T]: per segment, nonzero when one of its values cannot enter the
//                     products (a finite |v| beyond fp16) or its position ids are not a permutation;
//                     that segment's outputs are NaN, the others are computed as usual
// sched               the attention kernel's work counters (SCHED_BYTES, below)
// bkt                 int32 [2*NBKT]: first item and count of each cost class of the work order
struct WsHeader {
  int32_t status;  // OR of STATUS_* bits; reset by the plan kernel
  int32_t nseg;
  int32_t nitems;
  int32_t nbkt;     // backward plan: cost classes in the work order
  int32_t next[2];  // backward: work counters of the dq and the dk/dv kernel, reset by the plan kernel
  int32_t pad[58];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

constexpr int32_t STATUS_SEG_BIT = 1;    // segment ids decrease (no segmentation exists: every output is NaN)
constexpr int32_t STATUS_RANGE_BIT = 2;  // a finite |v| exceeds the fp16 range (in the flagged segments)

// The forward attention kernel's work queues, at the end of the forward workspace: one counter per
// XCD, each on its own 128-byte line (int index SCHED_STRIDE * x), and the count of workgroups that
// have left the work loop (index SCHED_DONE).  All zero between launches.
constexpr size_t SCHED_BYTES = 2048;
constexpr int SCHED_STRIDE = 32;
constexpr int SCHED_DONE = 8 * SCHED_STRIDE;

constexpr int NBKT = 32;  // cost classes of a work order: floor(log2(64-row tiles of the segment))

struct WsLayout {
  size_t segtab, items, khat, v16, qhat, tok2seg, segflag, sched, bkt, total;
  int64_t max_items;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline WsLayout ws_layout(int64_t T, int32_t H) {
  WsLayout w;
  w.max_items = T + (T + BQ - 1) / BQ;
  w.segtab = 256;
  w.items = w.segtab + align256((size_t)T * 8);
  w.khat = w.items + align256((size_t)w.max_items * 16);
  w.v16 = w.khat + align256((size_t)T * H * HD * 2);
  w.qhat = w.v16 + align256((size_t)T * H * HD * 2);
  w.tok2seg = w.qhat + align256((size_t)T * H * HD * 2);
  w.segflag = w.tok2seg + align256((size_t)T * 4);
  w.sched = w.segflag + align256((size_t)T * 4);
  w.bkt = w.sched + SCHED_BYTES;
  w.total = w.bkt + align256((size_t)NBKT * 2 * 4);
  return w;
}

constexpr int32_t STATUS_POS_BIT = 4;  // position ids are not a permutation of 0..L-1 in some segment

// The status code of a status word (the H3ATTN_ERR_* data errors, in this order of precedence).
__host__ __device__ inline int32_t status_code(int32_t bits) {
  return (bits & STATUS_SEG_BIT)     ? H3ATTN_ERR_SEGMENTS
         : (bits & STATUS_POS_BIT)   ? H3ATTN_ERR_POSITIONS
         : (bits & STATUS_RANGE_BIT) ? H3ATTN_ERR_RANGE
                                     : H3ATTN_OK;
}

// Mark segment sg as unusable (per-segment fail-closed; the caller also sets the status bit).
__device__ __forceinline__ void flag_segment(int32_t* segflag, int32_t sg, int32_t nseg) {
  if (sg >= 0 && sg < nseg) atomicOr(&segflag[sg], 1);
}

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

// Unpack 8 bf16 (one 16-byte chunk) to floats (exact).
__device__ __forceinline__ void unpack8_bf16(const u32x4& w, float* x) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

}  // namespace h3
