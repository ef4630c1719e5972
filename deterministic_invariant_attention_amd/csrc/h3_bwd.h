// Workspace layout and work decomposition of the backward (h3attn_bwd).
#pragma once

#include "h3_common.h"

namespace h3 {

constexpr int BT = 128;        // queries (dq kernel) or keys (dk/dv kernel) per backward work item
constexpr int NR = 16;         // rows (token, head) per workgroup of the norm backward
constexpr int DW_CHUNK = 64;   // partials per chunk of the weight-gradient reduction

// Backward workspace (h3attn_bwd_workspace_bytes):
// [0, 256)          header: status bits, segment and work-item counts, work counters
// segtab            int32 [2*T]
// items             int32 [4*(T + ceil(T/BT))]: (segment, tile, segment start, length) work items
// bkt               int32 [2*NBKT]: first item and count of each cost class in the work order
// qhat16, khat16    fp16 [H][T][128]: normed q, k (head-major, staged row order)
// v16, do16         fp16 [H][T][128]: v and dO
// lse2              fp32 [H][T]: the forward's log-sum-exp in log2 units
// delta             fp32 [H][T]: -D_i, D_i = sum_j P_ij dP_ij (the dq kernel's dP products start from it)
// dqh, dkh          fp32 [T][H][128]: dq^, dk^ (gradients of the normed operands)
// dw_part, dw_chunk fp32: 16-row weight-gradient partials and their first-level chunk sums
// tok2seg           int32 [T]: the segment (index into segtab) of every token
// segflag           int32 [T]: per segment, nonzero when it cannot be computed (see the forward's)
// dmax              uint32 [T][H]: per (segment, head), the largest |dO| as bf16 magnitude bits
//                   (slots [0, nseg*H) are used; reset by the plan kernel)
struct BwdLayout {
  size_t segtab, items, bkt, qhat16, khat16, v16, do16, lse2, delta, dqh, dkh, dw_part, dw_chunk, tok2seg, segflag,
      dmax, total;
  int64_t max_items, nparts, nchunks;
};

__host__ __device__ inline BwdLayout bwd_layout(int64_t T, int32_t H) {
  BwdLayout w;
  const size_t tens = align256((size_t)T * H * HD * 2);
  const size_t tens32 = align256((size_t)T * H * HD * 4);
  const size_t rowf = align256((size_t)T * H * 4);
  w.max_items = T + (T + BT - 1) / BT;
  w.nparts = (T * H + NR - 1) / NR;
  w.nchunks = (w.nparts + DW_CHUNK - 1) / DW_CHUNK;
  w.segtab = 256;
  w.items = w.segtab + align256((size_t)T * 8);
  w.bkt = w.items + align256((size_t)w.max_items * 16);
  w.qhat16 = w.bkt + align256((size_t)NBKT * 2 * 4);
  w.khat16 = w.qhat16 + tens;
  w.v16 = w.khat16 + tens;
  w.do16 = w.v16 + tens;
  w.lse2 = w.do16 + tens;
  w.delta = w.lse2 + rowf;
  w.dqh = w.delta + rowf;
  w.dkh = w.dqh + tens32;
  w.dw_part = w.dkh + tens32;
  w.dw_chunk = w.dw_part + align256((size_t)2 * w.nparts * HD * 4);
  w.tok2seg = w.dw_chunk + align256((size_t)2 * w.nchunks * HD * 4);
  w.segflag = w.tok2seg + align256((size_t)T * 4);
  w.dmax = w.segflag + align256((size_t)T * 4);
  w.total = w.dmax + align256((size_t)T * H * 4);
  return w;
}

// The power of two that scales dO before it enters the fp16 products of the backward.  fp16 keeps
// bf16's 8 significant bits only from 2^-14 (2^-17 with its subnormals) up to 65504, while dO may
// lie anywhere in bf16's range; so every (segment, head) is scaled by 2^s chosen from its own
// largest |dO| (m, bf16 magnitude bits) to bring that maximum into [4, 8) -- the range of N(0, 1)
// draws, which gets s = 0.  Every gradient is linear in dO, so the epilogues remove the factor
// exactly (ldexp by -s).  m = 0, infinity or NaN: s = 0 (infinities and NaN propagate unscaled).
__host__ __device__ inline int dout_scale_exp(uint32_t m) {
  if (m == 0 || m >= 0x7F80u) return 0;
  const int e = (int)(m >> 7);
  int fl;  // floor(log2(m's value))
  if (e > 0) {
    fl = e - 127;
  } else {  // subnormal: value = mantissa * 2^-133
    int top = 6;
    while (!((m >> top) & 1u)) top--;
    fl = top - 133;
  }
  return 2 - fl;
}

}  // namespace h3
