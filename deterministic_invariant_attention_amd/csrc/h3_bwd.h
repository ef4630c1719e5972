// Workspace layout and work decomposition of the backward (h3attn_bwd).
#pragma once

#include "h3_common.h"

namespace h3 {

constexpr int BT = 128;        // queries (dq kernel) or keys (dk/dv kernel) per backward work item
constexpr int NR = 16;         // rows (token, head) per workgroup of the norm backward
constexpr int DW_CHUNK = 64;   // partials per chunk of the weight-gradient reduction

constexpr int NBKT = 32;  // cost classes of the backward work order (floor(log2(64-row tiles)))

// Backward workspace (h3attn_bwd_workspace_bytes):
// [0, 256)          header: status bits, segment and work-item counts, work counters
// segtab            int32 [2*T]
// items             int32 [2*(T + ceil(T/BT))]: (segment, tile) work items
// bkt               int32 [2*NBKT]: first item and count of each cost class in the work order
// qhat16, khat16    fp16 [H][T][128]: normed q, k (head-major, staged row order)
// v16, do16         fp16 [H][T][128]: v and dO
// lse2              fp32 [H][T]: the forward's log-sum-exp in log2 units
// delta             fp32 [H][T]: -D_i, D_i = sum_j P_ij dP_ij (the dq kernel's dP products start from it)
// dqh, dkh          fp32 [T][H][128]: dq^, dk^ (gradients of the normed operands)
// dw_part, dw_chunk fp32: 16-row weight-gradient partials and their first-level chunk sums
struct BwdLayout {
  size_t segtab, items, bkt, qhat16, khat16, v16, do16, lse2, delta, dqh, dkh, dw_part, dw_chunk, total;
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
  w.bkt = w.items + align256((size_t)w.max_items * 8);
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
  w.total = w.dw_chunk + align256((size_t)2 * w.nchunks * HD * 4);
  return w;
}

}  // namespace h3
