// Position-ordered traversal (h3attn_fwd_pos, h3attn_bwd_pos): per-token position ids within each
// segment decide where a token's staged rows live, so every sum over keys (and, in the backward,
// over queries and over rows) runs in position order, whatever order the tokens were packed in.
// The "ws1_one_h3_block + full-model qualification" page (Results, control H-C3) reports that
// permuting packed rows with their positions changes output bits because keys are summed in packed
// order, and leaves that to the attention; this is the attention taking it.
//
// Workspace: the ordering area follows the plain layout of the forward or the backward.
//   slot  int32 [T]: token t -> staged row s0 + pos[t] (t itself when pos[t] is out of range)
//   inv   int32 [T]: staged row -> token (valid once the check has passed)
#pragma once

#include "h3_common.h"

namespace h3 {

struct OrderLayout {
  size_t slot, inv, total;
};

// base: the size of the plain layout the ordering area is appended to
__host__ __device__ inline OrderLayout order_layout(size_t base, int64_t T) {
  OrderLayout o;
  o.slot = align256(base);
  o.inv = o.slot + align256((size_t)T * 4);
  o.total = o.inv + align256((size_t)T * 4);
  return o;
}

}  // namespace h3
