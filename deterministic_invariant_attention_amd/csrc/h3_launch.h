// Host-side launchers of the kernels (one per translation unit); argument checking happens before
// these are called, in the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

// Segment decode into the workspace header, segment table and work list.  Resets the status word.
hipError_t launch_plan(const int32_t* seg, int64_t T, void* ws, int32_t H, hipStream_t stream);

// Standalone q/k RMSNorm of [T, H, 128] bf16 rows (y may equal x).
hipError_t launch_qknorm(const void* x, const void* w, void* y, int64_t T, int32_t H, float eps, hipStream_t stream);

// Q -> normed bf16 Q (only with wq; head-major, packed token order), K -> normed bf16 K (or a copy
// when wk is NULL) and V -> fp16, both head-major at staged row slot[t] (position order) or, with
// slot NULL, at row t; all into the workspace.  With rope tables (float32 [T][48], only with the
// weights) the normed Q and K are rotated (MM-RoPE on 96 channels) and rounded again to bf16.
hipError_t launch_prep_qkv(const void* q, const void* k, const void* v, const void* wq, const void* wk, int64_t T,
                           int32_t H, float eps, void* ws, const int32_t* slot, const float* rope_cos,
                           const float* rope_sin, hipStream_t stream);

// Position ids -> slot / inv maps of the ordering area, with the permutation check (STATUS_POS_BIT,
// and the failing segments flagged in segflag).  Needs the plan's segment table and token map.
hipError_t launch_order(const int32_t* pos, int64_t T, void* ws, const int32_t* segtab, const int32_t* tok2seg,
                        int32_t* segflag, int32_t* slot, int32_t* inv, hipStream_t stream);

// Attention over the planned work items.  Queries: the staged normed Q when normed is true, else
// the caller's q (token-major).  lse and o32 (the output before its bf16 rounding, fp32) are
// optional, and so is status_out (device int32: receives the call's data-error code).  grid_cap:
// most workgroups to launch (persistent grid).
hipError_t launch_attend(const void* q, bool normed, int64_t T, int32_t H, float scale, void* out, float* lse,
                         float* o32, int32_t* status_out, void* ws, int grid_cap, hipStream_t stream);

// Backward: segment decode with 128-token tiles into the backward workspace.
hipError_t launch_plan_bwd(const int32_t* seg, int64_t T, void* ws, int32_t H, hipStream_t stream);

// Backward operand staging (normed q/k, v and dO in fp16, LSE in log2 units), at staged rows slot[t]
// or, with slot NULL, at the token's own row.  With o32 (the forward's fp32 output) it also writes
// D = dO . O per row, and the dq kernel then skips its first pass.  Rope tables as for
// launch_prep_qkv.
hipError_t launch_bwd_prep(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           const float* o32, const void* wq, const void* wk, int64_t T, int32_t H, float eps, void* ws,
                           const int32_t* slot, const float* rope_cos, const float* rope_sin, hipStream_t stream);

// Backward attention on the staged operands: dq with D, then dk/dv; with norm weights, the norm
// backward (16-row weight-gradient partials in staged order) and the fixed-order reduction of the
// partials into dwq/dwk.  q and k are the raw inputs (the norm backward reads them).  inv maps a
// staged row to its token (position order) or is NULL.
hipError_t launch_bwd(const void* q, const void* k, const void* wq, const void* wk, int64_t T, int32_t H, float eps,
                      float scale, void* dq, void* dk, void* dv, float* dwq, float* dwk, void* ws, const int32_t* inv,
                      bool delta_ready, const float* rope_cos, const float* rope_sin, int grid_cap,
                      hipStream_t stream);

}  // namespace h3
