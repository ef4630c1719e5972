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

// K -> normed bf16 K (or a copy when wk is NULL) and V -> fp16, both head-major, into the workspace.
hipError_t launch_prep_kv(const void* k, const void* v, const void* wk, int64_t T, int32_t H, float eps, void* ws,
                          hipStream_t stream);

// Attention over the planned work items with the Q norm fused into the load prologue.
// grid_cap: most workgroups to launch (persistent grid).
hipError_t launch_attend(const void* q, const void* wq, int64_t T, int32_t H, float eps, float scale, void* out,
                         float* lse, void* ws, int grid_cap, hipStream_t stream);

// Backward: segment decode with 128-token tiles into the backward workspace.
hipError_t launch_plan_bwd(const int32_t* seg, int64_t T, void* ws, int32_t H, hipStream_t stream);

// Backward operand staging (normed q/k in bf16 and fp16, v, dO in bf16 and fp16, LSE in log2 units).
hipError_t launch_bwd_prep(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           const void* wq, const void* wk, int64_t T, int32_t H, float eps, void* ws,
                           hipStream_t stream);

// Backward attention on the staged operands: dq with D, then dk/dv (each with its norm backward and
// per-item weight-gradient partials), then the fixed-order reduction of the partials into dwq/dwk
// when the weights are given.  q and k are the raw inputs (the norm backward reads them).
hipError_t launch_bwd(const void* q, const void* k, const void* wq, const void* wk, int64_t T, int32_t H, float eps,
                      float scale, void* dq, void* dk, void* dv, float* dwq, float* dwk, void* ws, int grid_cap,
                      hipStream_t stream);

}  // namespace h3
