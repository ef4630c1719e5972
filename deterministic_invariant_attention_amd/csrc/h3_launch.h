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

}  // namespace h3
