// C ABI of libh3attn (declared and documented in include/h3attn.h): argument checks, workspace
// carve-up and kernel launches.  Strict mode of the H3 pages ("33B forward/backward" page, Scope):
// unsupported shapes, dtypes and devices raise instead of falling back -- every check below returns
// an error before anything is enqueued, and there is no other code path.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "h3_common.h"
#include "h3_bwd.h"
#include "h3_launch.h"
#include "h3_order.h"
#include "h3attn.h"

namespace {

using namespace h3;

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  bool ok = false;
  int cus = 0;
};

std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];

// Current device must be gfx950.  The properties are read once per device and cached.
int device_info(DeviceInfo* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return H3ATTN_ERR_DEVICE;
  }
  std::call_once(g_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    g_info[dev].ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_info[dev].cus = prop.multiProcessorCount;
  });
  if (!g_info[dev].ok) return H3ATTN_ERR_DEVICE;
  *out = g_info[dev];
  return H3ATTN_OK;
}

// The workspace of h3attn_fwd_noalloc, for callers that cannot allocate: a fixed array in device
// memory that every GPU the library runs on holds until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = (size_t)256 << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];

// The current device's address of `scratch` (resolved on the first call on that device).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return H3ATTN_ERR_DEVICE;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
    }
    g_scratch[dev] = p;
  });
  if (!g_scratch[dev]) return H3ATTN_ERR_LAUNCH;
  *out = g_scratch[dev];
  return H3ATTN_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Shape checks shared by every entry point; also bounds the index arithmetic of the kernels.
int check_shape(int64_t T, int32_t H, int32_t D) {
  if (T < 0 || H < 1 || D != HD) return H3ATTN_ERR_SHAPE;
  if (T > ((int64_t)1 << 28)) return H3ATTN_ERR_SHAPE;  // keeps every int32 index product of the kernels in range
  const int64_t max_items = T + (T + BQ - 1) / BQ;
  if (max_items * (int64_t)H > (int64_t)INT32_MAX) return H3ATTN_ERR_SHAPE;
  if ((T * H * 16 + 255) / 256 > (int64_t)INT32_MAX) return H3ATTN_ERR_SHAPE;
  return H3ATTN_OK;
}

int launch_status(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return H3ATTN_ERR_LAUNCH;
  }
  return H3ATTN_OK;
}

size_t tensor_bytes(int64_t T, int32_t H) { return (size_t)T * (size_t)H * HD * 2; }

}  // namespace

extern "C" {

int h3attn_version(void) { return H3ATTN_VERSION; }

const char* h3attn_strerror(int status) {
  switch (status) {
    case H3ATTN_OK: return "ok";
    case H3ATTN_ERR_NULL: return "a required pointer is NULL (or exactly one of wq/wk is NULL)";
    case H3ATTN_ERR_SHAPE: return "unsupported shape (tokens < 0, heads < 1, head_dim != 128, or too large)";
    case H3ATTN_ERR_ALIGN: return "misaligned buffer (tensors 16 B, seg_ids/lse 4 B, workspace 256 B)";
    case H3ATTN_ERR_ALIAS: return "an output overlaps an input or the workspace";
    case H3ATTN_ERR_WORKSPACE: return "workspace too small";
    case H3ATTN_ERR_DEVICE: return "no current device or it is not gfx950 (MI355X)";
    case H3ATTN_ERR_LAUNCH: return "the HIP runtime rejected a launch or copy";
    case H3ATTN_ERR_SEGMENTS: return "segment ids decrease (device status)";
    case H3ATTN_ERR_RANGE: return "a finite value beyond 65504 cannot enter an fp16 product (device status)";
    case H3ATTN_ERR_POSITIONS: return "position ids are not a permutation of 0..L-1 in some segment (device status)";
    case H3ATTN_ERR_SCRATCH:
      return "h3attn_workspace_bytes(tokens, heads) exceeds the 256 MiB static scratch of h3attn_fwd_noalloc";
    default: return "unknown status";
  }
}

// Large enough for both h3attn_fwd and h3attn_fwd_pos (the ordering area follows the plain layout).
size_t h3attn_workspace_bytes(int64_t tokens, int32_t heads) {
  if (check_shape(tokens, heads, HD) != H3ATTN_OK) return 0;
  return order_layout(ws_layout(tokens, heads).total, tokens).total;
}

int h3attn_qknorm(const void* x, const void* w, void* y, int64_t tokens, int32_t heads, int32_t head_dim, float eps,
                  void* stream) {
  int rc = check_shape(tokens, heads, head_dim);
  if (rc) return rc;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return H3ATTN_ERR_SHAPE;
  if (tokens == 0) return H3ATTN_OK;
  if (!x || !w || !y) return H3ATTN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return H3ATTN_ERR_ALIGN;
  const size_t n = tensor_bytes(tokens, heads);
  if (x != y && overlap(x, n, y, n)) return H3ATTN_ERR_ALIAS;
  if (overlap(w, HD * 2, y, n)) return H3ATTN_ERR_ALIAS;
  DeviceInfo di;
  if ((rc = device_info(&di))) return rc;
  return launch_status(launch_qknorm(x, w, y, tokens, heads, eps, (hipStream_t)stream));
}

// ---- argument checks of the three stages (no device access; nothing is enqueued)

static int check_plan(const int32_t* seg_ids, int64_t tokens, int32_t heads, void* workspace, size_t workspace_bytes) {
  if (!seg_ids || !workspace) return H3ATTN_ERR_NULL;
  if (!aligned(seg_ids, 4) || !aligned(workspace, 256)) return H3ATTN_ERR_ALIGN;
  if (overlap(seg_ids, (size_t)tokens * 4, workspace, workspace_bytes)) return H3ATTN_ERR_ALIAS;
  if (workspace_bytes < ws_layout(tokens, heads).total) return H3ATTN_ERR_WORKSPACE;
  return H3ATTN_OK;
}

static int check_prep(const void* q, const void* k, const void* v, const void* wq, const void* wk, int64_t tokens,
                      int32_t heads, float eps, void* workspace, size_t workspace_bytes) {
  if ((wq == nullptr) != (wk == nullptr)) return H3ATTN_ERR_NULL;
  if (wk && (!(eps > 0.0f) || !std::isfinite(eps))) return H3ATTN_ERR_SHAPE;
  if (!q || !k || !v || !workspace) return H3ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || (wq && !aligned(wq, 16)) || (wk && !aligned(wk, 16)) ||
      !aligned(workspace, 256))
    return H3ATTN_ERR_ALIGN;
  const size_t n = tensor_bytes(tokens, heads);
  if (overlap(q, n, workspace, workspace_bytes) || overlap(k, n, workspace, workspace_bytes) ||
      overlap(v, n, workspace, workspace_bytes) || overlap(wq, HD * 2, workspace, workspace_bytes) ||
      overlap(wk, HD * 2, workspace, workspace_bytes))
    return H3ATTN_ERR_ALIAS;
  if (workspace_bytes < ws_layout(tokens, heads).total) return H3ATTN_ERR_WORKSPACE;
  return H3ATTN_OK;
}

static int check_attend(const void* q, const void* wq, int64_t tokens, int32_t heads, float eps, float scale,
                        void* out, float* lse, void* workspace, size_t workspace_bytes) {
  if (wq && (!(eps > 0.0f) || !std::isfinite(eps))) return H3ATTN_ERR_SHAPE;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return H3ATTN_ERR_SHAPE;
  if (!q || !out || !workspace) return H3ATTN_ERR_NULL;
  if (!aligned(q, 16) || (wq && !aligned(wq, 16)) || !aligned(out, 16) || (lse && !aligned(lse, 4)) ||
      !aligned(workspace, 256))
    return H3ATTN_ERR_ALIGN;
  const size_t n = tensor_bytes(tokens, heads);
  const size_t nl = (size_t)tokens * heads * 4;
  if (overlap(out, n, q, n) || overlap(out, n, wq, HD * 2) || overlap(out, n, workspace, workspace_bytes) ||
      overlap(out, n, lse, nl) || overlap(lse, nl, q, n) || overlap(lse, nl, wq, HD * 2) ||
      overlap(lse, nl, workspace, workspace_bytes))
    return H3ATTN_ERR_ALIAS;
  if (workspace_bytes < ws_layout(tokens, heads).total) return H3ATTN_ERR_WORKSPACE;
  return H3ATTN_OK;
}

int h3attn_plan(const int32_t* seg_ids, int64_t tokens, int32_t heads, void* workspace, size_t workspace_bytes,
                void* stream) {
  int rc = check_shape(tokens, heads, HD);
  if (rc) return rc;
  if (tokens == 0) return H3ATTN_OK;
  if ((rc = check_plan(seg_ids, tokens, heads, workspace, workspace_bytes))) return rc;
  DeviceInfo di;
  if ((rc = device_info(&di))) return rc;
  return launch_status(launch_plan(seg_ids, tokens, workspace, heads, (hipStream_t)stream));
}

int h3attn_prep_qkv(const void* q, const void* k, const void* v, const void* wq, const void* wk, int64_t tokens,
                    int32_t heads, int32_t head_dim, float eps, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(tokens, heads, head_dim);
  if (rc) return rc;
  if (tokens == 0) return H3ATTN_OK;
  if ((rc = check_prep(q, k, v, wq, wk, tokens, heads, eps, workspace, workspace_bytes))) return rc;
  DeviceInfo di;
  if ((rc = device_info(&di))) return rc;
  return launch_status(
      launch_prep_qkv(q, k, v, wq, wk, tokens, heads, eps, workspace, nullptr, nullptr, nullptr, (hipStream_t)stream));
}

int h3attn_attend(const void* q, const void* wq, int64_t tokens, int32_t heads, int32_t head_dim, float eps,
                  float scale, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(tokens, heads, head_dim);
  if (rc) return rc;
  if (tokens == 0) return (!(scale > 0.0f) || !std::isfinite(scale)) ? H3ATTN_ERR_SHAPE : H3ATTN_OK;
  if ((rc = check_attend(q, wq, tokens, heads, eps, scale, out, lse, workspace, workspace_bytes))) return rc;
  DeviceInfo di;
  if ((rc = device_info(&di))) return rc;
  return launch_status(
      launch_attend(q, wq != nullptr, tokens, heads, scale, out, lse, nullptr, nullptr, workspace, di.cus,
                    (hipStream_t)stream));
}

// The forward; pos_ids NULL walks keys in packed order, else in position order; o32 (optional)
// receives the output before its bf16 rounding.
// MM-RoPE tables: both or neither, only with the norm weights (the fused q_norm -> rope chain), float32
// [T][48], 16-byte aligned; no output and not the workspace may overlap them.
static int check_rope(const float* rc, const float* rs, const void* wq, int64_t tokens, void* const* outs,
                      const size_t* out_n, int nout) {
  if ((rc == nullptr) != (rs == nullptr)) return H3ATTN_ERR_NULL;
  if (!rc) return H3ATTN_OK;
  if (!wq) return H3ATTN_ERR_NULL;
  if (!aligned(rc, 16) || !aligned(rs, 16)) return H3ATTN_ERR_ALIGN;
  const size_t nt = (size_t)tokens * 48 * 4;
  for (int i = 0; i < nout; i++)
    if (overlap(outs[i], out_n[i], rc, nt) || overlap(outs[i], out_n[i], rs, nt)) return H3ATTN_ERR_ALIAS;
  return H3ATTN_OK;
}

static int fwd_impl(const void* q, const void* k, const void* v, const int32_t* seg_ids, const int32_t* pos_ids,
                    bool ordered, const void* wq, const void* wk, int64_t tokens, int32_t heads, int32_t head_dim,
                    float eps, float scale, void* out, float* lse, float* o32, void* workspace,
                    size_t workspace_bytes, void* stream, int32_t* status_out = nullptr,
                    const float* rope_cos = nullptr, const float* rope_sin = nullptr) {
  int rc = check_shape(tokens, heads, head_dim);
  if (rc) return rc;
  if ((wq == nullptr) != (wk == nullptr)) return H3ATTN_ERR_NULL;
  if ((rope_cos == nullptr) != (rope_sin == nullptr) || (rope_cos && !wq)) return H3ATTN_ERR_NULL;
  if (wq && (!(eps > 0.0f) || !std::isfinite(eps))) return H3ATTN_ERR_SHAPE;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return H3ATTN_ERR_SHAPE;
  if (tokens == 0) return H3ATTN_OK;
  if (!q || !k || !v || !seg_ids || !out || !workspace || (ordered && !pos_ids)) return H3ATTN_ERR_NULL;
  if ((rc = check_plan(seg_ids, tokens, heads, workspace, workspace_bytes))) return rc;
  if ((rc = check_prep(q, k, v, wq, wk, tokens, heads, eps, workspace, workspace_bytes))) return rc;
  if ((rc = check_attend(q, wq, tokens, heads, eps, scale, out, lse, workspace, workspace_bytes))) return rc;
  const size_t n = tensor_bytes(tokens, heads);
  const size_t nl = (size_t)tokens * heads * 4;
  const size_t ns = (size_t)tokens * 4;
  if (overlap(out, n, k, n) || overlap(out, n, v, n) || overlap(out, n, seg_ids, ns) ||
      overlap(out, n, wk, HD * 2) || overlap(lse, nl, k, n) || overlap(lse, nl, v, n) ||
      overlap(lse, nl, seg_ids, ns) || overlap(lse, nl, wk, HD * 2))
    return H3ATTN_ERR_ALIAS;
  if (o32) {
    const size_t n32 = 2 * n;
    if (!aligned(o32, 16)) return H3ATTN_ERR_ALIGN;
    const void* ins[] = {q, k, v, seg_ids, wq, wk, workspace, pos_ids, out, lse};
    const size_t in_n[] = {n, n, n, ns, (size_t)HD * 2, (size_t)HD * 2, workspace_bytes, pos_ids ? ns : 0, n, nl};
    for (int i = 0; i < 10; i++)
      if (overlap(o32, n32, ins[i], in_n[i])) return H3ATTN_ERR_ALIAS;
  }
  const OrderLayout ol = order_layout(ws_layout(tokens, heads).total, tokens);
  if (ordered) {
    if (!aligned(pos_ids, 4)) return H3ATTN_ERR_ALIGN;
    if (overlap(out, n, pos_ids, ns) || overlap(lse, nl, pos_ids, ns) ||
        overlap(pos_ids, ns, workspace, workspace_bytes))
      return H3ATTN_ERR_ALIAS;
    if (workspace_bytes < ol.total) return H3ATTN_ERR_WORKSPACE;
  }
  {
    void* outs[] = {out, lse, o32, workspace};
    const size_t out_n[] = {n, nl, o32 ? 2 * n : 0, workspace_bytes};
    if ((rc = check_rope(rope_cos, rope_sin, wq, tokens, outs, out_n, 4))) return rc;
  }
  DeviceInfo di;
  if ((rc = device_info(&di))) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)workspace;
  int32_t* slot = ordered ? (int32_t*)(base + ol.slot) : nullptr;
  if ((rc = launch_status(launch_plan(seg_ids, tokens, workspace, heads, st)))) return rc;
  const WsLayout wl = ws_layout(tokens, heads);
  if (ordered && (rc = launch_status(launch_order(pos_ids, tokens, workspace, (const int32_t*)(base + wl.segtab),
                                                  (const int32_t*)(base + wl.tok2seg), (int32_t*)(base + wl.segflag),
                                                  slot, (int32_t*)(base + ol.inv), st))))
    return rc;
  if ((rc = launch_status(
           launch_prep_qkv(q, k, v, wq, wk, tokens, heads, eps, workspace, slot, rope_cos, rope_sin, st))))
    return rc;
  return launch_status(
      launch_attend(q, wq != nullptr, tokens, heads, scale, out, lse, o32, status_out, workspace, di.cus, st));
}

int h3attn_fwd(const void* q, const void* k, const void* v, const int32_t* seg_ids, const void* wq, const void* wk,
               int64_t tokens, int32_t heads, int32_t head_dim, float eps, float scale, void* out, float* lse,
               void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, seg_ids, nullptr, false, wq, wk, tokens, heads, head_dim, eps, scale, out, lse, nullptr,
                  workspace, workspace_bytes, stream);
}

int h3attn_fwd_pos(const void* q, const void* k, const void* v, const int32_t* seg_ids, const int32_t* pos_ids,
                   const void* wq, const void* wk, int64_t tokens, int32_t heads, int32_t head_dim, float eps,
                   float scale, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, seg_ids, pos_ids, true, wq, wk, tokens, heads, head_dim, eps, scale, out, lse, nullptr,
                  workspace, workspace_bytes, stream);
}

int h3attn_fwd_ex(const void* q, const void* k, const void* v, const int32_t* seg_ids, const int32_t* pos_ids,
                  const void* wq, const void* wk, const float* rope_cos, const float* rope_sin, int64_t tokens,
                  int32_t heads, int32_t head_dim, float eps, float scale, void* out, float* lse, float* o32,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, seg_ids, pos_ids, pos_ids != nullptr, wq, wk, tokens, heads, head_dim, eps, scale, out, lse,
                  o32, workspace, workspace_bytes, stream, nullptr, rope_cos, rope_sin);
}

// h3attn_fwd on the library's static scratch instead of a caller workspace: no allocation at all.
int h3attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* seg_ids, const void* wq,
                       const void* wk, int64_t tokens, int32_t heads, int32_t head_dim, float eps, float scale,
                       void* out, float* lse, int32_t* status, void* stream) {
  int rc = check_shape(tokens, heads, head_dim);
  if (rc) return rc;
  if (h3attn_workspace_bytes(tokens, heads) > kScratchBytes) return H3ATTN_ERR_SCRATCH;
  if (tokens == 0)  // no device work: only the scalar checks of h3attn_fwd
    return fwd_impl(q, k, v, seg_ids, nullptr, false, wq, wk, tokens, heads, head_dim, eps, scale, out, lse, nullptr,
                    nullptr, 0, stream);
  if (!q || !k || !v || !seg_ids || !out) return H3ATTN_ERR_NULL;
  if (status) {
    if (!aligned(status, 4)) return H3ATTN_ERR_ALIGN;
    const size_t n = tensor_bytes(tokens, heads);
    const void* bufs[] = {q, k, v, seg_ids, wq, wk, out, lse};
    const size_t sz[] = {n, n, n, (size_t)tokens * 4, (size_t)HD * 2, (size_t)HD * 2, n, (size_t)tokens * heads * 4};
    for (int i = 0; i < 8; i++)
      if (overlap(status, 4, bufs[i], sz[i])) return H3ATTN_ERR_ALIAS;
  }
  DeviceInfo di;
  if ((rc = device_info(&di))) return rc;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  if (status && overlap(status, 4, ws, kScratchBytes)) return H3ATTN_ERR_ALIAS;
  return fwd_impl(q, k, v, seg_ids, nullptr, false, wq, wk, tokens, heads, head_dim, eps, scale, out, lse, nullptr, ws,
                  kScratchBytes, stream, status);
}

// Large enough for both h3attn_bwd and h3attn_bwd_pos.
size_t h3attn_bwd_workspace_bytes(int64_t tokens, int32_t heads) {
  if (check_shape(tokens, heads, HD) != H3ATTN_OK) return 0;
  if (tokens + (tokens + BT - 1) / BT > (int64_t)INT32_MAX / heads) return 0;
  return order_layout(bwd_layout(tokens, heads).total, tokens).total;
}

// The backward; ordered: operands staged and every sum taken in position order; o32 (optional):
// the forward's fp32 output, from which D = dO . O is computed instead of recomputed from P and dP.
static int bwd_impl(const void* dout, const void* q, const void* k, const void* v, const float* lse, const float* o32,
                    const int32_t* seg_ids, const int32_t* pos_ids, bool ordered, const void* wq, const void* wk,
                    int64_t tokens, int32_t heads, int32_t head_dim, float eps, float scale, void* dq, void* dk,
                    void* dv, float* dwq, float* dwk, void* workspace, size_t workspace_bytes, void* stream,
                    const float* rope_cos = nullptr, const float* rope_sin = nullptr) {
  int rc = check_shape(tokens, heads, head_dim);
  if (rc) return rc;
  if (tokens + (tokens + BT - 1) / BT > (int64_t)INT32_MAX / heads) return H3ATTN_ERR_SHAPE;
  if ((wq == nullptr) != (wk == nullptr)) return H3ATTN_ERR_NULL;
  if ((rope_cos == nullptr) != (rope_sin == nullptr) || (rope_cos && !wq)) return H3ATTN_ERR_NULL;
  if (wq && (!(eps > 0.0f) || !std::isfinite(eps))) return H3ATTN_ERR_SHAPE;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return H3ATTN_ERR_SHAPE;
  if (tokens == 0) return H3ATTN_OK;
  if (!dout || !q || !k || !v || !lse || !seg_ids || !dq || !dk || !dv || !workspace || (ordered && !pos_ids))
    return H3ATTN_ERR_NULL;
  if (wq && (!dwq || !dwk)) return H3ATTN_ERR_NULL;
  if (!aligned(dout, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(lse, 4) ||
      !aligned(seg_ids, 4) || (wq && (!aligned(wq, 16) || !aligned(wk, 16) || !aligned(dwq, 4) || !aligned(dwk, 4))) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 256) ||
      (ordered && !aligned(pos_ids, 4)) || (o32 && !aligned(o32, 16)))
    return H3ATTN_ERR_ALIGN;
  const OrderLayout ol = order_layout(bwd_layout(tokens, heads).total, tokens);
  if (workspace_bytes < (ordered ? ol.total : bwd_layout(tokens, heads).total)) return H3ATTN_ERR_WORKSPACE;
  const size_t n = tensor_bytes(tokens, heads);
  const size_t nl = (size_t)tokens * heads * 4;
  const size_t ns = (size_t)tokens * 4;
  // every output against every input, the workspace and the other outputs
  const void* ins[] = {dout, q, k, v, lse, seg_ids, wq, wk, workspace, pos_ids, o32};
  const size_t in_n[] = {n, n, n, n, nl, ns, (size_t)HD * 2, (size_t)HD * 2, workspace_bytes, ordered ? ns : 0,
                         o32 ? 2 * n : 0};
  void* outs[] = {dq, dk, dv, dwq, dwk};
  const size_t out_n[] = {n, n, n, wq ? (size_t)HD * 4 : 0, wq ? (size_t)HD * 4 : 0};
  if (ordered && overlap(pos_ids, ns, workspace, workspace_bytes)) return H3ATTN_ERR_ALIAS;
  if (o32 && overlap(o32, 2 * n, workspace, workspace_bytes)) return H3ATTN_ERR_ALIAS;
  for (int o = 0; o < 5; o++) {
    for (int i = 0; i < 11; i++)
      if (overlap(outs[o], out_n[o], ins[i], in_n[i])) return H3ATTN_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 5; o2++)
      if (overlap(outs[o], out_n[o], outs[o2], out_n[o2])) return H3ATTN_ERR_ALIAS;
  }
  {
    void* outs6[] = {dq, dk, dv, dwq, dwk, workspace};
    const size_t out_n6[] = {n, n, n, out_n[3], out_n[4], workspace_bytes};
    if ((rc = check_rope(rope_cos, rope_sin, wq, tokens, outs6, out_n6, 6))) return rc;
  }
  DeviceInfo di;
  if ((rc = device_info(&di))) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)workspace;
  int32_t* slot = ordered ? (int32_t*)(base + ol.slot) : nullptr;
  int32_t* inv = ordered ? (int32_t*)(base + ol.inv) : nullptr;
  if ((rc = launch_status(launch_plan_bwd(seg_ids, tokens, workspace, heads, st)))) return rc;
  const BwdLayout bl = bwd_layout(tokens, heads);
  if (ordered && (rc = launch_status(launch_order(pos_ids, tokens, workspace, (const int32_t*)(base + bl.segtab),
                                                  (const int32_t*)(base + bl.tok2seg), (int32_t*)(base + bl.segflag),
                                                  slot, inv, st))))
    return rc;
  if ((rc = launch_status(launch_bwd_prep(q, k, v, dout, lse, o32, wq, wk, tokens, heads, eps, workspace, slot,
                                          rope_cos, rope_sin, st))))
    return rc;
  return launch_status(launch_bwd(q, k, wq, wk, tokens, heads, eps, scale, dq, dk, dv, dwq, dwk, workspace, inv,
                                  o32 != nullptr, rope_cos, rope_sin, di.cus, st));
}

int h3attn_bwd(const void* dout, const void* q, const void* k, const void* v, const float* lse,
               const int32_t* seg_ids, const void* wq, const void* wk, int64_t tokens, int32_t heads,
               int32_t head_dim, float eps, float scale, void* dq, void* dk, void* dv, float* dwq, float* dwk,
               void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(dout, q, k, v, lse, nullptr, seg_ids, nullptr, false, wq, wk, tokens, heads, head_dim, eps, scale, dq,
                  dk, dv, dwq, dwk, workspace, workspace_bytes, stream);
}

int h3attn_bwd_pos(const void* dout, const void* q, const void* k, const void* v, const float* lse,
                   const int32_t* seg_ids, const int32_t* pos_ids, const void* wq, const void* wk, int64_t tokens,
                   int32_t heads, int32_t head_dim, float eps, float scale, void* dq, void* dk, void* dv, float* dwq,
                   float* dwk, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(dout, q, k, v, lse, nullptr, seg_ids, pos_ids, true, wq, wk, tokens, heads, head_dim, eps, scale, dq,
                  dk, dv, dwq, dwk, workspace, workspace_bytes, stream);
}

int h3attn_bwd_ex(const void* dout, const void* q, const void* k, const void* v, const float* lse, const float* o32,
                  const int32_t* seg_ids, const int32_t* pos_ids, const void* wq, const void* wk,
                  const float* rope_cos, const float* rope_sin, int64_t tokens, int32_t heads, int32_t head_dim,
                  float eps, float scale, void* dq, void* dk, void* dv, float* dwq, float* dwk, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return bwd_impl(dout, q, k, v, lse, o32, seg_ids, pos_ids, pos_ids != nullptr, wq, wk, tokens, heads, head_dim, eps,
                  scale, dq, dk, dv, dwq, dwk, workspace, workspace_bytes, stream, rope_cos, rope_sin);
}

int h3attn_status_read(const void* workspace, int32_t* device_status, void* stream) {
  if (!workspace || !device_status) return H3ATTN_ERR_NULL;
  if (!aligned(workspace, 256)) return H3ATTN_ERR_ALIGN;
  int32_t bits = 0;
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(&bits, workspace, sizeof(bits), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    (void)hipGetLastError();
    return H3ATTN_ERR_LAUNCH;
  }
  *device_status = status_code(bits);
  return H3ATTN_OK;
}

}  // extern "C"
