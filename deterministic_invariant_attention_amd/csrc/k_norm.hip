// The q_norm / k_norm node (RMSNorm over each 128-wide head, one 128-element weight shared by all
// heads: "ws1_one_h3_block" page, Bindings table and Results) as a standalone kernel, the operand
// staging kernel of the attention (Q and K normed with the same arithmetic, V converted to fp16)
// and the operand staging kernel of the backward.
//
// Mapping: 16 lanes per (token, head) row, lane c holds channels 8c..8c+7 (one 16-byte chunk), so
// each wave moves 4 rows with fully coalesced 16-byte accesses.  The sum of squares follows the
// fixed tree of h3_norm.h, so every kernel here gives the bits of the standalone norm.
#include "h3_common.h"
#include "h3_norm.h"
#include "h3_bwd.h"
#include "h3_launch.h"

namespace h3 {

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(uint16_t* p, const u32x4& v) { *(u32x4*)p = v; }

// Norm one row chunk held by this lane (16-lane mapping) with the lane's chunk of the weights;
// every lane of the group must call it.
__device__ __forceinline__ u32x4 norm_16lane(const u32x4& xv, const u32x4& wv, float eps) {
  float x[8], wf[8];
  unpack8_bf16(xv, x);
  const double total = row_total_16lanes(chunk_sumsq(x));
  const double r = norm_rscale(total, eps);
  unpack8_bf16(wv, wf);
  return norm_chunk(x, wf, r);
}

__global__ __launch_bounds__(256) void k_qknorm(const uint16_t* x, const uint16_t* __restrict__ w, uint16_t* y,
                                               int64_t rows, float eps) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g >> 4;
  const int c = threadIdx.x & 15;
  const bool valid = row < rows;  // uniform over each 16-lane group
  u32x4 xv = {0, 0, 0, 0};
  if (valid) xv = ld16(x + row * HD + c * 8);
  const u32x4 o = norm_16lane(xv, ld16(w + c * 8), eps);
  if (valid) st16(y + row * HD + c * 8, o);
}

// Operand staging of the attention.  With norm weights, Q is normed into qhat (head-major, packed
// token order: the queries are walked in packed order); K is normed (or copied) and V converted to
// fp16, both at the token's staged row (slot[t] in position order, else t), where the key walk
// reads them.
struct PrepParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* wq;  // NULL: Q is not staged (the attention reads the caller's q)
  const uint16_t* wk;
  uint16_t* qhat;
  uint16_t* khat;
  uint16_t* v16;
  const int32_t* slot;  // staged row of each token (position order), or NULL for packed order
  const int32_t* tok2seg;
  int32_t* segflag;  // a segment with a value beyond fp16 is flagged (its outputs become NaN)
  const float* rope_cos;  // optional MM-RoPE tables, float32 [T][48] (only with norm weights)
  const float* rope_sin;
  WsHeader* hdr;
  int64_t T;
  int32_t H;
  float eps;
};

// The rope tables' entries for the lane's chunk (chunks 0..11 of token t); zeros elsewhere.
__device__ __forceinline__ void rope_entries(const float* rc, const float* rs, int64_t t, int c, bool valid, f32x4& cs,
                                             f32x4& sn) {
  cs = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  sn = cs;
  if (rc && valid && c < ROPE_CHUNKS) {
    cs = *(const f32x4*)(rc + t * ROPE_PAIRS + 4 * c);
    sn = *(const f32x4*)(rs + t * ROPE_PAIRS + 4 * c);
  }
}

// Rows are visited token-major (r = t*H + h) so the reads are contiguous; each row is written to
// its head-major staged row.  Every load of the row precedes every store (the outputs live in
// another buffer, but the compiler cannot know that), so each lane's three reads are in flight
// together.
__global__ __launch_bounds__(256) void k_prep_qkv(PrepParams p) {
  const int c = threadIdx.x & 15;
  const int64_t T = p.T;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const bool valid = row < T * p.H;
  // T * H < 2^31 (the shape check of every entry point), so 32-bit division places the row
  const int64_t t = valid ? (int64_t)((uint32_t)row / (uint32_t)p.H) : 0;
  const int64_t h = valid ? row - t * p.H : 0;
  const int64_t ts = (valid && p.slot) ? (int64_t)p.slot[t] : t;  // slot[t] is in [0, T) by construction
  const u32x4 zero4 = {0, 0, 0, 0};
  const u32x4 wqv = p.wq ? ld16(p.wq + c * 8) : zero4, wkv = p.wk ? ld16(p.wk + c * 8) : zero4;
  {
    const int64_t src = row * HD + c * 8;
    u32x4 qv = {0, 0, 0, 0}, kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (valid) {
      // read once: nontemporal loads keep them from displacing cached lines (92 against 103 us in
      // one same-box comparison at 8349 tokens x 40 heads)
      if (p.wq) qv = __builtin_nontemporal_load((const u32x4*)(p.q + src));
      kv = __builtin_nontemporal_load((const u32x4*)(p.k + src));
      vv = __builtin_nontemporal_load((const u32x4*)(p.v + src));
    }
    f32x4 rcs, rsn;
    rope_entries(p.rope_cos, p.rope_sin, t, c, valid, rcs, rsn);
    const bool rot = p.rope_cos && c < ROPE_CHUNKS;  // this lane's chunk is rotated
    if (p.wq) {
      u32x4 qo = norm_16lane(qv, wqv, p.eps);
      if (rot) qo = rope_chunk(qo, rcs, rsn);
      if (valid) st16(p.qhat + (h * T + t) * HD + c * 8, qo);
    }
    u32x4 ko = p.wk ? norm_16lane(kv, wkv, p.eps) : kv;
    if (rot) ko = rope_chunk(ko, rcs, rsn);

    // V: bf16 -> fp16, exact for normal fp16 magnitudes; a finite |v| > 65504 would overflow.
    u32x4 vo;
    bool over = false;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float a = bf16_lo(vv[i]), b = bf16_hi(vv[i]);
      over |= (__builtin_fabsf(a) > 65504.0f && __builtin_fabsf(a) != __builtin_inff());
      over |= (__builtin_fabsf(b) > 65504.0f && __builtin_fabsf(b) != __builtin_inff());
      vo[i] = pack_f16(a, b);
    }
    const int64_t dst = (h * T + ts) * HD + c * 8;
    if (valid) {
      st16(p.khat + dst, ko);
      st16(p.v16 + dst, vo);
    }
    if (valid && over) flag_segment(p.segflag, p.tok2seg[t], p.hdr->nseg);
    const uint64_t any_over = __ballot(valid && over);
    if (any_over && (threadIdx.x & 63) == __builtin_ctzll(any_over)) atomicOr(&p.hdr->status, STATUS_RANGE_BIT);
  }
}

// Operand staging of the backward: per (token, head) row, the normed q and k (the forward's exact
// bits), v and dO, all in fp16 and head-major; the forward's LSE in log2 units.  A finite value
// beyond the fp16 range in a converted operand sets STATUS_RANGE_BIT.
struct BwdPrepParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* o32;  // optional: the forward's output before its bf16 rounding
  const uint16_t* wq;
  const uint16_t* wk;
  uint16_t* qhat16;
  uint16_t* khat16;
  uint16_t* v16;
  uint16_t* do16;
  float* lse2;
  float* delta;         // -D, D = dO . O per row (with o32)
  const int32_t* slot;  // staged row of each token (position order), or NULL for packed order
  const int32_t* tok2seg;  // segment of each token
  int32_t* segflag;        // a segment with a q^, k^ or v value beyond fp16 is flagged (NaN outputs)
  const float* rope_cos;   // optional MM-RoPE tables, float32 [T][48]
  const float* rope_sin;
  const uint32_t* dmax;    // per (segment, head): largest |dO| (bf16 magnitude bits)
  WsHeader* hdr;
  int64_t T;
  int32_t H;
  float eps;
};

// The largest |dO| of every (segment, head): one workgroup per 16 tokens x 16 heads (workgroup
// b: tokens 16 (b / n) .., heads 16 (b % n) .., n = ceil(H / 16)), so each pass of 16 rows reads one token's 16 heads, 4 KB
// in a row; 16 lanes per (token, head) row.  Each row's maximum (bf16 magnitude bits, exact
// integers) goes to LDS; then 16 lanes per head, one per token, take a segmented running maximum
// over the block's tokens (segments are runs of tokens, so a lane o places back belongs to the
// same run exactly when it has the same segment), and the last lane of each run folds the run's
// maximum into the segment's slot with an integer atomicMax, so the result is the same whatever the
// order of the workgroups.
constexpr int DMAX_TOK = 16;  // tokens per workgroup
__device__ __forceinline__ uint32_t max_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }
constexpr int DMAX_HEADS = 16;  // heads per workgroup

__global__ __launch_bounds__(256) void k_bwd_dmax(const uint16_t* __restrict__ dout, const int32_t* __restrict__ tok2seg,
                                                  uint32_t* __restrict__ dmax, const WsHeader* hdr, int64_t T,
                                                  int32_t H) {
  __shared__ uint32_t s_max[DMAX_TOK][DMAX_HEADS];
  __shared__ int32_t s_seg[DMAX_TOK];
  const int c = threadIdx.x & 15, rr = threadIdx.x >> 4;  // lane in the row, row in the pass (= head)
  const int nhc = (H + DMAX_HEADS - 1) / DMAX_HEADS;
  const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)nhc) * DMAX_TOK;
  const int h0 = (int)(blockIdx.x % (unsigned)nhc) * DMAX_HEADS;
  const int h = h0 + rr;
  // every load of the block's rows is issued before the first is reduced: rows past the end read
  // the last row (no branch around the loads) and count as zero
  u32x4 w[DMAX_TOK];
  const int hc = h < H ? h : H - 1;
#pragma unroll
  for (int i = 0; i < DMAX_TOK; i++) {
    const int64_t t = t0 + i < T ? t0 + i : T - 1;
    w[i] = *(const u32x4*)(dout + (t * H + hc) * HD + c * 8);
  }
#pragma unroll
  for (int i = 0; i < DMAX_TOK; i++)
    if (t0 + i >= T || h >= H) w[i] = u32x4{0u, 0u, 0u, 0u};
  if (threadIdx.x < DMAX_TOK) s_seg[threadIdx.x] = t0 + threadIdx.x < T ? tok2seg[t0 + threadIdx.x] : -1;
#pragma unroll
  for (int i = 0; i < DMAX_TOK; i++) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t a = w[i][j] & 0x7FFFu, b = (w[i][j] >> 16) & 0x7FFFu;
      m = a > m ? a : m;
      m = b > m ? b : m;
    }
    // the row's 16 lanes: rotations by 8, 4, 2, 1 within the row (DPP, no LDS traffic); a
    // maximum does not depend on the order
    m = max_u32(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xF, 0xF, false));  // row_ror:8
    m = max_u32(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x124, 0xF, 0xF, false));  // row_ror:4
    m = max_u32(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x122, 0xF, 0xF, false));  // row_ror:2
    m = max_u32(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x121, 0xF, 0xF, false));  // row_ror:1
    if (c == 0) s_max[i][rr] = m;
  }
  __syncthreads();
  // fold: lane (head rr, token c)
  {
    const int i = c;
    const int nseg = hdr->nseg;  // 0 after a segment-id error: nothing is folded
    const int sg = s_seg[i];
    uint32_t m = s_max[i][rr];
#pragma unroll
    for (int o = 1; o < DMAX_TOK; o <<= 1) {
      const uint32_t y = (uint32_t)__shfl_up((int)m, o, 16);
      const int ys = __shfl_up(sg, o, 16);
      if (i >= o && ys == sg) m = y > m ? y : m;
    }
    const int next = __shfl_down(sg, 1, 16);
    const bool last = i + 1 == DMAX_TOK || next != sg;
    if (last && h < H && sg >= 0 && sg < nseg) atomicMax(&dmax[(int64_t)sg * H + h], m);
  }
}

// bf16 chunk -> fp16 chunk: exact for every bf16 value from 2^-17 up to 65504 in magnitude (and
// zero); below 2^-17 fp16 subnormals round it, by at most 2^-25.  over |= a finite value beyond
// 65504.
__device__ __forceinline__ u32x4 bf16_chunk_to_f16(const u32x4& x, bool& over) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float a = bf16_lo(x[i]), b = bf16_hi(x[i]);
    over |= (__builtin_fabsf(a) > 65504.0f && __builtin_fabsf(a) != __builtin_inff());
    over |= (__builtin_fabsf(b) > 65504.0f && __builtin_fabsf(b) != __builtin_inff());
    o[i] = pack_f16(a, b);
  }
  return o;
}

// The backward's operands, head-major, in fp16 (every product of the backward runs on fp16 MFMA
// with FP32 accumulation): the normed q and k (rounded to bf16 exactly as in the forward, then
// converted), v and dO; and the LSE in log2 units.
// Same mapping as k_prep_qkv.
__global__ __launch_bounds__(256) void k_bwd_prep(BwdPrepParams p) {
  const int c = threadIdx.x & 15;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const bool valid = row < p.T * p.H;
  const int64_t t = valid ? (int64_t)((uint32_t)row / (uint32_t)p.H) : 0;
  const int64_t h = valid ? row - t * p.H : 0;
  const int64_t ts = (valid && p.slot) ? (int64_t)p.slot[t] : t;
  const u32x4 zero4 = {0, 0, 0, 0};
  const u32x4 wqv = p.wq ? ld16(p.wq + c * 8) : zero4, wkv = p.wk ? ld16(p.wk + c * 8) : zero4;
  {
    const int64_t dst = (h * p.T + ts) * HD + c * 8;

    // every load before any store (see k_prep_qkv)
    u32x4 qv = {0, 0, 0, 0}, kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0}, gv = {0, 0, 0, 0};
    f32x4 o0 = {0.0f, 0.0f, 0.0f, 0.0f}, o1 = o0;
    float lse = 0.0f;
    if (valid) {
      qv = ld16(p.q + row * HD + c * 8);
      kv = ld16(p.k + row * HD + c * 8);
      vv = ld16(p.v + row * HD + c * 8);
      gv = ld16(p.dout + row * HD + c * 8);
      if (p.o32) {
        o0 = *(const f32x4*)(p.o32 + row * HD + c * 8);
        o1 = *(const f32x4*)(p.o32 + row * HD + c * 8 + 4);
      }
      if (c == 0) lse = p.lse[row];
    }
    u32x4 qo = p.wq ? norm_16lane(qv, wqv, p.eps) : qv;
    u32x4 ko = p.wk ? norm_16lane(kv, wkv, p.eps) : kv;
    if (p.rope_cos && c < ROPE_CHUNKS) {  // the rotated operands, bitwise those of the forward
      f32x4 rcs, rsn;
      rope_entries(p.rope_cos, p.rope_sin, t, c, valid, rcs, rsn);
      qo = rope_chunk(qo, rcs, rsn);
      ko = rope_chunk(ko, rcs, rsn);
    }
    bool over = false;
    const u32x4 q16 = bf16_chunk_to_f16(qo, over);
    const u32x4 k16 = bf16_chunk_to_f16(ko, over);
    const u32x4 v16 = bf16_chunk_to_f16(vv, over);
    // dO times 2^s of its (segment, head) (exact: a power of two; the largest |dO| lands in [4, 8),
    // so the fp16 conversion neither overflows nor loses the small values of a small gradient)
    int sx = 0;
    const int nseg = p.hdr->nseg;
    const int sg = valid ? p.tok2seg[t] : -1;
    if (sg >= 0 && sg < nseg) sx = dout_scale_exp(p.dmax[(int64_t)sg * p.H + h]);
    if (valid && over) flag_segment(p.segflag, sg, nseg);
    u32x4 g16;
#pragma unroll
    for (int i = 0; i < 4; i++)
      g16[i] = pack_f16(__builtin_ldexpf(bf16_lo(gv[i]), sx), __builtin_ldexpf(bf16_hi(gv[i]), sx));
    if (valid) {
      st16(p.qhat16 + dst, q16);
      st16(p.khat16 + dst, k16);
      st16(p.v16 + dst, v16);
      st16(p.do16 + dst, g16);
      if (c == 0) p.lse2[h * p.T + ts] = lse * 1.44269504088896340736f;
    }
    if (p.o32) {
      // D_i = sum_d dO_id O_id: products and sums in FP64 (each lane its 8 channels in order, then a
      // fixed butterfly over the 16 lanes of the row), rounded once to fp32
      float g[8];
      unpack8_bf16(gv, g);
      double d = 0.0;
#pragma unroll
      for (int i = 0; i < 4; i++) d = __builtin_fma((double)g[i], (double)o0[i], d);
#pragma unroll
      for (int i = 0; i < 4; i++) d = __builtin_fma((double)g[4 + i], (double)o1[i], d);
      d = d + __shfl_xor(d, 1, 64);
      d = d + __shfl_xor(d, 2, 64);
      d = d + __shfl_xor(d, 4, 64);
      d = d + __shfl_xor(d, 8, 64);
      // D of the scaled dO: the same power of two, applied in FP64 before the one fp32 rounding
      if (valid && c == 0) p.delta[h * p.T + ts] = -(float)__builtin_ldexp(d, sx);
    }
    const uint64_t any_over = __ballot(valid && over);
    if (any_over && (threadIdx.x & 63) == __builtin_ctzll(any_over)) atomicOr(&p.hdr->status, STATUS_RANGE_BIT);
  }
}

static inline unsigned grid_for_rows(int64_t rows) { return (unsigned)((rows * 16 + 255) / 256); }


hipError_t launch_bwd_prep(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           const float* o32, const void* wq, const void* wk, int64_t T, int32_t H, float eps, void* ws,
                           const int32_t* slot, const float* rope_cos, const float* rope_sin, hipStream_t stream) {
  const int64_t rows = T * H;
  if (rows == 0) return hipSuccess;
  const BwdLayout L = bwd_layout(T, H);
  char* base = (char*)ws;
  BwdPrepParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.o32 = o32;
  p.wq = (const uint16_t*)wq;
  p.wk = (const uint16_t*)wk;
  p.qhat16 = (uint16_t*)(base + L.qhat16);
  p.khat16 = (uint16_t*)(base + L.khat16);
  p.v16 = (uint16_t*)(base + L.v16);
  p.do16 = (uint16_t*)(base + L.do16);
  p.lse2 = (float*)(base + L.lse2);
  p.delta = (float*)(base + L.delta);
  p.slot = slot;
  p.tok2seg = (const int32_t*)(base + L.tok2seg);
  p.segflag = (int32_t*)(base + L.segflag);
  p.rope_cos = rope_cos;
  p.rope_sin = rope_sin;
  p.dmax = (const uint32_t*)(base + L.dmax);
  p.hdr = (WsHeader*)base;
  p.T = T;
  p.H = H;
  p.eps = eps;
  hipLaunchKernelGGL(k_bwd_dmax, dim3((unsigned)((T + DMAX_TOK - 1) / DMAX_TOK * ((H + DMAX_HEADS - 1) / DMAX_HEADS))),
                     dim3(256), 0, stream,
                     (const uint16_t*)dout, p.tok2seg, (uint32_t*)(base + L.dmax), (const WsHeader*)base, T, H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bwd_prep, dim3(grid_for_rows(rows)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_qknorm(const void* x, const void* w, void* y, int64_t T, int32_t H, float eps, hipStream_t stream) {
  const int64_t rows = T * H;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_qknorm, dim3(grid_for_rows(rows)), dim3(256), 0, stream, (const uint16_t*)x,
                     (const uint16_t*)w, (uint16_t*)y, rows, eps);
  return hipGetLastError();
}

hipError_t launch_prep_qkv(const void* q, const void* k, const void* v, const void* wq, const void* wk, int64_t T,
                           int32_t H, float eps, void* ws, const int32_t* slot, const float* rope_cos,
                           const float* rope_sin, hipStream_t stream) {
  const int64_t rows = T * H;
  if (rows == 0) return hipSuccess;
  const WsLayout L = ws_layout(T, H);
  char* base = (char*)ws;
  PrepParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.wq = (const uint16_t*)wq;
  p.wk = (const uint16_t*)wk;
  p.qhat = (uint16_t*)(base + L.qhat);
  p.khat = (uint16_t*)(base + L.khat);
  p.v16 = (uint16_t*)(base + L.v16);
  p.slot = slot;
  p.tok2seg = (const int32_t*)(base + L.tok2seg);
  p.segflag = (int32_t*)(base + L.segflag);
  p.rope_cos = rope_cos;
  p.rope_sin = rope_sin;
  p.hdr = (WsHeader*)base;
  p.T = T;
  p.H = H;
  p.eps = eps;
  hipLaunchKernelGGL(k_prep_qkv, dim3(grid_for_rows(rows)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace h3
