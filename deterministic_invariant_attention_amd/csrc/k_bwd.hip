// Backward of the H3 attention node: gradients with respect to q, k, v and the two RMSNorm weights
// for an upstream gradient dO ("33B forward/backward" page: the node runs inside the training step's
// backward; "ws1_one_h3_block" page, Bindings: q_norm / k_norm, then attention with causal=False).
// The bf16 rounding of the normed operands is the identity for gradients (straight-through).
//
// Per segment and head, with P recomputed from the forward's log-sum-exp:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P o (dP - D),
//   dq^ = scale dS K^,  dk^ = scale dS^T Q^,  then the RMSNorm backward of each row and the weight
//   gradients dw = sum over rows of dy o x r.
//
// Two attention kernels, neither with atomics, both walking their inner dimension in ascending,
// segment-anchored 64-row tiles, so every gradient row is a fixed function of its own segment:
//   k_bwd_dq    work item = (segment, 128-query tile, head).  Pass 1 over the key tiles computes
//               D_i exactly (in fp32, a fixed tree per tile); pass 2 recomputes S and dP, forms dS
//               and accumulates dQ^T += K^16^T dS^T.  Epilogue: norm backward of q, per-item
//               partial of dwq.
//   k_bwd_dkdv  work item = (segment, 128-key tile, head).  One pass over the query tiles:
//               S = Q^ K^T and dP = dO V^T with the wave's 32 keys in registers, P and dS in fp16,
//               dV^T += dO16^T P and dK^T += Q^16^T dS.  Epilogue: norm backward of k, dwk partial.
// Then three small kernels sum the per-item weight partials in a fixed tree (heads, items, chunks).
//
// D is recomputed rather than taken as rowsum(dO o O) from the forward's bf16 output: with a sharp
// softmax the rounding of O moves D enough to cost dq and dk about twice the accuracy bound.
// P and dS enter their products as fp16 (bf16 would miss the bound, as for the forward's P).
#include "h3_common.h"
#include "h3_launch.h"
#include "h3_tiles.h"

namespace h3 {

constexpr int BW = 4;  // waves per workgroup, one per SIMD; each owns 32 rows (queries or keys)
static_assert(BT == 32 * BW, "one 32-row block per wave");
static_assert(TILE_ROWS == 64, "64-row tiles of the contracted dimension");

struct BwdParams {
  const uint16_t* q;  // raw inputs, token-major (norm backward)
  const uint16_t* k;
  const uint16_t* wq;
  const uint16_t* wk;
  const uint16_t* qhat;  // staged operands, head-major
  const uint16_t* qhat16;
  const uint16_t* khat;
  const uint16_t* khat16;
  const uint16_t* vh;
  const uint16_t* doh;
  const uint16_t* do16;
  const float* lse2;
  float* delta;
  uint16_t* dq;  // outputs, token-major
  uint16_t* dk;
  uint16_t* dv;
  float* dwq_part;  // [max_items][H][128]
  float* dwk_part;
  const WsHeader* hdr;
  const int32_t* segtab;
  const int32_t* items;
  int64_t T;
  int32_t H;
  float eps;
  float c;      // scale * log2(e)
  float scale;
  int32_t xcd_slots;
};

// One work item of the persistent walk (XCD-aware head-major order, as in the forward).
struct WorkItem {
  int head, item, s0, L, tile;
};

__device__ __forceinline__ bool next_item(const BwdParams& p, int round, int nitems, int nseg, WorkItem& w, bool& done) {
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int64_t v = ((int64_t)round * 8 + xcd) * p.xcd_slots + slot;
  done = v >= (int64_t)nitems * p.H;
  if (done) return false;
  w.head = (int)(v / nitems);
  w.item = (int)(v - (int64_t)w.head * nitems);
  const int seg = p.items[2 * w.item];
  w.tile = p.items[2 * w.item + 1];
  if ((unsigned)seg >= (unsigned)nseg) return false;
  w.s0 = p.segtab[2 * seg];
  w.L = p.segtab[2 * seg + 1];
  return !(w.s0 < 0 || w.L <= 0 || (int64_t)w.s0 + w.L > p.T || w.tile < 0 || w.tile * BT >= w.L);
}

// The lane's 32-row block as a B operand of a 32x32x16 MFMA: row l32 of rows [row0, row0+32) of a
// head-major [.][128] array, dims 16m + 8hh .. +8 in register m; rows at or past nvalid are zero.
__device__ __forceinline__ void load_b_rows(const uint16_t* rows, int nvalid, int l32, int hh, bf16x8* out) {
  const bool ok = l32 < nvalid;
  const uint16_t* r = rows + (int64_t)(ok ? l32 : 0) * HD;
#pragma unroll
  for (int m = 0; m < 8; m++) {
    u32x4 w = {0, 0, 0, 0};
    if (ok) w = *(const u32x4*)(r + 16 * m + 8 * hh);
    out[m] = __builtin_bit_cast(bf16x8, w);
  }
}

// Copy 64 fp32 values (rows [0, valid) of a row vector; the rest read as zero) into LDS: one
// dword per lane of one wave.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ void rowvec_to_lds(const float* g, int valid, lds_char* lds, int lane) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g, (short)0, (valid < TILE_ROWS ? valid : TILE_ROWS) * 4, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 4, lane * 4, 0, 0, 0);
}

// Rows of the dw terms in LDS are padded to 132 floats: with 128 the 32 rows a wave writes at once
// would all start in the same bank.
constexpr int RED_STRIDE = HD + 4;
static_assert(BT * RED_STRIDE * 4 <= 6 * TILE_ELEMS * 2, "dw rows fit in the tiles they replace");

// RMSNorm backward of one row held as a lane pair in the accumulator layout (dims 32db + 8g + 4hh +
// e in dy[db][4g + e]), dy = the gradient with respect to the normed output; x: the raw row (bf16,
// token-major), w: the weight.  Writes dx = r g - (r^3 / 128) x (g . x), g = w o dy, rounded once
// to bf16 (if store), and the row's dw terms dy o x r into red[row][dim] (LDS, row stride
// RED_STRIDE).  r is the forward's FP64 value (same fixed tree); the rest is evaluated in FP64,
// g . x over the lane's dims in a fixed order and then across the pair.
__device__ __forceinline__ void norm_bwd_pair(const f32x16* dy, const uint16_t* x, const uint16_t* w, float eps,
                                              int hh, bool store, uint16_t* dx, float* red, int row) {
  double part[8];
  {
    float xs[8][8];
#pragma unroll
    for (int m = 0; m < 8; m++) unpack8_bf16(*(const u32x4*)(x + 16 * m + 8 * hh), xs[m]);
#pragma unroll
    for (int m = 0; m < 8; m++) part[m] = chunk_sumsq(xs[m]);
  }
  const double r = norm_rscale(row_total_2lanes(part), eps);
  auto chunk = [&](int db, int g, float* xf, float* wf) {
    const int d0 = 32 * db + 8 * g + 4 * hh;
    const u32x2 xw = *(const u32x2*)(x + d0);
    const u32x2 ww = *(const u32x2*)(w + d0);
    xf[0] = bf16_lo(xw[0]), xf[1] = bf16_hi(xw[0]), xf[2] = bf16_lo(xw[1]), xf[3] = bf16_hi(xw[1]);
    wf[0] = bf16_lo(ww[0]), wf[1] = bf16_hi(ww[0]), wf[2] = bf16_lo(ww[1]), wf[3] = bf16_hi(ww[1]);
  };
  double gx = 0.0;
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int g = 0; g < 4; g++) {
      float xf[4], wf[4];
      chunk(db, g, xf, wf);
#pragma unroll
      for (int e = 0; e < 4; e++) gx = __builtin_fma((double)wf[e] * (double)dy[db][4 * g + e], (double)xf[e], gx);
    }
  gx = gx + __shfl_xor(gx, 32, 64);  // both halves of the row (commutative: same bits in both lanes)
  const double k3 = r * r * r * 0.0078125 * gx;
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const int d0 = 32 * db + 8 * g + 4 * hh;
      float xf[4], wf[4];
      chunk(db, g, xf, wf);
      uint32_t o[4];
      f32x4 t4;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const double dyv = (double)dy[db][4 * g + e];
        o[e] = f64_to_bf16_rne(r * ((double)wf[e] * dyv) - k3 * (double)xf[e]);
        t4[e] = store ? (float)(dyv * (double)xf[e] * r) : 0.0f;
      }
      *(f32x4*)&red[row * RED_STRIDE + d0] = t4;
      if (store) {
        u32x2 o2;
        o2[0] = o[0] | (o[1] << 16);
        o2[1] = o[2] | (o[3] << 16);
        *(u32x2*)(dx + d0) = o2;
      }
    }
}

// Sum the workgroup's 128 rows of dw terms (red[row][dim], LDS) into one partial [128] in a fixed
// order (rows ascending).  The caller has written every row (zeros for rows past the segment end).
__device__ __forceinline__ void dw_reduce(const float* red, int tid, float* out) {
  __syncthreads();
  if (tid < HD) {
    float s = 0.0f;
    for (int r = 0; r < BT; r++) s += red[r * RED_STRIDE + tid];
    out[tid] = s;
  }
}

// Store a row held as a lane pair in the accumulator layout, times s, rounded once to bf16.
__device__ __forceinline__ void store_row(const f32x16* acc, float s, int hh, uint16_t* out) {
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const int d0 = 32 * db + 8 * g + 4 * hh;
      u32x2 o2;
      o2[0] = pack_bf16(acc[db][4 * g] * s, acc[db][4 * g + 1] * s);
      o2[1] = pack_bf16(acc[db][4 * g + 2] * s, acc[db][4 * g + 3] * s);
      *(u32x2*)(out + d0) = o2;
    }
}

__device__ __forceinline__ bool fill_nan_if_bad(const BwdParams& p, uint16_t* a, uint16_t* b) {
  if (p.hdr->status == 0) return false;
  const int64_t n16 = p.T * p.H * HD / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n16; e += stride) {
    *(u32x4*)(a + e * 8) = nan4;
    if (b) *(u32x4*)(b + e * 8) = nan4;
  }
  return true;
}

template <int N>
struct Par2 {
  static constexpr int value = N;
};

// ============================================================================== dq (and D)

__global__ __launch_bounds__(64 * BW, 1) void k_bwd_dq(BwdParams p) {
  // tiles 0, 1: K^16 (transposed reads) of stage 0 / 1; 2, 3: K^; 4, 5: V (row reads)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[6 * TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  if (fill_nan_if_bad(p, p.dq, nullptr)) return;

  const int64_t T = p.T;
  const int H = p.H;
  const int64_t max_items = T + (T + BT - 1) / BT;
  const int nseg = (int)min((int64_t)max(p.hdr->nseg, 0), T);
  const int nitems = (int)min((int64_t)max(p.hdr->nitems, 0), max_items);
  const int krow_off = tile_lane_offset(false, wv, lane);
  const int ktr_off = tile_lane_offset(true, wv, lane);
  uint32_t vb[4];
  tr_bases(lds, lane, vb);
  const float c = p.c;

  for (int round = 0;; round++) {
    WorkItem w;
    bool done;
    const bool ok = next_item(p, round, nitems, nseg, w, done);
    if (done) break;
    if (!ok) continue;
    const int ntk = (w.L + TILE_ROWS - 1) / TILE_ROWS;
    const int rem = w.L - (ntk - 1) * TILE_ROWS;
    const int64_t hT = (int64_t)w.head * T;
    const uint16_t* kb = p.khat + (hT + w.s0) * HD;
    const uint16_t* k16b = p.khat16 + (hT + w.s0) * HD;
    const uint16_t* vbp = p.vh + (hT + w.s0) * HD;
    const int row0 = w.tile * BT + wv * 32;  // the wave's first query (segment-relative)
    const int qrow = row0 + l32;
    const bool qvalid = qrow < w.L;

    __syncthreads();  // the previous item's LDS reads are done
    tile_to_lds<BW>(kb, w.L, lds + 2 * TILE_ELEMS, wv, krow_off);
    tile_to_lds<BW>(vbp, w.L, lds + 4 * TILE_ELEMS, wv, krow_off);

    bf16x8 qf[8], gf[8];
    load_b_rows(p.qhat + (hT + w.s0 + row0) * HD, w.L - row0, l32, hh, qf);
    load_b_rows(p.doh + (hT + w.s0 + row0) * HD, w.L - row0, l32, hh, gf);
    const float lq = qvalid ? p.lse2[hT + w.s0 + qrow] : 0.0f;

    // scores and dP of tile j from stage ST; keys past the segment end get P = 0
    auto scores = [&](auto st, int j, f32x16* S, f32x16* dP) {
      constexpr int ST = decltype(st)::value;
      gemm_scores<4>(lds + (2 + ST) * TILE_ELEMS, qf, l32, hh, S);
      gemm_scores<4>(lds + (4 + ST) * TILE_ELEMS, gf, l32, hh, dP);
      if (j == ntk - 1 && rem < TILE_ROWS) mask_tail(S, rem, hh);
    };

    // ---- pass 1: D_i = sum_j P_ij dP_ij
    float dacc = 0.0f;
    auto pass1 = [&](auto st, int j) {
      constexpr int ST = decltype(st)::value;
      copies_barrier();  // tile j has landed, every wave is done with stage 1 - ST
      if (j + 1 < ntk) {
        tile_to_lds<BW>(kb + (int64_t)(j + 1) * TILE_ELEMS, w.L - (j + 1) * TILE_ROWS, lds + (3 - ST) * TILE_ELEMS, wv,
                        krow_off);
        tile_to_lds<BW>(vbp + (int64_t)(j + 1) * TILE_ELEMS, w.L - (j + 1) * TILE_ROWS, lds + (5 - ST) * TILE_ELEMS,
                        wv, krow_off);
      }
      f32x16 S[2], dP[2];
      scores(st, j, S, dP);
      float pd[32];
#pragma unroll
      for (int kbk = 0; kbk < 2; kbk++)
#pragma unroll
        for (int i = 0; i < 16; i++)
          pd[16 * kbk + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kbk][i], c, -lq)) * dP[kbk][i];
      dacc += tree_sum<32>(pd);
    };
    {
      int j = 0;
      for (; j + 1 < ntk; j += 2) {
        pass1(Par2<0>{}, j);
        pass1(Par2<1>{}, j + 1);
      }
      if (j < ntk) pass1(Par2<0>{}, j);
    }
    float da, db_;
    swap_halves(dacc, da, db_);
    const float Dq = da + db_;
    if (qvalid && hh == 0) p.delta[hT + w.s0 + qrow] = Dq;

    // ---- pass 2: dQ^T += K^16^T dS^T
    __syncthreads();
    tile_to_lds<BW>(k16b, w.L, lds, wv, ktr_off);
    tile_to_lds<BW>(kb, w.L, lds + 2 * TILE_ELEMS, wv, krow_off);
    tile_to_lds<BW>(vbp, w.L, lds + 4 * TILE_ELEMS, wv, krow_off);
    f32x16 acc[4];
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[d][i] = 0.0f;
    auto pass2 = [&](auto st, int j) {
      constexpr int ST = decltype(st)::value;
      copies_barrier();  // tile j has landed, every wave is done with stage 1 - ST
      if (j + 1 < ntk) {
        const int64_t o = (int64_t)(j + 1) * TILE_ELEMS;
        const int v = w.L - (j + 1) * TILE_ROWS;
        tile_to_lds<BW>(k16b + o, v, lds + (1 - ST) * TILE_ELEMS, wv, ktr_off);
        tile_to_lds<BW>(kb + o, v, lds + (3 - ST) * TILE_ELEMS, wv, krow_off);
        tile_to_lds<BW>(vbp + o, v, lds + (5 - ST) * TILE_ELEMS, wv, krow_off);
      }
      f32x16 S[2], dP[2];
      scores(st, j, S, dP);
      float ds[32];
#pragma unroll
      for (int kbk = 0; kbk < 2; kbk++)
#pragma unroll
        for (int i = 0; i < 16; i++)
          ds[16 * kbk + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kbk][i], c, -lq)) * (dP[kbk][i] - Dq);
      f16x8 dsf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ks++) dsf[ks] = pack_p(&ds[8 * ks]);
      __builtin_amdgcn_sched_barrier(0);
      tr_gemm<ST>(vb, dsf, acc);
    };
    {
      int j = 0;
      for (; j + 1 < ntk; j += 2) {
        pass2(Par2<0>{}, j);
        pass2(Par2<1>{}, j + 1);
      }
      if (j < ntk) pass2(Par2<0>{}, j);
    }

    // ---- epilogue: dq^ = scale dQ, norm backward, dwq partial
    const int qr = qvalid ? qrow : 0;
    uint16_t* dqrow = p.dq + ((int64_t)(w.s0 + qr) * H + w.head) * HD;
    if (p.wq) {
      f32x16 dy[4];
#pragma unroll
      for (int d = 0; d < 4; d++)
#pragma unroll
        for (int i = 0; i < 16; i++) dy[d][i] = acc[d][i] * p.scale;
      __syncthreads();  // every wave is done with the LDS tiles: they become the dw rows
      norm_bwd_pair(dy, p.q + ((int64_t)(w.s0 + qr) * H + w.head) * HD, p.wq, p.eps, hh, qvalid, dqrow,
                    (float*)lds, wv * 32 + l32);
      dw_reduce((const float*)lds, tid, p.dwq_part + ((int64_t)w.item * H + w.head) * HD);
    } else if (qvalid) {
      store_row(acc, p.scale, hh, dqrow);
    }
  }
}

// ============================================================================== dk, dv

__global__ __launch_bounds__(64 * BW, 1) void k_bwd_dkdv(BwdParams p) {
  // tiles 0, 1: Q^16, 2, 3: dO16 (transposed reads) of stage 0 / 1; 4, 5: Q^, 6, 7: dO (row reads);
  // then the fp32 rows [stage][lse2, D][64 queries]
  __shared__ __attribute__((aligned(1024))) uint16_t lds[8 * TILE_ELEMS + 2 * 2 * TILE_ROWS * 2];
  const float* lrow = (const float*)(lds + 8 * TILE_ELEMS);  // lrow[(2 * stage + which) * 64 + query]
  lds_char* const lrow3 = (lds_char*)lds + 8 * TILE_ELEMS * 2;  // the same rows as an LDS address

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  if (fill_nan_if_bad(p, p.dk, p.dv)) return;

  const int64_t T = p.T;
  const int H = p.H;
  const int64_t max_items = T + (T + BT - 1) / BT;
  const int nseg = (int)min((int64_t)max(p.hdr->nseg, 0), T);
  const int nitems = (int)min((int64_t)max(p.hdr->nitems, 0), max_items);
  const int row_off = tile_lane_offset(false, wv, lane);
  const int tr_off = tile_lane_offset(true, wv, lane);
  uint32_t vb[4];
  tr_bases(lds, lane, vb);
  const float c = p.c;

  for (int round = 0;; round++) {
    WorkItem w;
    bool done;
    const bool ok = next_item(p, round, nitems, nseg, w, done);
    if (done) break;
    if (!ok) continue;
    const int ntq = (w.L + TILE_ROWS - 1) / TILE_ROWS;
    const int64_t hT = (int64_t)w.head * T;
    const uint16_t* qb = p.qhat + (hT + w.s0) * HD;
    const uint16_t* q16b = p.qhat16 + (hT + w.s0) * HD;
    const uint16_t* gb = p.doh + (hT + w.s0) * HD;
    const uint16_t* g16b = p.do16 + (hT + w.s0) * HD;
    const float* lb = p.lse2 + hT + w.s0;
    const float* db = p.delta + hT + w.s0;
    const int row0 = w.tile * BT + wv * 32;  // the wave's first key (segment-relative)
    const int krow = row0 + l32;
    const bool kvalid = krow < w.L;

    // stage ST of the tiles of query tile j (ST a compile-time constant at every call, so the
    // compiler sees that a copy never writes the stage being read and adds no wait for it)
    auto copies = [&](int j, auto stage) {
      constexpr int st = decltype(stage)::value;
      const int64_t o = (int64_t)j * TILE_ELEMS;
      const int v = w.L - j * TILE_ROWS;
      tile_to_lds<BW>(q16b + o, v, lds + (0 + st) * TILE_ELEMS, wv, tr_off);
      tile_to_lds<BW>(g16b + o, v, lds + (2 + st) * TILE_ELEMS, wv, tr_off);
      tile_to_lds<BW>(qb + o, v, lds + (4 + st) * TILE_ELEMS, wv, row_off);
      tile_to_lds<BW>(gb + o, v, lds + (6 + st) * TILE_ELEMS, wv, row_off);
      if (wv == 0) rowvec_to_lds(lb + j * TILE_ROWS, v, lrow3 + (2 * st + 0) * TILE_ROWS * 4, lane);
      if (wv == 1) rowvec_to_lds(db + j * TILE_ROWS, v, lrow3 + (2 * st + 1) * TILE_ROWS * 4, lane);
    };

    __syncthreads();  // the previous item's LDS reads are done
    copies(0, Par2<0>{});
    bf16x8 kf[8], vf[8];
    load_b_rows(p.khat + (hT + w.s0 + row0) * HD, w.L - row0, l32, hh, kf);
    load_b_rows(p.vh + (hT + w.s0 + row0) * HD, w.L - row0, l32, hh, vf);

    f32x16 dv[4], dk[4];
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int i = 0; i < 16; i++) dv[d][i] = dk[d][i] = 0.0f;

    auto step = [&](auto st, int j) {
      constexpr int ST = decltype(st)::value;
      copies_barrier();  // tile j has landed, every wave is done with stage 1 - ST
      if (j + 1 < ntq) copies(j + 1, Par2<1 - ST>{});
      // S[qb][i] / dP[qb][i]: query 32qb + 8(i/4) + 4hh + (i%4) of the tile, key = the lane's key
      f32x16 S[2], dP[2];
      gemm_scores<4>(lds + (4 + ST) * TILE_ELEMS, kf, l32, hh, S);
      gemm_scores<4>(lds + (6 + ST) * TILE_ELEMS, vf, l32, hh, dP);
      float pr[2][16], ds[2][16];
#pragma unroll
      for (int qb = 0; qb < 2; qb++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const f32x4 l4 = *(const f32x4*)&lrow[(2 * ST + 0) * TILE_ROWS + 32 * qb + 8 * g + 4 * hh];
          const f32x4 d4 = *(const f32x4*)&lrow[(2 * ST + 1) * TILE_ROWS + 32 * qb + 8 * g + 4 * hh];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][4 * g + e], c, -l4[e]));
            pr[qb][4 * g + e] = pv;
            ds[qb][4 * g + e] = pv * (dP[qb][4 * g + e] - d4[e]);
          }
        }
      f16x8 pf[4], dsf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        pf[ks] = pack_p(&pr[ks >> 1][8 * (ks & 1)]);
        dsf[ks] = pack_p(&ds[ks >> 1][8 * (ks & 1)]);
      }
      __builtin_amdgcn_sched_barrier(0);
      tr_gemm<2 + ST>(vb, pf, dv);   // dV^T += dO16^T P
      tr_gemm<0 + ST>(vb, dsf, dk);  // dK^T += Q^16^T dS
    };
    {
      int j = 0;
      for (; j + 1 < ntq; j += 2) {
        step(Par2<0>{}, j);
        step(Par2<1>{}, j + 1);
      }
      if (j < ntq) step(Par2<0>{}, j);
    }

    // ---- epilogue: dv, dk^ = scale dK, norm backward, dwk partial
    const int kr = kvalid ? krow : 0;
    const int64_t orow = ((int64_t)(w.s0 + kr) * H + w.head) * HD;
    if (kvalid) store_row(dv, 1.0f, hh, p.dv + orow);
    if (p.wk) {
      f32x16 dy[4];
#pragma unroll
      for (int d = 0; d < 4; d++)
#pragma unroll
        for (int i = 0; i < 16; i++) dy[d][i] = dk[d][i] * p.scale;
      __syncthreads();  // every wave is done with the LDS tiles: they become the dw rows
      norm_bwd_pair(dy, p.k + orow, p.wk, p.eps, hh, kvalid, p.dk + orow, (float*)lds, wv * 32 + l32);
      dw_reduce((const float*)lds, tid, p.dwk_part + ((int64_t)w.item * H + w.head) * HD);
    } else if (kvalid) {
      store_row(dk, p.scale, hh, p.dk + orow);
    }
  }
}

// ============================================================================== dw

// dw[d] = the sum of the per-(item, head) partials in a fixed tree whose shape depends only on the
// number of work items: (1) per item, over heads ascending; (2) per chunk of DW_CHUNK consecutive
// items, ascending; (3) over the chunks, ascending.  Every level keeps several independent loads
// in flight per thread (the sums themselves stay sequential), so the chains are short.  Thread t of
// a 256-thread block: t < 128 works on dwq, else on dwk, channel t % 128.

__device__ __forceinline__ float sum_strided(const float* base, int64_t n, int64_t stride) {
  float s = 0.0f;
  int64_t i = 0;
  for (; i + 8 <= n; i += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; u++) v[u] = base[(i + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; u++) s += v[u];
  }
  for (; i < n; i++) s += base[i * stride];
  return s;
}

__device__ __forceinline__ int64_t dw_items(const WsHeader* hdr, int64_t max_items) {
  return min((int64_t)max(hdr->nitems, 0), max_items);
}

// (1) item_part[item][q/k][d] = sum over heads of part[item][head][d]
__global__ __launch_bounds__(256) void k_bwd_dw_items(const WsHeader* hdr, const float* qpart, const float* kpart,
                                                      int64_t max_items, int32_t H, float* item_part) {
  const int t = threadIdx.x, d = t & (HD - 1), which = t >> 7;
  const float* part = which ? kpart : qpart;
  const int64_t n = dw_items(hdr, max_items);
  for (int64_t it = blockIdx.x; it < n; it += gridDim.x)
    item_part[(it * 2 + which) * HD + d] = sum_strided(part + it * H * HD + d, H, HD);
}

// (2) chunk_part[c][q/k][d] = sum over items c*DW_CHUNK .. of item_part
__global__ __launch_bounds__(256) void k_bwd_dw_chunks(const WsHeader* hdr, const float* item_part, int64_t max_items,
                                                       float* chunk_part) {
  const int t = threadIdx.x, d = t & (HD - 1), which = t >> 7;
  const int64_t n = dw_items(hdr, max_items);
  const int64_t nc = (n + DW_CHUNK - 1) / DW_CHUNK;
  for (int64_t c = blockIdx.x; c < nc; c += gridDim.x) {
    const int64_t i0 = c * DW_CHUNK, cnt = min((int64_t)DW_CHUNK, n - i0);
    chunk_part[(c * 2 + which) * HD + d] = sum_strided(item_part + (i0 * 2 + which) * HD + d, cnt, 2 * HD);
  }
}

// (3) dw = sum over chunks.  With a recorded data error the weights' gradients are NaN like the other
// outputs.
__global__ __launch_bounds__(256) void k_bwd_dw_final(const WsHeader* hdr, const float* chunk_part, int64_t max_items,
                                                      float* dwq, float* dwk) {
  const int t = threadIdx.x, d = t & (HD - 1), which = t >> 7;
  float* out = which ? dwk : dwq;
  if (hdr->status != 0) {
    out[d] = __builtin_nanf("");
    return;
  }
  const int64_t nc = (dw_items(hdr, max_items) + DW_CHUNK - 1) / DW_CHUNK;
  out[d] = sum_strided(chunk_part + which * HD + d, nc, 2 * HD);
}

hipError_t launch_bwd(const void* q, const void* k, const void* wq, const void* wk, int64_t T, int32_t H, float eps,
                      float scale, void* dq, void* dk, void* dv, float* dwq, float* dwk, void* ws, int grid_cap,
                      hipStream_t stream) {
  const BwdLayout Lw = bwd_layout(T, H);
  char* base = (char*)ws;
  BwdParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.wq = (const uint16_t*)wq;
  p.wk = (const uint16_t*)wk;
  p.qhat = (const uint16_t*)(base + Lw.qhat);
  p.qhat16 = (const uint16_t*)(base + Lw.qhat16);
  p.khat = (const uint16_t*)(base + Lw.khat);
  p.khat16 = (const uint16_t*)(base + Lw.khat16);
  p.vh = (const uint16_t*)(base + Lw.vh);
  p.doh = (const uint16_t*)(base + Lw.doh);
  p.do16 = (const uint16_t*)(base + Lw.do16);
  p.lse2 = (const float*)(base + Lw.lse2);
  p.delta = (float*)(base + Lw.delta);
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.dwq_part = (float*)(base + Lw.dwq);
  p.dwk_part = (float*)(base + Lw.dwk);
  p.hdr = (const WsHeader*)base;
  p.segtab = (const int32_t*)(base + Lw.segtab);
  p.items = (const int32_t*)(base + Lw.items);
  p.T = T;
  p.H = H;
  p.eps = eps;
  p.scale = scale;
  p.c = (float)((double)scale * 1.4426950408889634074);
  const int64_t max_work = Lw.max_items * H;
  int64_t grid = grid_cap < max_work ? grid_cap : max_work;
  grid = (grid + 7) & ~(int64_t)7;
  p.xcd_slots = (int32_t)(grid / 8);
  hipLaunchKernelGGL(k_bwd_dq, dim3((unsigned)grid), dim3(64 * BW), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bwd_dkdv, dim3((unsigned)grid), dim3(64 * BW), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (wq) {
    const WsHeader* hdr = (const WsHeader*)base;
    float* item_part = (float*)(base + Lw.dw_item);
    float* chunk_part = (float*)(base + Lw.dw_chunk);
    const unsigned g1 = (unsigned)(Lw.max_items < 1024 ? Lw.max_items : 1024);
    const unsigned g2 = (unsigned)(Lw.max_chunks < 256 ? Lw.max_chunks : 256);
    hipLaunchKernelGGL(k_bwd_dw_items, dim3(g1), dim3(256), 0, stream, hdr, p.dwq_part, p.dwk_part, Lw.max_items, H,
                       item_part);
    hipLaunchKernelGGL(k_bwd_dw_chunks, dim3(g2), dim3(256), 0, stream, hdr, item_part, Lw.max_items, chunk_part);
    hipLaunchKernelGGL(k_bwd_dw_final, dim3(1), dim3(256), 0, stream, hdr, chunk_part, Lw.max_items, dwq, dwk);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace h3
