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
//               D_i exactly (in fp32, a fixed tree per tile) unless the staging kernel formed it
//               from the forward's fp32 output; pass 2 recomputes S and dP, forms dS and
//               accumulates dQ^T += K^16^T dS^T.  Two workgroups share a CU (two waves per
//               SIMD, at most 256 registers each), so one wave's vector work runs beside the
//               other's MFMAs.
// The workspace keeps -D per staged row.
//   k_bwd_dkdv  work item = (segment, 128-key tile, head).  One pass over the query tiles, eight
//               waves in two roles over the item's keys (32 per wave pair, in registers): waves
//               0-3 form S = Q^ K^T, P (fp16) and dV^T += dO16^T P, and hand P through LDS to
//               waves 4-7, which form dP = dO V^T, dS in fp16 and dK^T += Q^16^T dS.  The two
//               waves of a SIMD hold different roles, so one's vector work runs beside the
//               other's MFMAs.
// With norm weights both write dq^ / dk^ in fp32 and k_bwd_norm applies the RMSNorm backward per
// row (FP64, one bf16 rounding) and writes fixed-order weight-gradient partials, which two small
// kernels sum in a fixed tree; without weights the kernels write dq, dk directly.
//
// D is recomputed (or formed from the forward's fp32 output) rather than taken as rowsum(dO o O)
// from the bf16 output: with a sharp softmax that rounding moves D enough to cost dq and dk about
// twice the accuracy bound.
// P and dS enter their products as fp16 (bf16 would miss the bound, as for the forward's P).
#include "h3_common.h"
#include "h3_norm.h"
#include "h3_bwd.h"
#include "h3_launch.h"
#include "h3_tiles_bwd.h"

namespace h3 {

constexpr int BW = 4;  // waves per workgroup, one per SIMD; each owns 32 rows (queries or keys)
static_assert(BT == 32 * BW, "one 32-row block per wave");
static_assert(TILE_ROWS == 64, "64-row tiles of the contracted dimension");

struct BwdParams {
  const uint16_t* q;  // raw inputs, token-major (norm backward)
  const uint16_t* k;
  const uint16_t* wq;
  const uint16_t* wk;
  const uint16_t* qhat16;  // staged operands, fp16, head-major
  const uint16_t* khat16;
  const uint16_t* v16;
  const uint16_t* do16;
  const float* lse2;
  float* delta;          // -D per staged row: the dP products start from it
  uint16_t* dq;  // outputs, token-major
  uint16_t* dk;
  uint16_t* dv;
  float* dqh;  // with norm weights: gradients with respect to the normed q / k, fp32, staged row-major
  float* dkh;
  const int32_t* inv;  // token of each staged row (position order), or NULL (staged row = token)
  const uint32_t* dmax;  // per (segment, head): largest |dO|, which fixes the staged dO's power of two
  const int32_t* segflag;  // per segment: nonzero = a value cannot enter the products (NaN outputs)
  int32_t delta_ready;  // D was written by the staging kernel (from the forward's fp32 output)
  const WsHeader* hdr;
  int32_t* next;  // the kernel's work counter (in the header)
  const int32_t* segtab;
  const int32_t* items;
  const int32_t* bkt;  // cost classes of the work order: (first item, item count), most expensive first
  int64_t T;
  int32_t H;
  float eps;
  float c;      // scale * log2(e)
  float scale;
};

// One work item of the persistent walk.  Items are handed out by an atomic counter (the order only
// decides which workgroup runs an item, never a result); the work index v runs over the cost
// classes of the plan in order (most expensive first) and, inside a class, head-major, so
// consecutive items share a head's operands and the cheap ones come last.
struct WorkItem {
  int head, item, seg, s0, L, tile;
};

// bkt: the plan's cost classes (first item, count), staged in LDS at the kernel's start.
__device__ __forceinline__ bool item_of(const BwdParams& p, const int32_t* bkt, int64_t v, int nitems, int nseg,
                                        int nbkt, WorkItem& w, bool& done) {
  done = v >= (int64_t)nitems * p.H;
  if (done) return false;
  int64_t base = 0;
  int b = 0, start = 0, cnt = 0;
  for (; b < nbkt; b++) {
    start = bkt[2 * b];
    cnt = bkt[2 * b + 1];
    const int64_t span = (int64_t)cnt * p.H;
    if (v < base + span) break;
    base += span;
  }
  if (b == nbkt || cnt <= 0) return false;
  const int64_t local = v - base;
  w.head = (int)(local / cnt);
  w.item = start + (int)(local - (int64_t)w.head * cnt);
  if ((unsigned)w.item >= (unsigned)nitems || (unsigned)w.head >= (unsigned)p.H) return false;
  // the item: (segment, tile, the segment's start, its length)
  const u32x4 it4 = *(const u32x4*)(p.items + 4 * w.item);
  const int seg = (int)it4[0];
  w.tile = (int)it4[1];
  if ((unsigned)seg >= (unsigned)nseg) return false;
  w.seg = seg;
  w.s0 = (int)it4[2];
  w.L = (int)it4[3];
  return !(w.s0 < 0 || w.L <= 0 || (int64_t)w.s0 + w.L > p.T || w.tile < 0 || w.tile * BT >= w.L);
}

// The next work index for the workgroup: thread 0 hands out the index it fetched during the previous
// item and fetches the following one, so the atomic's latency is hidden.  The first barrier also
// ends the previous item's LDS reads.  Both barriers guard LDS only: the previous item's output
// stores need not have landed, and the new fetch's reply is awaited with the next item's first
// copies (each kernel ties `prefetched` after that wait, and after an explicit one on the paths
// that skip the copies, so the compiler needs no memory wait here).
__device__ __forceinline__ int64_t take_work(const BwdParams& p, int tid, int32_t& prefetched, int32_t* s_next) {
  lds_barrier();
  if (tid == 0) {
    *s_next = prefetched;
    prefetched = atomicAdd(p.next, 1);
  }
  lds_barrier();
  return *s_next;
}

// After an explicit vmcnt(0): the counter's reply has arrived; from here on the compiler treats
// the register as written by ordinary code, so no later use waits for memory.
__device__ __forceinline__ void reply_landed(int32_t& prefetched) { asm volatile("" : "+v"(prefetched)); }

// The lane's 32-row block as a B operand of a 32x32x16 MFMA: row l32 of rows [row0, row0+32) of a
// head-major [.][128] array, dims 16m + 8hh .. +8 in register m; rows at or past nvalid are zero.
__device__ __forceinline__ void load_b_rows(const uint16_t* rows, int nvalid, int l32, int hh, f16x8* out) {
  const bool ok = l32 < nvalid;
  const uint16_t* r = rows + (int64_t)(ok ? l32 : 0) * HD;
#pragma unroll
  for (int m = 0; m < 8; m++) {
    u32x4 w = {0, 0, 0, 0};
    if (ok) w = *(const u32x4*)(r + 16 * m + 8 * hh);
    out[m] = __builtin_bit_cast(f16x8, w);
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

// Store a row held as a lane pair in the accumulator layout, times s and then 2^ex (which removes
// the staged dO's power of two exactly), rounded once to bf16.
__device__ __forceinline__ void store_row(const f32x16* acc, float s, int ex, int hh, uint16_t* out) {
  auto f = [&](float a) { return __builtin_ldexpf(a * s, ex); };
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const int d0 = 32 * db + 8 * g + 4 * hh;
      u32x2 o2;
      o2[0] = pack_bf16(f(acc[db][4 * g]), f(acc[db][4 * g + 1]));
      o2[1] = pack_bf16(f(acc[db][4 * g + 2]), f(acc[db][4 * g + 3]));
      *(u32x2*)(out + d0) = o2;
    }
}

// Store a row held as a lane pair in the accumulator layout, times s and then 2^ex, in fp32.
__device__ __forceinline__ void store_row_f32(const f32x16* acc, float s, int ex, int hh, float* out) {
  auto f = [&](float a) { return __builtin_ldexpf(a * s, ex); };
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const int d0 = 32 * db + 8 * g + 4 * hh;
      const f32x4 v = {f(acc[db][4 * g]), f(acc[db][4 * g + 1]), f(acc[db][4 * g + 2]), f(acc[db][4 * g + 3])};
      *(f32x4*)(out + d0) = v;
    }
}

// Decreasing segment ids: no segmentation exists, every output is NaN.
__device__ __forceinline__ bool fill_nan_if_bad(const BwdParams& p, uint16_t* a, uint16_t* b) {
  if (!(p.hdr->status & STATUS_SEG_BIT)) return false;
  const int64_t n16 = p.T * p.H * HD / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n16; e += stride) {
    *(u32x4*)(a + e * 8) = nan4;
    if (b) *(u32x4*)(b + e * 8) = nan4;
  }
  return true;
}

__device__ __forceinline__ f32x16 nan_acc() {
  f32x16 a;
#pragma unroll
  for (int i = 0; i < 16; i++) a[i] = __builtin_nanf("");
  return a;
}

template <int N>
struct Par2 {
  static constexpr int value = N;
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for2(F&& f) {
  if constexpr (I < N) {
    f(StepIdx<I>{});
    static_for2<I + 1, N>(f);
  }
}

// ============================================================================== dq (and D)

__global__ __launch_bounds__(64 * BW, 2) void k_bwd_dq(BwdParams p) {
  // tiles 0, 1: K^16 of stage 0 / 1 (read by rows for S and transposed for dQ); 2, 3: V16 of
  // stage 0 / 1; both in the unified layout
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * TILE_ELEMS];

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
  const int uoff = tile_lane_offset_u(wv, lane);
  uint32_t vb[8];
  tr_bases_u(lds, lane, vb);
  const RowBases rb = row_bases_u(lds, l32, hh);
  const float c = p.c;

  const int nbkt = min(max(p.hdr->nbkt, 0), NBKT);
  __shared__ int32_t s_next;
  __shared__ int32_t s_bkt[2 * NBKT];
  if (tid < 2 * NBKT) s_bkt[tid] = tid < 2 * nbkt ? p.bkt[tid] : 0;
  int32_t prefetched = tid == 0 ? atomicAdd(p.next, 1) : 0;
  __builtin_amdgcn_s_waitcnt(0xF70);
  reply_landed(prefetched);
  for (;;) {
    WorkItem w;
    bool done;
    const int64_t v = take_work(p, tid, prefetched, &s_next);
    const bool ok = item_of(p, s_bkt, v, nitems, nseg, nbkt, w, done);
    if (done) break;
    if (!ok) {
      __builtin_amdgcn_s_waitcnt(0xF70);
      reply_landed(prefetched);
      continue;
    }
    // the segment's flag and dO scale: loaded now, used once the first copies have landed
    const int flag = p.segflag[w.seg];
    const uint32_t dmx = p.dmax[(int64_t)w.seg * H + w.head];
    const int ntk = (w.L + TILE_ROWS - 1) / TILE_ROWS;
    const int rem = w.L - (ntk - 1) * TILE_ROWS;
    const int64_t hT = (int64_t)w.head * T;
    const uint16_t* k16b = p.khat16 + (hT + w.s0) * HD;
    const uint16_t* v16b = p.v16 + (hT + w.s0) * HD;
    const int row0 = w.tile * BT + wv * 32;  // the wave's first query (segment-relative)
    const int qrow = row0 + l32;
    const bool qvalid = qrow < w.L;

    // key tile j into stage ST (compile-time, so the compiler sees that a copy never writes the
    // stage being read)
    auto copies = [&](int j, auto stage) {
      constexpr int ST = decltype(stage)::value;
      const int64_t o = (int64_t)j * TILE_ELEMS;
      const int v = w.L - j * TILE_ROWS;
      tile_to_lds<BW>(k16b + o, v, lds + (0 + ST) * TILE_ELEMS, wv, uoff);
      tile_to_lds<BW>(v16b + o, v, lds + (2 + ST) * TILE_ELEMS, wv, uoff);
    };

    copies(0, Par2<0>{});
    f16x8 qf[8], gf[8];
    load_b_rows(p.qhat16 + (hT + w.s0 + row0) * HD, w.L - row0, l32, hh, qf);
    load_b_rows(p.do16 + (hT + w.s0 + row0) * HD, w.L - row0, l32, hh, gf);
    const float lq = qvalid ? p.lse2[hT + w.s0 + qrow] : 0.0f;
    const float d_staged = (p.delta_ready && qvalid) ? -p.delta[hT + w.s0 + qrow] : 0.0f;
    __builtin_amdgcn_s_waitcnt(0xF70);  // tile 0, the rows, the flag and the counter's reply have landed
    reply_landed(prefetched);
    if (flag != 0) {  // a flagged segment: NaN rows (the order maps are not trusted there)
      const int qr = w.tile * BT + wv * 32 + l32;
      if (qr < w.L) {
        const int64_t srow = w.s0 + qr;
        const f32x16 nan16 = nan_acc();
        const f32x16 nan4[4] = {nan16, nan16, nan16, nan16};
        if (p.wq) store_row_f32(nan4, 1.0f, 0, hh, p.dqh + (srow * H + w.head) * HD);
        else store_row(nan4, 1.0f, 0, hh, p.dq + (srow * H + w.head) * HD);
      }
      continue;
    }

    // S = K^ Q^T and dP = V dO^T of key tile j from stage ST (key 32kb + 8(i/4) + 4hh + (i%4), the
    // lane's query); keys past the segment end get P = 0
    auto scores = [&](auto stage, int j, f32x16* S, f32x16* dP) {
      constexpr int ST = decltype(stage)::value;
      gemm_rows<0 + ST>(rb, qf, S, [](auto) {});
      gemm_rows<2 + ST>(rb, gf, dP, [](auto) {});
      if (j == ntk - 1 && rem < TILE_ROWS) mask_tail(S, rem, hh);
    };

    // ---- pass 1: D_i = sum_j P_ij dP_ij (unless the staging kernel computed D = dO . O)
    float Dq;
    if (p.delta_ready) {
      Dq = d_staged;
    } else {
      float dacc = 0.0f;
      auto pass1 = [&](auto stage, int j) {
        constexpr int ST = decltype(stage)::value;
        copies_barrier();  // tile j has landed, every wave is done with stage 1 - ST
        if (j + 1 < ntk) copies(j + 1, Par2<1 - ST>{});
        f32x16 S[2], dP[2];
        scores(stage, j, S, dP);
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
      Dq = da + db_;
      if (qvalid && hh == 0) p.delta[hT + w.s0 + qrow] = -Dq;
      __syncthreads();  // every wave is done with pass 1's tiles
      copies(0, Par2<0>{});
    }

    // ---- pass 2: dQ^T += K^16^T dS^T
    f32x16 acc[4];
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[d][i] = 0.0f;
    auto pass2 = [&](auto stage, int j) {
      constexpr int ST = decltype(stage)::value;
      copies_barrier();  // tile j has landed, every wave is done with stage 1 - ST
      if (j + 1 < ntk) copies(j + 1, Par2<1 - ST>{});
      f32x16 S[2], dP[2];
      gemm_rows<0 + ST>(rb, qf, S, [](auto) {});
      if (j == ntk - 1 && rem < TILE_ROWS) mask_tail(S, rem, hh);
      float pr[32], ds[32];
      f16x8 dsf[4];
      // dS = P (dP - D) in fp16, dP block-major: P (four elements per step) between the first
      // eight MFMAs, block 0's dS (two per step) between the last eight, block 1's after them
      gemm_rows<2 + ST, 4, true>(rb, gf, dP, [&](auto st) {
        constexpr int s = decltype(st)::value;
        if constexpr (s < 8) {
#pragma unroll
          for (int u = 0; u < 4; u++) {
            const int e = 4 * s + u;
            pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e >> 4][e & 15], c, -lq));
          }
        } else {
#pragma unroll
          for (int u = 0; u < 2; u++) {
            const int e = 2 * (s - 8) + u;
            ds[e] = pr[e] * (dP[0][e] - Dq);
          }
          if constexpr ((s & 3) == 3) dsf[(s - 8) >> 2] = pack_p(&ds[8 * ((s - 8) >> 2)]);
        }
      });
#pragma unroll
      for (int e = 16; e < 32; e++) ds[e] = pr[e] * (dP[1][e - 16] - Dq);
      dsf[2] = pack_p(&ds[16]);
      dsf[3] = pack_p(&ds[24]);
      const f16x8* bop[1] = {dsf};
      f32x16* accp[1] = {acc};
      tr_gemm_hooked<TilePair<ST, ST>, 1>(vb, bop, accp, [](auto) {});
    };
    {
      int j = 0;
      for (; j + 1 < ntk; j += 2) {
        pass2(Par2<0>{}, j);
        pass2(Par2<1>{}, j + 1);
      }
      if (j < ntk) pass2(Par2<0>{}, j);
    }

    // ---- epilogue: dq^ = scale dQ 2^-s (fp32 for the norm backward, else the output itself)
    if (qvalid) {
      const int64_t srow = w.s0 + qrow;
      const int ex = -dout_scale_exp(dmx);
      if (p.wq) {
        store_row_f32(acc, p.scale, ex, hh, p.dqh + (srow * H + w.head) * HD);
      } else {
        const int64_t trow = p.inv ? (int64_t)p.inv[srow] : srow;
        store_row(acc, p.scale, ex, hh, p.dq + (trow * H + w.head) * HD);
      }
    }
  }
}

// ============================================================================== dk, dv

// The P exchange of the dk/dv kernel: wave kw of the P role writes its lanes' packed fp16 P (the
// B operand of its dV products; lane-major 16-byte pieces, so both sides are free of bank
// conflicts) and wave kw + 4 reads it back after a barrier; one asm block each, with the wait
// inside, so no register of the exchange is touched while an LDS operation on it is in flight.
__device__ __forceinline__ void xch_write(uint32_t a, const f16x8 (&pf)[4]) {
  asm volatile(
      "ds_write_b128 %0, %1\n\t"
      "ds_write_b128 %0, %2 offset:1024\n\t"
      "ds_write_b128 %0, %3 offset:2048\n\t"
      "ds_write_b128 %0, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "v"(a), "v"(pf[0]), "v"(pf[1]), "v"(pf[2]), "v"(pf[3])
      : "memory");
}
__device__ __forceinline__ void xch_read(uint32_t a, f16x8 (&pf)[4]) {
  f16x8 v0, v1, v2, v3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
      : "v"(a)
      : "memory");
  pf[0] = v0; pf[1] = v1; pf[2] = v2; pf[3] = v3;
}

// Eight waves, two per SIMD, in two roles over the same 128 keys: wave kw (< 4) recomputes
// S = Q^ K^T and P for keys 32kw .. 32kw + 31, hands P (fp16, as its dV products take it) to wave
// kw + 4 through LDS and accumulates dV^T += dO16^T P; wave kw + 4 computes dP = dO V^T,
// dS = P (dP - D) and dK^T += Q^16^T dS.  Waves kw and kw + 4 share a SIMD, so each one's vector
// work runs beside the other's MFMAs.
constexpr int BWK = 2 * BW;

__global__ __launch_bounds__(64 * BWK, 1) void k_bwd_dkdv(BwdParams p) {
  // tiles 0, 1: Q^16 and 2, 3: dO16 of stage 0 / 1, in the unified layout (read by rows for S and
  // dP, transposed for dK and dV); then the fp32 rows [stage][lse2, D][64 queries]; then the P
  // exchange, 4 KB per key block
  constexpr int XCH_OFF = 4 * TILE_ELEMS * 2 + 2 * 2 * TILE_ROWS * 4;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[XCH_OFF / 2 + BW * 64 * 32];
  lds_char* const lrow3 = (lds_char*)lds + 4 * TILE_ELEMS * 2;  // the same rows as an LDS address

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wv >> 2, kw = wv & 3;  // role 0: P and dV; 1: dS and dK; kw: the key block
  const int hh = lane >> 5, l32 = lane & 31;
  if (fill_nan_if_bad(p, p.dk, p.dv)) return;

  const int64_t T = p.T;
  const int H = p.H;
  const int64_t max_items = T + (T + BT - 1) / BT;
  const int nseg = (int)min((int64_t)max(p.hdr->nseg, 0), T);
  const int nitems = (int)min((int64_t)max(p.hdr->nitems, 0), max_items);
  const int uoff = tile_lane_offset_u(wv, lane);
  uint32_t vb[8];
  tr_bases_u(lds, lane, vb);
  const RowBases rb = row_bases_u(lds, l32, hh);
  const uint32_t lrow_lane = (uint32_t)(size_t)lrow3 + 16 * hh;  // lrow[4hh] as an LDS byte address
  const uint32_t xch = (uint32_t)(size_t)((lds_char*)lds + XCH_OFF) + kw * 4096 + lane * 16;
  const float c = p.c;

  const int nbkt = min(max(p.hdr->nbkt, 0), NBKT);
  __shared__ int32_t s_next;
  __shared__ int32_t s_bkt[2 * NBKT];
  if (tid < 2 * NBKT) s_bkt[tid] = tid < 2 * nbkt ? p.bkt[tid] : 0;
  int32_t prefetched = tid == 0 ? atomicAdd(p.next, 1) : 0;
  __builtin_amdgcn_s_waitcnt(0xF70);
  reply_landed(prefetched);
  for (;;) {
    WorkItem w;
    bool done;
    const int64_t v = take_work(p, tid, prefetched, &s_next);
    const bool ok = item_of(p, s_bkt, v, nitems, nseg, nbkt, w, done);
    if (done) break;
    if (!ok) {
      __builtin_amdgcn_s_waitcnt(0xF70);
      reply_landed(prefetched);
      continue;
    }
    const int row0 = w.tile * BT + kw * 32;  // the wave's first key (segment-relative)
    const int krow = row0 + l32;
    const bool kvalid = krow < w.L;
    // the segment's flag and dO scale: loaded now, used once the first copies have landed
    const int flag = p.segflag[w.seg];
    const uint32_t dmx = p.dmax[(int64_t)w.seg * H + w.head];
    const int ntq = (w.L + TILE_ROWS - 1) / TILE_ROWS;
    const int64_t hT = (int64_t)w.head * T;
    const uint16_t* q16b = p.qhat16 + (hT + w.s0) * HD;
    const uint16_t* g16b = p.do16 + (hT + w.s0) * HD;
    const float* lb = p.lse2 + hT + w.s0;
    const float* db = p.delta + hT + w.s0;
    const int64_t srow = w.s0 + krow;

    // query tile j into stage ST (compile-time: the compiler sees that a copy never writes the
    // stage being read); all eight waves share the copies
    auto copies = [&](int j, auto stage) {
      constexpr int st = decltype(stage)::value;
      const int64_t o = (int64_t)j * TILE_ELEMS;
      const int v = w.L - j * TILE_ROWS;
      tile_to_lds<BWK>(q16b + o, v, lds + (0 + st) * TILE_ELEMS, wv, uoff);
      tile_to_lds<BWK>(g16b + o, v, lds + (2 + st) * TILE_ELEMS, wv, uoff);
      if (wv == 0) rowvec_to_lds(lb + j * TILE_ROWS, v, lrow3 + (2 * st + 0) * TILE_ROWS * 4, lane);
      if (wv == 1) rowvec_to_lds(db + j * TILE_ROWS, v, lrow3 + (2 * st + 1) * TILE_ROWS * 4, lane);
    };

    copies(0, Par2<0>{});
    // the wave's 32 rows of K^ (P role) or V (dS role): the B operand of its S or dP products
    f16x8 bf[8];
    load_b_rows((role == 0 ? p.khat16 : p.v16) + (hT + w.s0 + row0) * HD, w.L - row0, l32, hh, bf);
    __builtin_amdgcn_s_waitcnt(0xF70);  // tile 0, the rows, the flag and the counter's reply have landed
    reply_landed(prefetched);
    if (flag != 0) {  // a flagged segment: NaN rows (the order maps are not trusted there)
      if (kvalid) {
        const int64_t srow = w.s0 + krow;
        const f32x16 nan16 = nan_acc();
        const f32x16 nan4[4] = {nan16, nan16, nan16, nan16};
        if (role == 0) store_row(nan4, 1.0f, 0, hh, p.dv + (srow * H + w.head) * HD);
        else if (p.wk) store_row_f32(nan4, 1.0f, 0, hh, p.dkh + (srow * H + w.head) * HD);
        else store_row(nan4, 1.0f, 0, hh, p.dk + (srow * H + w.head) * HD);
      }
      continue;
    }
    const int ex = -dout_scale_exp(dmx);
    // lse (R = 0) or -D (R = 1) of the tile's queries in the S layout (query 32q2 + 8g + 4hh + i),
    // read as assembly: a plain LDS load here would make the compiler wait for every outstanding
    // copy first (it cannot tell the copies' targets from these rows), which would expose the
    // latency of the copies just issued
    auto rowvals = [&](auto stage, auto which, f32x4 (&r4)[2][4]) {
      constexpr int ST = decltype(stage)::value, R = decltype(which)::value;
      static_for2<0, 8>([&](auto gi) {
        constexpr int q2 = decltype(gi)::value >> 2, g = decltype(gi)::value & 3;
        r4[q2][g] = __builtin_bit_cast(f32x4, ds_read_b128_asm<((2 * ST + R) * TILE_ROWS + 32 * q2 + 8 * g) * 4>(lrow_lane));
      });
    };
    auto rowvals_wait = [&](f32x4 (&r4)[2][4]) {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r4[0][0]));
#pragma unroll
      for (int q2 = 0; q2 < 2; q2++)
#pragma unroll
        for (int g = 0; g < 4; g++) asm volatile("" : "+v"(r4[q2][g]));
    };

    if (role == 0) {
      const f16x8* kf = bf;
      f32x16 dv[4];
#pragma unroll
      for (int d = 0; d < 4; d++)
#pragma unroll
        for (int i = 0; i < 16; i++) dv[d][i] = 0.0f;
      // query tile j from stage ST: S = Q^ K^T (query 32q2 + 8(i/4) + 4hh + (i%4), the lane's
      // key), P = exp2(S c - lse2) to the exchange, then dV^T += dO16^T P16
      auto step = [&](auto stage, int j) {
        constexpr int ST = decltype(stage)::value;
        copies_barrier();  // tile j has landed, every wave is done with stage 1 - ST
        if (j + 1 < ntq) copies(j + 1, Par2<1 - ST>{});
        f32x4 l4[2][4];
        rowvals(stage, Par2<0>{}, l4);
        f32x16 S[2];
        float pr[2][16];
        // block-major S: block 0 is complete after step 7, and its P is formed between the MFMAs of
        // block 1 (two elements per step)
        gemm_rows<0 + ST, 4, true>(rb, kf, S, [&](auto st) {
          constexpr int s = decltype(st)::value;
          if constexpr (s == 0) {  // step 0 waited for every read but the newest four: the lse rows are in
            asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(l4[0][0]), "+v"(l4[0][1]), "+v"(l4[0][2]), "+v"(l4[0][3]),
                         "+v"(l4[1][0]), "+v"(l4[1][1]), "+v"(l4[1][2]), "+v"(l4[1][3]));
          }
          if constexpr (s >= 8) {
#pragma unroll
            for (int u = 0; u < 2; u++) {
              const int i = 2 * (s - 8) + u;
              pr[0][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[0][i], c, -l4[0][i >> 2][i & 3]));
            }
          }
        });
#pragma unroll
        for (int i = 0; i < 16; i++) pr[1][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[1][i], c, -l4[1][i >> 2][i & 3]));
        f16x8 pf[4];
#pragma unroll
        for (int sl = 0; sl < 4; sl++) pf[sl] = pack_p(&pr[sl >> 1][8 * (sl & 1)]);
        xch_write(xch, pf);
        phase_barrier();  // P of tile j is visible to the dS waves
        const f16x8* bop[1] = {pf};
        f32x16* acc[1] = {dv};
        tr_gemm_hooked<TilePair<2 + ST, 2 + ST>, 1>(vb, bop, acc, [](auto) {});
      };
      int j = 0;
      for (; j + 1 < ntq; j += 2) {
        step(Par2<0>{}, j);
        step(Par2<1>{}, j + 1);
      }
      if (j < ntq) step(Par2<0>{}, j);
      // ---- epilogue: dv 2^-s
      if (kvalid) {
        const int64_t trow = p.inv ? (int64_t)p.inv[srow] : srow;
        store_row(dv, 1.0f, ex, hh, p.dv + (trow * H + w.head) * HD);
      }
    } else {
      const f16x8* vf = bf;
      f32x16 dk[4];
#pragma unroll
      for (int d = 0; d < 4; d++)
#pragma unroll
        for (int i = 0; i < 16; i++) dk[d][i] = 0.0f;
      // query tile j from stage ST: dP = dO V^T, then (once P is in the exchange) dS = P (dP - D)
      // in fp16 and dK^T += Q^16^T dS
      auto step = [&](auto stage, int j) {
        constexpr int ST = decltype(stage)::value;
        copies_barrier();  // tile j has landed, every wave is done with stage 1 - ST
        if (j + 1 < ntq) copies(j + 1, Par2<1 - ST>{});
        f32x4 d4[2][4];
        rowvals(stage, Par2<1>{}, d4);
        f32x16 dP[2];
        gemm_rows<2 + ST>(rb, vf, dP, [](auto) {});
        rowvals_wait(d4);
        phase_barrier();  // P of tile j is in the exchange
        float pr[2][16], ds[2][16];
        {
          f16x8 pf[4];
          xch_read(xch, pf);
#pragma unroll
          for (int sl = 0; sl < 4; sl++)
#pragma unroll
            for (int e = 0; e < 8; e++) pr[sl >> 1][8 * (sl & 1) + e] = (float)pf[sl][e];
        }
#pragma unroll
        for (int q2 = 0; q2 < 2; q2++)
#pragma unroll
          for (int i = 0; i < 16; i++) ds[q2][i] = pr[q2][i] * (dP[q2][i] + d4[q2][i >> 2][i & 3]);  // d4 holds -D
        f16x8 dsf[4];
#pragma unroll
        for (int sl = 0; sl < 4; sl++) dsf[sl] = pack_p(&ds[sl >> 1][8 * (sl & 1)]);
        const f16x8* bop[1] = {dsf};
        f32x16* acc[1] = {dk};
        tr_gemm_hooked<TilePair<0 + ST, 0 + ST>, 1>(vb, bop, acc, [](auto) {});
      };
      int j = 0;
      for (; j + 1 < ntq; j += 2) {
        step(Par2<0>{}, j);
        step(Par2<1>{}, j + 1);
      }
      if (j < ntq) step(Par2<0>{}, j);
      // ---- epilogue: dk^ = scale dK 2^-s (fp32 for the norm backward, else the output itself)
      if (kvalid) {
        if (p.wk) {
          store_row_f32(dk, p.scale, ex, hh, p.dkh + (srow * H + w.head) * HD);
        } else {
          const int64_t trow = p.inv ? (int64_t)p.inv[srow] : srow;
          store_row(dk, p.scale, ex, hh, p.dk + (trow * H + w.head) * HD);
        }
      }
    }
  }
}

// ============================================================================== norm backward, dw

// RMSNorm backward of every (token, head) row: with y = (x r) o w and the gradient dy with respect
// to y (dq^ or dk^, fp32), dx = r g - (r^3 / 128) x (g . x) where g = w o dy, rounded once to bf16,
// and the weight-gradient terms dy o x r.  16 lanes per row (8 channels each), 16 rows per
// workgroup; r is the forward's FP64 value (the same fixed tree as the norm itself); g . x is
// summed in FP64, per lane over its 8 channels in order and then across the lanes in a fixed
// butterfly (partners add the same two values, so every lane holds the same bits).  Rows are walked
// in staged order (the order of dy), so the workgroup's dw partial sums its 16 rows in that order;
// x and dx are the token's rows.  blockIdx.y: 0 = q, 1 = k.
struct NormBwdParams {
  const uint16_t* x[2];  // raw q, k (token-major)
  const uint16_t* w[2];
  const float* dy[2];    // dq^, dk^
  uint16_t* dx[2];       // dq, dk
  float* part;           // [2][nparts][128]
  const int32_t* inv;    // token of each staged row, or NULL
  const int32_t* tok2seg;
  const int32_t* segflag;  // rows of a flagged segment are NaN, written at their own token row
  const float* rope_cos;   // optional MM-RoPE tables, float32 [T][48]: dy goes back through the
  const float* rope_sin;   // transposed rotation before the norm backward
  const WsHeader* hdr;
  int64_t rows;          // T * H
  int32_t H;
  int64_t nparts;
  float eps;
};

__global__ __launch_bounds__(256) void k_bwd_norm(NormBwdParams p) {
  __shared__ float red[NR][HD];
  const int which = blockIdx.y;
  const int tid = threadIdx.x;
  const int c = tid & 15;
  const int64_t row = (int64_t)blockIdx.x * NR + (tid >> 4);  // staged row: slot * H + head
  const bool valid = row < p.rows;
  if (p.hdr->status & STATUS_SEG_BIT) return;  // the attention kernels have filled the outputs with NaN
  // A staged row lies in the rows of the same segment as the token of that index, so tok2seg names
  // its segment.  In a flagged segment the order maps may be invalid: the row is NaN and stays at
  // its own index (every flag also sets the status, so dw is NaN then and the row's terms in it do
  // not matter).  Loads are unconditional, from clamped indices, so the independent ones go out
  // together: dy, w, the segment and (position order) the token first, then the flag, x and the
  // rotary table.
  const bool pos = p.inv != nullptr;
  const int64_t rc = valid ? row : p.rows - 1;
  const int64_t T = p.rows / p.H;
  const int64_t sl = rc / p.H;
  const f32x4 d0 = *(const f32x4*)(p.dy[which] + rc * HD + 8 * c);
  const f32x4 d1 = *(const f32x4*)(p.dy[which] + rc * HD + 8 * c + 4);
  const u32x4 wv = *(const u32x4*)(p.w[which] + 8 * c);
  const int sg = p.tok2seg[sl];
  int64_t tok = sl;  // the token of the staged row
  if (pos) {
    const int64_t t = p.inv[sl];
    tok = t >= 0 && t < T ? t : sl;
  }
  const int nseg = p.hdr->nseg;
  const bool sg_ok = sg >= 0 && sg < nseg;
  const bool bad = valid && sg_ok && p.segflag[sg_ok ? sg : 0] != 0;
  const int64_t xt = tok * p.H + (rc - sl * p.H);  // the token's row
  const u32x4 xv = *(const u32x4*)(p.x[which] + xt * HD + 8 * c);
  const int64_t xrow = bad ? row : xt;  // where dx goes

  float x[8], wf[8];
  double dy[8];  // the gradient with respect to the norm's output (through the rope when given)
  {
    unpack8_bf16(xv, x);
    unpack8_bf16(wv, wf);
#pragma unroll
    for (int i = 0; i < 4; i++) dy[i] = (double)d0[i], dy[4 + i] = (double)d1[i];
    if (p.rope_cos && c < ROPE_CHUNKS) {
      const f32x4 cs = *(const f32x4*)(p.rope_cos + tok * ROPE_PAIRS + 4 * c);
      const f32x4 sn = *(const f32x4*)(p.rope_sin + tok * ROPE_PAIRS + 4 * c);
      rope_chunk_transpose(dy, cs, sn);
    }
  }
  const double r = norm_rscale(row_total_16lanes(chunk_sumsq(x)), p.eps);
  double gx = 0.0;
#pragma unroll
  for (int i = 0; i < 8; i++) gx = __builtin_fma((double)wf[i] * dy[i], (double)x[i], gx);
  gx = gx + __shfl_xor(gx, 1, 64);
  gx = gx + __shfl_xor(gx, 2, 64);
  gx = gx + __shfl_xor(gx, 4, 64);
  gx = gx + __shfl_xor(gx, 8, 64);
  const double k3 = r * r * r * 0.0078125 * gx;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    o[i] = f64x2_to_bf16x2_rne(r * ((double)wf[2 * i] * dy[2 * i]) - k3 * (double)x[2 * i],
                               r * ((double)wf[2 * i + 1] * dy[2 * i + 1]) - k3 * (double)x[2 * i + 1]);
  }
  if (bad) o = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  if (valid) *(u32x4*)(p.dx[which] + xrow * HD + 8 * c) = o;
  f32x4 t0, t1;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    t0[i] = valid ? (float)(dy[i] * (double)x[i] * r) : 0.0f;
    t1[i] = valid ? (float)(dy[4 + i] * (double)x[4 + i] * r) : 0.0f;
  }
  *(f32x4*)&red[tid >> 4][8 * c] = t0;
  *(f32x4*)&red[tid >> 4][8 * c + 4] = t1;
  __syncthreads();
  if (tid < HD) {
    float s = 0.0f;
#pragma unroll
    for (int rr = 0; rr < NR; rr++) s += red[rr][tid];
    p.part[((int64_t)which * p.nparts + blockIdx.x) * HD + tid] = s;
  }
}

// dw = the workgroup partials summed in a fixed tree whose shape depends only on their number:
// each chunk of DW_CHUNK consecutive partials as its two halves, each summed in order, then added;
// the chunks as eight consecutive runs, each summed in order, then added pairwise.  Several
// independent loads are kept in flight per thread (the sums themselves stay sequential).

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

// blockIdx.y: 0 = q, 1 = k; thread = (half, channel).
__global__ __launch_bounds__(2 * HD) void k_bwd_dw_chunks(const WsHeader* hdr, const float* part, int64_t nparts,
                                                          int64_t nchunks, float* chunk_part) {
  __shared__ float upper[HD];
  const int d = threadIdx.x & (HD - 1), g = threadIdx.x >> 7, which = blockIdx.y;
  if (hdr->status != 0) return;
  for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const int64_t i0 = ch * DW_CHUNK, cnt = min((int64_t)DW_CHUNK, nparts - i0);
    const int64_t lo = min(cnt, (int64_t)(DW_CHUNK / 2));
    const float* b = part + ((int64_t)which * nparts + i0) * HD + d;
    const float sh = g == 0 ? sum_strided(b, lo, HD) : sum_strided(b + lo * HD, cnt - lo, HD);
    if (g == 1) upper[d] = sh;
    __syncthreads();
    if (g == 0) chunk_part[((int64_t)which * nchunks + ch) * HD + d] = sh + upper[d];
    __syncthreads();
  }
}

// With a recorded data error the weights' gradients are NaN like the other outputs.  blockIdx.x:
// 0 = q, 1 = k; thread = (run, channel).
constexpr int DW_RUNS = 8;
__global__ __launch_bounds__(DW_RUNS * HD) void k_bwd_dw_final(const WsHeader* hdr, const float* chunk_part,
                                                               int64_t nchunks, float* dwq, float* dwk) {
  __shared__ float run[DW_RUNS][HD];
  const int d = threadIdx.x & (HD - 1), g = threadIdx.x >> 7, which = blockIdx.x;
  float* out = which ? dwk : dwq;
  if (hdr->status != 0) {
    if (g == 0) out[d] = __builtin_nanf("");
    return;
  }
  const int64_t per = (nchunks + DW_RUNS - 1) / DW_RUNS;
  const int64_t c0 = min(nchunks, g * per), c1 = min(nchunks, c0 + per);
  run[g][d] = sum_strided(chunk_part + ((int64_t)which * nchunks + c0) * HD + d, c1 - c0, HD);
  __syncthreads();
  static_assert(DW_RUNS == 8, "the pairwise tree below");
  if (g == 0)
    out[d] = ((run[0][d] + run[1][d]) + (run[2][d] + run[3][d])) + ((run[4][d] + run[5][d]) + (run[6][d] + run[7][d]));
}

hipError_t launch_bwd(const void* q, const void* k, const void* wq, const void* wk, int64_t T, int32_t H, float eps,
                      float scale, void* dq, void* dk, void* dv, float* dwq, float* dwk, void* ws,
                      const int32_t* inv, bool delta_ready, const float* rope_cos, const float* rope_sin,
                      int grid_cap, hipStream_t stream) {
  const BwdLayout Lw = bwd_layout(T, H);
  char* base = (char*)ws;
  BwdParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.wq = (const uint16_t*)wq;
  p.wk = (const uint16_t*)wk;
  p.qhat16 = (const uint16_t*)(base + Lw.qhat16);
  p.khat16 = (const uint16_t*)(base + Lw.khat16);
  p.v16 = (const uint16_t*)(base + Lw.v16);
  p.do16 = (const uint16_t*)(base + Lw.do16);
  p.lse2 = (const float*)(base + Lw.lse2);
  p.delta = (float*)(base + Lw.delta);
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.dqh = (float*)(base + Lw.dqh);
  p.dkh = (float*)(base + Lw.dkh);
  p.inv = inv;
  p.dmax = (const uint32_t*)(base + Lw.dmax);
  p.segflag = (const int32_t*)(base + Lw.segflag);
  p.delta_ready = delta_ready ? 1 : 0;
  p.hdr = (const WsHeader*)base;
  p.segtab = (const int32_t*)(base + Lw.segtab);
  p.items = (const int32_t*)(base + Lw.items);
  p.bkt = (const int32_t*)(base + Lw.bkt);
  p.T = T;
  p.H = H;
  p.eps = eps;
  p.scale = scale;
  p.c = (float)((double)scale * 1.4426950408889634074);
  const int64_t max_work = Lw.max_items * H;
  int64_t grid = grid_cap < max_work ? grid_cap : max_work;
  grid = (grid + 7) & ~(int64_t)7;
  p.next = &((WsHeader*)base)->next[0];
  // grid_cap is the CU count: dq runs two workgroups per CU, dk/dv one
  hipLaunchKernelGGL(k_bwd_dq, dim3((unsigned)(2 * grid)), dim3(64 * BW), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.next = &((WsHeader*)base)->next[1];
  hipLaunchKernelGGL(k_bwd_dkdv, dim3((unsigned)grid), dim3(64 * BWK), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (wq) {
    NormBwdParams np;
    np.x[0] = (const uint16_t*)q;
    np.x[1] = (const uint16_t*)k;
    np.w[0] = (const uint16_t*)wq;
    np.w[1] = (const uint16_t*)wk;
    np.dy[0] = p.dqh;
    np.dy[1] = p.dkh;
    np.dx[0] = (uint16_t*)dq;
    np.dx[1] = (uint16_t*)dk;
    np.part = (float*)(base + Lw.dw_part);
    np.inv = inv;
    np.tok2seg = (const int32_t*)(base + Lw.tok2seg);
    np.segflag = (const int32_t*)(base + Lw.segflag);
    np.rope_cos = rope_cos;
    np.rope_sin = rope_sin;
    np.hdr = (const WsHeader*)base;
    np.rows = T * H;
    np.H = H;
    np.nparts = Lw.nparts;
    np.eps = eps;
    hipLaunchKernelGGL(k_bwd_norm, dim3((unsigned)Lw.nparts, 2), dim3(256), 0, stream, np);
    float* chunk_part = (float*)(base + Lw.dw_chunk);
    const unsigned g2 = (unsigned)(Lw.nchunks < 1024 ? Lw.nchunks : 1024);
    hipLaunchKernelGGL(k_bwd_dw_chunks, dim3(g2, 2), dim3(2 * HD), 0, stream, (const WsHeader*)base, np.part,
                       Lw.nparts, Lw.nchunks, chunk_part);
    hipLaunchKernelGGL(k_bwd_dw_final, dim3(2), dim3(DW_RUNS * HD), 0, stream, (const WsHeader*)base, chunk_part,
                       Lw.nchunks, dwq, dwk);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace h3
