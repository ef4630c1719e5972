// Forward attention of the H3 node: non-causal softmax attention inside each packed segment
// ("ws1_one_h3_block" page, Bindings table: attention with causal=False over packed layouts), with
// the q RMSNorm fused into the Q load prologue, FP32 accumulation and one bf16 rounding of the
// output ("33B forward/backward" page, Scope: strict mode).
//
// Work item = (segment, 128-query tile, head); a persistent grid walks the items.  Each wave owns 32
// queries.  The products are computed transposed so that one lane pair owns one query:
//   S^T[key][query] = Khat . Qhat^T   (A = 32 keys x 16 dims from LDS, B = the wave's normed Q held
//                                      in registers; v_mfma_f32_32x32x16_bf16)
//   O^T[dim][query] += V^T . P^T      (A = 32 dims x 16 keys, read from the row-major V tile with
//                                      ds_read_b64_tr_b16; B = P in fp16; v_mfma_f32_32x32x16_f16)
// With that layout the softmax row max and row sum are lane-local over 32 scores plus one exchange
// with lane ^ 32 (the other half of the query's keys), done with v_permlane32_swap.
//
// Pipeline.  K and V tiles (64 keys, 16 KB each) are copied from the workspace straight into LDS
// with global_load_lds_dwordx4 (no register staging), double-buffered: at the top of iteration j
// the loads of K(j+2) and V(j+1) are issued, and they have the whole iteration to land.  Within a
// wave, iteration j overlaps the S MFMAs of tile j+1 with the softmax of tile j, then the P.V MFMAs
// of tile j with the row maximum of tile j+1.  One barrier per iteration.
//
// LDS layouts are XOR-swizzled by 16-byte chunk (the copy picks, per lane, which global chunk
// lands in its LDS slot), so that both read patterns are free of bank conflicts:
//   K: row r, chunk c at slot c ^ (r & 15)        (ds_read_b128 of 32 rows x 16 B)
//   V: row r, chunk c at slot c ^ 4 * (r & 3)     (ds_read_b64_tr_b16 of 8 rows x 64 B)
//
// Determinism and batch invariance: tiles are anchored at the segment's first key and walked in
// ascending order; keys past the segment end are masked to -inf by a select (their K rows are
// in-segment duplicates, their V rows likewise and they meet p = 0); every sum is a fixed tree; the
// code path depends only on the segment length.  So each output row is a function of its own
// segment's bytes, never of the batch, the offset, neighbours or the grid.  (Maxima are exact, so
// their evaluation order cannot change a bit.)
//
// Online softmax with a lazy maximum: the running maximum m (log2 units) moves only when a tile's
// maximum exceeds it by more than 8, so p = exp2(s*c - m) <= 2^8 stays well inside fp16, and the
// O/l rescale is skipped on most tiles.  Lanes whose m does not move take alpha = 1 exactly.
#include "h3_common.h"
#include "h3_launch.h"

namespace h3 {

constexpr float LN2 = 0.69314718055994530942f;
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units
constexpr int TILE_ELEMS = BK * HD;        // 16-bit elements in one K or V tile (16 KB)

struct AttnParams {
  const uint16_t* q;
  const uint16_t* wq;
  const uint16_t* khat;
  const uint16_t* v16;
  uint16_t* out;
  float* lse;
  const WsHeader* hdr;
  const int32_t* segtab;
  const int32_t* items;
  int64_t T;
  int32_t H;
  float eps;
  float c;  // scale * log2(e)
  int32_t xcd_slots;  // workgroups per XCD (grid / 8), for the XCD-aware item order
};

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Element offsets of a 16-bit value (row r, column d) inside a swizzled tile.
__device__ __forceinline__ int k_off(int r, int d) { return r * HD + ((((d >> 3) ^ (r & 15))) << 3) + (d & 7); }
__device__ __forceinline__ int v_off(int r, int d) { return r * HD + ((((d >> 3) ^ ((r & 3) << 2))) << 3) + (d & 7); }

// Copy one 64-row tile of a head-major [rows][128] 16-bit array into a swizzled LDS tile with
// buffer_load_dwordx4 ... lds.  The buffer resource covers only the tile's rows inside the segment
// (`valid` rows), so the rows past the segment end read as zeros: nothing outside the segment can
// reach the products.  256 threads, 4 x 1 KB per wave; each lane's 16 bytes land at LDS base +
// lane * 16, so the lane fetches the global chunk that belongs in that slot.  The slot pattern
// repeats every 16 rows, so one lane offset serves all four blocks.
__device__ __forceinline__ int tile_lane_offset(bool is_v, int wv, int lane) {
  const int r = 4 * wv + (lane >> 4);  // tile row of the lane's slot in block wv (rows 4wv..4wv+3)
  const int slot = lane & 15;
  const int c = is_v ? (slot ^ ((r & 3) << 2)) : (slot ^ (r & 15));
  return r * 256 + c * 16;  // bytes
}

__device__ __forceinline__ void tile_to_lds(const uint16_t* gtile, int valid, uint16_t* lds_tile, int wv,
                                            int lane_off) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)gtile, (short)0, (valid < BK ? valid : BK) * 256, 0x00020000);
#pragma unroll
  for (int i = 0; i < 4; i++)  // block 4i + wv = rows 16i + 4wv .. +3
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_tile + (4 * i + wv) * 4 * HD), 16,
                                             lane_off + i * 4096, 0, 0, 0);
}

// Transposed LDS read (gfx950): within each 16-lane group, lane s supplies the address of 4
// consecutive 16-bit elements C_s; lane s receives {C_{s/4}[s%4], C_{4+s/4}[s%4], C_{8+s/4}[s%4],
// C_{12+s/4}[s%4]}.  With C_s = V[key0 + s/4][dim0 + 4(s%4) .. +3] lane s gets V[key0 + i][dim0 + s],
// i = 0..3: four consecutive keys of one dim, the A-operand layout of a P.V MFMA.
__device__ __forceinline__ i16x4 tr_read(const uint16_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uint16_t*)lds_ptr);
}

// The value of lane ^ 32 (the other half of this query's keys), exchanged without LDS.
__device__ __forceinline__ void swap_halves(float x, float& lo_half, float& hi_half) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  // r[0]: lanes 0-31 keep x, lanes 32-63 receive x of lanes 0-31; r[1]: the other way round.  So
  // every lane holds (x of lane l%32, x of lane l%32 + 32), in that order, in both halves.
  lo_half = __builtin_bit_cast(float, (uint32_t)r[0]);
  hi_half = __builtin_bit_cast(float, (uint32_t)r[1]);
}

template <int N>
__device__ __forceinline__ float tree_sum(const float* x) {
  if constexpr (N == 1) {
    return x[0];
  } else {
    return tree_sum<N / 2>(x) + tree_sum<N / 2>(x + N / 2);
  }
}

// S^T for the 64 keys of one LDS tile: S[kb] holds keys 32kb + 8(i/4) + 4hh + (i%4) of the lane's
// query.  The k-slices are accumulated in ascending dimension order.
__device__ __forceinline__ void tile_scores(const uint16_t* Ks, const bf16x8* qf, int l32, int hh, f32x16* S) {
#pragma unroll
  for (int kb = 0; kb < 2; kb++) {
#pragma unroll
    for (int i = 0; i < 16; i++) S[kb][i] = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; m++) {
      const bf16x8 a = *(const bf16x8*)(Ks + k_off(32 * kb + l32, 16 * m + 8 * hh));
      S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[m], S[kb], 0, 0, 0);
    }
  }
}

// Keys at or past `rem` (the valid keys of the segment's last tile) get -inf.
__device__ __forceinline__ void mask_tail(f32x16* S, int rem, int hh) {
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++)
      if (32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3) >= rem) S[kb][i] = -__builtin_inff();
}

// Maximum over the query's 64 keys of one tile (exact, so any evaluation order gives these bits).
__device__ __forceinline__ float tile_max(const f32x16* S) {
  float a = __builtin_fmaxf(__builtin_fmaxf(S[0][0], S[0][1]), S[0][2]);
  float b = __builtin_fmaxf(__builtin_fmaxf(S[1][0], S[1][1]), S[1][2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) {
    a = __builtin_fmaxf(__builtin_fmaxf(a, S[0][i]), S[0][i + 1]);
    b = __builtin_fmaxf(__builtin_fmaxf(b, S[1][i]), S[1][i + 1]);
  }
  a = __builtin_fmaxf(a, S[0][15]);
  b = __builtin_fmaxf(b, S[1][15]);
  float lo, hi;
  swap_halves(__builtin_fmaxf(a, b), lo, hi);
  return __builtin_fmaxf(lo, hi);
}

template <int N>
struct Par {
  static constexpr int value = N;
};

// Modes of one KV iteration j (tile j's softmax and P.V, tile j+1's scores):
//   FULL  j + 2 < ntiles: tile j+1 is a full tile, K(j+2) and V(j+1) are prefetched
//   MASK  j + 2 == ntiles: tile j+1 is the segment's last tile (masked past `rem`), V(j+1) prefetched
//   LAST  j + 1 == ntiles: no next tile
enum Mode { FULL = 0, MASK = 1, LAST = 2 };

__global__ __launch_bounds__(256, 2) void k_attn_fwd(AttnParams p) {
  // K tiles in buffers 0, 1 and V tiles in buffers 2, 3 (16 KB each)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hh = lane >> 5;    // which half of the 16-wide MFMA k-slice this lane feeds
  const int l32 = lane & 31;   // query (B / D column) index within the wave
  const int64_t T = p.T;
  const int H = p.H;

  if (p.hdr->status != 0) {
    // A data error was recorded: make the result unmistakably invalid.
    const int64_t n16 = T * H * HD / 8;
    const u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    for (int64_t e = (int64_t)blockIdx.x * 256 + tid; e < n16; e += (int64_t)gridDim.x * 256)
      *(u32x4*)(p.out + e * 8) = nan4;
    if (p.lse)
      for (int64_t e = (int64_t)blockIdx.x * 256 + tid; e < T * H; e += (int64_t)gridDim.x * 256)
        p.lse[e] = __builtin_nanf("");
    return;
  }

  // Counts come from the plan kernel; clamp them so that even a workspace that was never planned
  // cannot send a work item outside the tensors.
  const int64_t max_items = T + (T + BQ - 1) / BQ;
  const int nseg = (int)min((int64_t)max(p.hdr->nseg, 0), T);
  const int nitems = (int)min((int64_t)max(p.hdr->nitems, 0), max_items);
  const int nwork = nitems * H;

  // XCD-aware order: workgroup b runs on XCD b % 8; the workgroups of one XCD take consecutive
  // positions of the head-major work order, so they share the K/V tiles of one head in that XCD's L2.
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int nslots = p.xcd_slots;

  const int k_lane_off = tile_lane_offset(false, wv, lane);
  const int v_lane_off = tile_lane_offset(true, wv, lane);
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const float c = p.c;

  for (int round = 0;; round++) {
    const int64_t v = ((int64_t)round * 8 + xcd) * nslots + slot;
    if (v >= nwork) break;
    const int head = (int)(v / nitems);
    const int item = (int)(v - (int64_t)head * nitems);
    const int seg = p.items[2 * item];
    const int qt = p.items[2 * item + 1];
    if ((unsigned)seg >= (unsigned)nseg) continue;
    const int s0 = p.segtab[2 * seg];
    const int L = p.segtab[2 * seg + 1];
    if (s0 < 0 || L <= 0 || (int64_t)s0 + L > T || qt < 0 || qt * BQ >= L) continue;

    const int ntiles = (L + BK - 1) / BK;
    const int rem = L - (ntiles - 1) * BK;  // valid keys of the last tile, 1..64
    const uint16_t* kbase = p.khat + ((int64_t)head * T + s0) * HD;
    const uint16_t* vbase = p.v16 + ((int64_t)head * T + s0) * HD;

    // Every wave has finished reading LDS for the previous item before it is overwritten.
    __syncthreads();
    tile_to_lds(kbase, L, lds, wv, k_lane_off);
    tile_to_lds(vbase, L, lds + 2 * TILE_ELEMS, wv, v_lane_off);
    if (ntiles > 1) tile_to_lds(kbase + BK * HD, L - BK, lds + TILE_ELEMS, wv, k_lane_off);

    // ---------------- Q prologue: load, RMSNorm (2 lanes per row), round to bf16 B-operands
    const int qrow = qt * BQ + wv * 32 + l32;
    const bool qvalid = qrow < L;
    bf16x8 qf[8];
    {
      float x[8][8];
      const uint16_t* qp = p.q + ((int64_t)(s0 + (qvalid ? qrow : 0)) * H + head) * HD;
#pragma unroll
      for (int m = 0; m < 8; m++) {
        u32x4 w4 = {0, 0, 0, 0};
        if (qvalid) w4 = *(const u32x4*)(qp + 16 * m + 8 * hh);
        unpack8_bf16(w4, x[m]);
      }
      if (p.wq) {
        double part[8];
#pragma unroll
        for (int m = 0; m < 8; m++) part[m] = chunk_sumsq(x[m]);
        const double r = norm_rscale(row_total_2lanes(part), p.eps);
#pragma unroll
        for (int m = 0; m < 8; m++) {
          float wf[8];
          unpack8_bf16(*(const u32x4*)(p.wq + 16 * m + 8 * hh), wf);
          const u32x4 o = norm_chunk(x[m], wf, r);
          qf[m] = __builtin_bit_cast(bf16x8, o);
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; m++) {
          u32x4 o;
#pragma unroll
          for (int i = 0; i < 4; i++) o[i] = pack_bf16(x[m][2 * i], x[m][2 * i + 1]);
          qf[m] = __builtin_bit_cast(bf16x8, o);
        }
      }
      if (!qvalid) {
#pragma unroll
        for (int m = 0; m < 8; m++) qf[m] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      }
    }

    // ---------------- scores of tile 0
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's tile copies have landed
    __syncthreads();                    // ... and every other wave's
    f32x16 S[2];
    tile_scores(lds, qf, l32, hh, S);
    if (ntiles == 1 && rem < BK) mask_tail(S, rem, hh);

    f32x16 O[4];
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int i = 0; i < 16; i++) O[d][i] = 0.0f;
    float lsum = 0.0f;
    float m_run = tile_max(S) * c;  // first tile: m is the tile maximum (log2 units)

    // One KV iteration; PAR = j & 1 selects the buffers: K(j) and V(j) live in buffers PAR and 2+PAR.
    auto iteration = [&](auto par, auto mode, int j) {
      constexpr int PAR = decltype(par)::value;
      constexpr int MODE = decltype(mode)::value;
      uint16_t* const Kcur = lds + PAR * TILE_ELEMS;         // K(j): free once the iteration starts
      const uint16_t* const Knext = lds + (1 - PAR) * TILE_ELEMS;  // K(j+1)
      const uint16_t* const Vcur = lds + (2 + PAR) * TILE_ELEMS;   // V(j)
      uint16_t* const Vnext = lds + (3 - PAR) * TILE_ELEMS;        // V(j+1): its buffer held V(j-1)
      __builtin_amdgcn_s_waitcnt(0xF70);
      __syncthreads();
      if constexpr (MODE == FULL) tile_to_lds(kbase + (int64_t)(j + 2) * BK * HD, L - (j + 2) * BK, Kcur, wv, k_lane_off);
      if constexpr (MODE != LAST) tile_to_lds(vbase + (int64_t)(j + 1) * BK * HD, L - (j + 1) * BK, Vnext, wv, v_lane_off);

      // scores of tile j+1 (MFMA) alongside the softmax of tile j (VALU)
      f32x16 Sn[2];
      if constexpr (MODE != LAST) tile_scores(Knext, qf, l32, hh, Sn);

      float pr[32];
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) pr[16 * kb + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][i], c, -m_run));
      lsum += tree_sum<32>(pr);
      f16x8 pf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        u32x4 w4;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const f32x2 two = {pr[8 * ks + 2 * i], pr[8 * ks + 2 * i + 1]};
          w4[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(two, f16x2));  // RNE
        }
        pf[ks] = __builtin_bit_cast(f16x8, w4);
      }

      // O^T += V^T P^T ; A rows = dims 32db + l32, A k-slots = keys 16ks + {4hh..4hh+3, 8+4hh..8+4hh+3}
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const i16x4 lo = tr_read(Vcur + v_off(16 * ks + tr_row, 32 * db + tr_col));
          const i16x4 hi = tr_read(Vcur + v_off(16 * ks + 8 + tr_row, 32 * db + tr_col));
          const f16x4 flo = __builtin_bit_cast(f16x4, lo), fhi = __builtin_bit_cast(f16x4, hi);
          const f16x8 a = {flo[0], flo[1], flo[2], flo[3], fhi[0], fhi[1], fhi[2], fhi[3]};
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], O[db], 0, 0, 0);
        }
      }

      if constexpr (MODE != LAST) {
        if constexpr (MODE == MASK) {
          if (rem < BK) mask_tail(Sn, rem, hh);
        }
        const float mt = tile_max(Sn) * c;
        const bool need = mt > m_run + RESCALE_THRESHOLD;
        if (__builtin_expect(__ballot(need) != 0, 0)) {  // rare: keep it a branch, not a select
          const float m_new = need ? mt : m_run;
          const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
          lsum *= alpha;
#pragma unroll
          for (int d = 0; d < 4; d++)
#pragma unroll
            for (int i = 0; i < 16; i++) O[d][i] *= alpha;
          m_run = m_new;
        }
        S[0] = Sn[0];
        S[1] = Sn[1];
      }
    };

    // j = 0 .. ntiles-3 in FULL mode (unrolled by two so the buffers are fixed), then MASK, LAST
    int j = 0;
    for (; j + 3 < ntiles; j += 2) {
      iteration(Par<0>{}, Par<FULL>{}, j);
      iteration(Par<1>{}, Par<FULL>{}, j + 1);
    }
    if (j + 2 < ntiles) {
      iteration(Par<0>{}, Par<FULL>{}, j);
      j++;
    }
    // now j == ntiles - 2 (or ntiles == 1 and j == 0)
    if (j + 2 == ntiles) {
      if (j & 1) iteration(Par<1>{}, Par<MASK>{}, j);
      else iteration(Par<0>{}, Par<MASK>{}, j);
      j++;
    }
    if (j & 1) iteration(Par<1>{}, Par<LAST>{}, j);
    else iteration(Par<0>{}, Par<LAST>{}, j);

    // ---------------- epilogue: one division per row, one bf16 rounding per element
    float l_lo, l_hi;
    swap_halves(lsum, l_lo, l_hi);
    const float l = l_lo + l_hi;
    const float inv = __fdiv_rn(1.0f, l);
    if (qvalid) {
      uint16_t* op = p.out + ((int64_t)(s0 + qrow) * H + head) * HD;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const int d0 = 32 * db + 8 * g + 4 * hh;
          u32x2 o2;
          o2[0] = pack_bf16(O[db][4 * g] * inv, O[db][4 * g + 1] * inv);
          o2[1] = pack_bf16(O[db][4 * g + 2] * inv, O[db][4 * g + 3] * inv);
          *(u32x2*)(op + d0) = o2;
        }
      if (p.lse && hh == 0) p.lse[(int64_t)(s0 + qrow) * H + head] = (m_run + __builtin_amdgcn_logf(l)) * LN2;
    }
  }
}

hipError_t launch_attend(const void* q, const void* wq, int64_t T, int32_t H, float eps, float scale, void* out,
                         float* lse, void* ws, int grid_cap, hipStream_t stream) {
  const WsLayout Lw = ws_layout(T, H);
  char* base = (char*)ws;
  AttnParams p;
  p.q = (const uint16_t*)q;
  p.wq = (const uint16_t*)wq;
  p.khat = (const uint16_t*)(base + Lw.khat);
  p.v16 = (const uint16_t*)(base + Lw.v16);
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.hdr = (const WsHeader*)base;
  p.segtab = (const int32_t*)(base + Lw.segtab);
  p.items = (const int32_t*)(base + Lw.items);
  p.T = T;
  p.H = H;
  p.eps = eps;
  p.c = (float)((double)scale * 1.4426950408889634074);
  // a multiple of 8 workgroups (one slot per XCD each), at most grid_cap and no more than the work
  const int64_t max_work = Lw.max_items * H;
  int64_t grid = grid_cap < max_work ? grid_cap : max_work;
  grid = (grid + 7) & ~(int64_t)7;
  p.xcd_slots = (int32_t)(grid / 8);
  hipLaunchKernelGGL(k_attn_fwd, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace h3
