// Forward attention of the H3 node: non-causal softmax attention inside each packed segment
// ("ws1_one_h3_block" page, Bindings table: attention with causal=False over packed layouts) on the
// normed Q and K that the staging kernel wrote, FP32 accumulation and one bf16 rounding of the
// output ("33B forward/backward" page, Scope: strict mode).
//
// Work item = (segment, 256-query tile, head); a persistent grid of one workgroup per CU walks the
// items, each XCD its own eighth of them (a sparse last round runs as 128-query halves, see the
// work order in the kernel).  The workgroup has 8 waves of 32 queries; waves w and w + 4 share a
// SIMD.  The products
// are computed transposed so that one lane pair owns one query:
//   S^T[key][query] = Khat . Qhat^T   (A = 32 keys x 16 dims from LDS, B = the wave's normed Q held
//                                      in registers; v_mfma_f32_32x32x16_bf16)
//   O^T[dim][query] += V^T . P^T      (A = 32 dims x 16 keys, read from the row-major V tile with
//                                      ds_read_b64_tr_b16; B = P in fp16; v_mfma_f32_32x32x16_f16)
// A KV tile is 96 keys: three 32-key blocks.  The softmax row sums (and, when needed, row maxima)
// are lane-local over the lane's 48 scores of a tile (16 of each block); the two halves of a
// query's keys (lanes l and l ^ 32) meet through v_permlane32_swap.
//
// Ping-pong.  The KV walk of a wave alternates two kinds of phase: a matrix phase G(k) (the 24
// score MFMAs of tile k+1 and the 24 P.V MFMAs of tile k, operands read from LDS a few MFMAs
// ahead) and a vector phase V(k) (the softmax of tile k+1: exp, sum, fp16 packing, and the rare
// rescale).  Waves 4..7 run one phase behind waves 0..3, and every phase ends at a workgroup
// barrier, so on each SIMD one wave issues MFMAs back to back while its partner does the vector
// work: the matrix cores stay busy and the softmax is hidden behind them.
//
// K and V tiles (96 keys, 24 KB each) are copied from the workspace straight into LDS with
// buffer_load_dwordx4 ... lds (no register staging), double-buffered.  Copies are issued only in
// vector phases, a quarter of a tile per wave: K(m+1) at the start of phase slot 2m by the
// trailing waves (two slots to land) and V(m) at the start of slot 2m+1 by the leading waves (one
// slot to land).  The phase barriers carry no memory fence; each wave waits for its own copies
// only before slot 2m+2, where both are first read.
//
// LDS layouts are XOR-swizzled by 16-byte chunk (the copy picks, per lane, which global chunk
// lands in its LDS slot), so that both read patterns are free of bank conflicts:
//   K: row r, chunk c at slot c ^ (r & 15)        (ds_read_b128 of 32 rows x 16 B)
//   V: row r, chunk c at slot c ^ 4 * (r & 3)     (ds_read_b64_tr_b16 of 8 rows x 64 B)
//
// Determinism and batch invariance: tiles are anchored at the segment's first key and walked in
// ascending order; rows past the segment end are zero in LDS and their scores are replaced by -inf;
// every sum is a fixed tree; the code path depends only on the segment length.  So each output row
// is a function of its own segment's bytes, never of the batch, the offset, neighbours or the grid.
// (Maxima are exact, so their evaluation order cannot change a bit.)
//
// Online softmax with a lazy maximum, checked after the fact: p = exp2(s*c - m) is formed with the
// running maximum m (log2 units) as it stands, and m moves only when the row's p over one tile no
// longer fit: when a lane's 48 values sum past 4096 (or to infinity or NaN, as on the first tile,
// where m starts at -inf).  Then the tile's maximum is taken, O and l are rescaled, and the tile's
// p are formed again; until then every p is at most 4096, well inside fp16, and the common path
// needs no maximum at all.  The decision is the row's own (both halves of the query's keys), and
// rows whose m does not move take alpha = 1 exactly and re-form the same p, so a row's bits never
// depend on its neighbours in the wave.
#include "h3_common.h"
#include "h3_launch.h"
#include "h3_tiles.h"

namespace h3 {

constexpr float LN2 = 0.69314718055994530942f;
constexpr float P_SUM_LIMIT = 4096.0f;     // a lane's 48 p values of one tile sum to at most this
constexpr int NWAVES = 8;                 // waves per workgroup (two per SIMD)
constexpr int FROWS = BK;          // keys per KV tile
static_assert(FROWS % 32 == 0, "whole 32-key blocks");
constexpr int NKB = FROWS / 32;    // 32-key blocks per tile
constexpr int NKS = FROWS / 16;    // 16-key slices per tile
constexpr int FTILE = FROWS * HD;  // 16-bit elements per LDS tile

template <int NW>
__device__ __forceinline__ void ftile_to_lds_o(const uint16_t* gtile, int valid, uint16_t* lds_tile, int wv,
                                               const int* offs) {
  static_assert(FROWS % (4 * NW) == 0, "whole 1 KB blocks per wave");
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)gtile, (short)0, (valid < FROWS ? valid : FROWS) * 256, 0x00020000);
  int wofs = wv * 4 * HD;
  asm volatile("" : "+s"(wofs));
#pragma unroll
  for (int i = 0; i < FROWS / (4 * NW); i++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_tile + NW * i * 4 * HD + wofs), 16, offs[i], 0, 0, 0);
}

template <int NW>
__device__ __forceinline__ void ftile_to_lds(const uint16_t* gtile, int valid, uint16_t* lds_tile, int wv,
                                             int lane_off) {
  static_assert(FROWS % (4 * NW) == 0, "whole 1 KB blocks per wave");
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)gtile, (short)0, (valid < FROWS ? valid : FROWS) * 256, 0x00020000);
  int wofs = wv * 4 * HD;
  asm volatile("" : "+s"(wofs));
#pragma unroll
  for (int i = 0; i < FROWS / (4 * NW); i++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_tile + NW * i * 4 * HD + wofs), 16,
                                             lane_off + i * NW * 1024, 0, 0, 0);
}

template <int NPRE>
__device__ __forceinline__ void fscores(const uint16_t* Kb, const bf16x8* qf, int l32, int hh, f32x16* S) {
  constexpr int NS = 8 * NKB;
  bf16x8 ka[NS];
  auto kread = [&](int s) {
    const int kb = s % NKB, m = s / NKB;
    ka[s] = *(const bf16x8*)(Kb + k_off(32 * kb + l32, 16 * m + 8 * hh));
  };
#pragma unroll
  for (int kb = 0; kb < NKB; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++) S[kb][i] = 0.0f;
#pragma unroll
  for (int s = 0; s < NPRE; s++) kread(s);
#pragma unroll
  for (int s = 0; s < NS; s++) {  // step s = NKB m + kb
    if (s + NPRE < NS) kread(s + NPRE);
    S[s % NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qf[s / NKB], S[s % NKB], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// P.V over the tile's NKS 16-key slices, V buffer VB (vb: the lane's addresses in V buffer 0)
template <int VB, int T>
__device__ __forceinline__ void ftr_read_step(const uint32_t* vb, u32x2 (&va)[4 * NKS][2]) {
  constexpr int ks = T >> 2, db = T & 3;
  constexpr int off = VB * FTILE * 2 + 16 * ks * HD * 2;
  va[T][0] = tr_read_asm<off>(vb[db]);
  va[T][1] = tr_read_asm<off + 8 * HD * 2>(vb[db]);
}
template <int VB, int T>
__device__ __forceinline__ void ftr_gemm_step(const uint32_t* vb, const f16x8* pf, f32x16* O, u32x2 (&va)[4 * NKS][2]) {
  constexpr int NT = 4 * NKS;
  if constexpr (T + 4 < NT) ftr_read_step<VB, T + 4>(vb, va);
  constexpr int ahead = (T + 4 < NT ? T + 4 : NT - 1) - T;
  if constexpr (ahead == 4) LGKM_WAIT_TIED(8, va[T][0], va[T][1]);
  else if constexpr (ahead == 3) LGKM_WAIT_TIED(6, va[T][0], va[T][1]);
  else if constexpr (ahead == 2) LGKM_WAIT_TIED(4, va[T][0], va[T][1]);
  else if constexpr (ahead == 1) LGKM_WAIT_TIED(2, va[T][0], va[T][1]);
  else LGKM_WAIT_TIED(0, va[T][0], va[T][1]);
  const f16x4 lo = __builtin_bit_cast(f16x4, va[T][0]), hi = __builtin_bit_cast(f16x4, va[T][1]);
  const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  O[T & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[T >> 2], O[T & 3], 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (T + 1 < NT) ftr_gemm_step<VB, T + 1>(vb, pf, O, va);
}
template <int VB>
__device__ __forceinline__ void ftr_gemm(const uint32_t* vb, const f16x8* pf, f32x16* O) {
  u32x2 va[4 * NKS][2];
  ftr_read_step<VB, 0>(vb, va);
  ftr_read_step<VB, 1>(vb, va);
  ftr_read_step<VB, 2>(vb, va);
  ftr_read_step<VB, 3>(vb, va);
  ftr_gemm_step<VB, 0>(vb, pf, O, va);
}

__device__ __forceinline__ void fmask_tail_rel(f32x16* S, int rel) {
#pragma unroll
  for (int kb = 0; kb < NKB; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++)
      if (32 * kb + 8 * (i >> 2) + (i & 3) >= rel) S[kb][i] = -__builtin_inff();
}
static_assert(BQ == 32 * NWAVES, "one 32-query block per wave");

struct AttnParams {
  const uint16_t* q;  // normed Q (head-major) or the caller's q (token-major): element (t, h, d) at
  int64_t q_rs;       // t * q_rs + h * q_hs + d
  int64_t q_hs;
  const uint16_t* khat;
  const uint16_t* v16;
  uint16_t* out;
  float* lse;
  float* o32;  // optional: the output before its bf16 rounding, fp32 token-major
  int32_t* status_out;  // optional: receives the call's data-error code (H3ATTN_OK or H3ATTN_ERR_*)
  const WsHeader* hdr;
  const int32_t* segtab;
  const int32_t* items;
  const int32_t* segflag;  // per segment: nonzero = a value cannot enter the products (NaN outputs)
  int32_t* sched;          // the per-XCD work counters and the done count (zero between launches)
  const int32_t* bkt;      // cost classes of the item list: first item and count, most expensive first
  int64_t T;
  int32_t H;
  float c;            // scale * log2(e)
  int32_t xcd_slots;  // workgroups per XCD (grid / 8), for the XCD-aware item order
};

// Maximum over the query's 96 keys of one tile (exact: any evaluation order gives these bits).
__device__ __forceinline__ float tile_max(const f32x16* S) {
  float a = -__builtin_inff();
#pragma unroll
  for (int kb = 0; kb < NKB; kb++)
#pragma unroll
    for (int i = 0; i < 16; i += 2) a = __builtin_fmaxf(__builtin_fmaxf(a, S[kb][i]), S[kb][i + 1]);
  float x, y;
  swap_halves(a, x, y);
  return __builtin_fmaxf(x, y);
}

// Q prologue for one 32-query block: the lane's 64 bf16 values of its query row (lane half hh
// holds dims 16m + 8hh .. +7), which are the B operands as they are; zeros past the segment end.
__device__ __forceinline__ void load_q(const AttnParams& p, int s0, int qrow, bool qvalid, int head, int hh,
                                       bf16x8* qf) {
  const uint16_t* qp = p.q + (int64_t)head * p.q_hs + (int64_t)(s0 + (qvalid ? qrow : 0)) * p.q_rs;
#pragma unroll
  for (int m = 0; m < 8; m++) {
    u32x4 w4 = {0, 0, 0, 0};
    if (qvalid) w4 = *(const u32x4*)(qp + 16 * m + 8 * hh);
    qf[m] = __builtin_bit_cast(bf16x8, w4);
  }
}

// p = exp2(s*c - m) for the lane's 48 keys, packed to fp16 B operands; returns the sum of the
// FP32 values in a fixed order (a binary tree within each 32-key block, then the blocks in order).
__device__ __forceinline__ float exp_pack_sum(const f32x16* S, float c, float m, f16x8* pf) {
  // one 32-key block at a time, so at most 16 values of p are live
  float t = 0.0f;
#pragma unroll
  for (int kb = 0; kb < NKB; kb++) {
    float pr[16];
#pragma unroll
    for (int i = 0; i < 16; i++) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][i], c, -m));
    pf[2 * kb] = pack_p(&pr[0]);
    pf[2 * kb + 1] = pack_p(&pr[8]);
    const float tb = tree_sum<16>(pr);
    t = kb == 0 ? tb : t + tb;
  }
  return t;
}

template <int N>
struct Par {
  static constexpr int value = N;
};

__global__ __launch_bounds__(64 * NWAVES, 1) void k_attn_fwd(AttnParams p) {
  // K tiles in buffers 0, 1 and V tiles in buffers 2, 3 (24 KB each)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * FTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int grp = wv >> 2;     // 0: leading waves, 1: waves one phase behind (same SIMDs)
  const int hh = lane >> 5;    // which half of the 16-wide MFMA k-slice this lane feeds
  const int l32 = lane & 31;   // query (B / D column) index within the wave
  const int64_t T = p.T;
  const int H = p.H;

  // Every kernel that records data errors ran before this one on the stream: the word is final.
  if (p.status_out && blockIdx.x == 0 && tid == 0) *p.status_out = status_code(p.hdr->status);
  if (p.hdr->status & STATUS_SEG_BIT) {
    // The segment ids decrease, so no segmentation exists: make the whole result unmistakably invalid.
    const int64_t n16 = T * H * HD / 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + tid; e < n16; e += stride) *(u32x4*)(p.out + e * 8) = nan4;
    if (p.lse)
      for (int64_t e = (int64_t)blockIdx.x * blockDim.x + tid; e < T * H; e += stride) p.lse[e] = __builtin_nanf("");
    if (p.o32) {
      const f32x4 nanf4 = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      for (int64_t e = (int64_t)blockIdx.x * blockDim.x + tid; e < T * H * HD / 4; e += stride)
        *(f32x4*)(p.o32 + e * 4) = nanf4;
    }
    return;
  }

  // Counts come from the plan kernel; clamp them so that even a workspace that was never planned
  // cannot send a work item outside the tensors.
  const int64_t max_items = T + (T + BQ - 1) / BQ;
  const int nseg = (int)min((int64_t)max(p.hdr->nseg, 0), T);
  const int nitems = (int)min((int64_t)max(p.hdr->nitems, 0), max_items);
  const int nwork = nitems * H;

  // Work order: workgroup b runs on XCD b % 8, and XCD x owns the x-th eighth of the head-major
  // order of (segment, 256-query tile, head) items, so the workgroups of one XCD share the K/V tiles
  // of one head in that XCD's L2.  A workgroup's first unit is its slot s; after that the XCD's
  // workgroups take units from a counter of their own, so one that finishes early (items of short
  // segments cost less) takes the next.  When the XCD's last round of items would be at most half
  // full, those items are split into 128-query halves: waves 0..3 compute a half with no partner on
  // their SIMDs (each phase slot is then one wave's phase, not the longer of two), while waves 4..7
  // issue only their K copies and meet the barriers.  Whether an item runs whole or in halves, and
  // which workgroup runs it, changes no bit of any output: every row runs the same instructions
  // either way.
  // A unit's start waits on memory once: the item entry (which carries the segment's start and
  // length), then the segment's flag, the counter's reply, K(0) and Q all in flight together.  The
  // barriers at a unit's start and end guard LDS only, so no unit waits for the previous one's
  // output stores; the next unit's index goes through LDS slot it & 1, written as soon as the
  // counter's reply is known to have arrived.
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int nslots = p.xcd_slots;
  // One round (no XCD has more of the list's units than workgroups): units in list order, each
  // workgroup's slot its only unit.  Otherwise longest first: the plan groups the items by the cost
  // class of their segment, most expensive first, and XCD x takes the x-th eighth of every class
  // (head-major inside a class, so a head's items still share an L2), so the cheap units come last
  // and even out the workgroups' ends.  Either order changes which workgroup runs an item, never a
  // result.
  const bool one_round = (nwork + 7) / 8 <= nslots;
  const int nbkt = min(max(p.hdr->nbkt, 0), NBKT);
  __shared__ int32_t s_bkt[2 * NBKT];
  int64_t lo = 0, cnt = 0;
  if (one_round) {
    lo = (int64_t)nwork * xcd / 8;
    cnt = (int64_t)nwork * (xcd + 1) / 8 - lo;
  } else {
    if (tid < 2 * NBKT) s_bkt[tid] = tid < 2 * nbkt ? p.bkt[tid] : 0;
    lds_barrier();
    for (int b = 0; b < nbkt; b++) {
      const int64_t span = (int64_t)max(s_bkt[2 * b + 1], 0) * H;
      cnt += span * (xcd + 1) / 8 - span * xcd / 8;
    }
  }
  const int64_t last = cnt % nslots;  // items of the XCD's last round
  const int64_t nfull = (last != 0 && 2 * last <= nslots) ? cnt - last : cnt;
  const int64_t nunits = nfull + 2 * (cnt - nfull);
  // In one round no XCD has more units than workgroups (nunits <= nslots holds exactly when
  // cnt <= nslots, and cnt <= ceil(nwork / 8)): every unit is some workgroup's first, and the
  // counters stay untouched.

  const int k_lane_off = tile_lane_offset(false, wv, lane);
  // the loop's copies: each wave of a group issues a quarter of a tile
  const int k_lane_off4 = tile_lane_offset(false, wv & 3, lane);
  const int v_lane_off4 = tile_lane_offset(true, wv & 3, lane);
  // the loop's copies: each wave copies one kind (K in the trailing group, V in the leading one);
  // its six lane offsets are kept in registers of their own
  int coffs[FROWS / 16];
#pragma unroll
  for (int i = 0; i < FROWS / 16; i++) {
    coffs[i] = (grp ? k_lane_off4 : v_lane_off4) + i * 4096;
    asm volatile("" : "+v"(coffs[i]));
  }
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const float c = p.c;
  uint32_t vb[4];  // LDS byte addresses of the lane's V operand rows (buffer 0, rows tr_row), by db
#pragma unroll
  for (int db = 0; db < 4; db++)
    vb[db] = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint16_t*)(lds + 2 * FTILE +
                                                                                   v_off(tr_row, 32 * db + tr_col));

  __shared__ int32_t s_unit[2];  // the next unit, written during unit i into slot i & 1
  int32_t fetched = 0;  // thread 0: the counter value fetched during the current unit
  int it = 0;           // units this workgroup has started
  for (int64_t u = slot; u < nunits;) {
    bool posted = false;  // thread 0: the next unit is in s_unit[it & 1]
    do {  // one unit; its early exits (continue) end the do, not the walk over units
    // the next unit's counter value, fetched now and posted once K(0) has landed (below)
    if (!one_round && tid == 0) fetched = atomicAdd(&p.sched[SCHED_STRIDE * xcd], 1);
    // unit u: the XCD's k-th item, whole (half = -1) or its first or second 128 queries (half = 0, 1)
    const int64_t k = u < nfull ? u : nfull + ((u - nfull) >> 1);
    const int half = u < nfull ? -1 : (int)((u - nfull) & 1);
    int head = -1, item = -1;
    if (one_round) {
      const int64_t v = lo + k;
      head = (int)(v / nitems);
      item = (int)(v - (int64_t)head * nitems);
    } else {
      int64_t kc = k;
      for (int b = 0; b < nbkt; b++) {
        const int cb = max(s_bkt[2 * b + 1], 0);
        const int64_t span = (int64_t)cb * H, blo = span * xcd / 8, blen = span * (xcd + 1) / 8 - blo;
        if (kc < blen) {
          const int64_t g = blo + kc;
          head = (int)(g / cb);
          item = s_bkt[2 * b] + (int)(g - (int64_t)head * cb);
          break;
        }
        kc -= blen;
      }
    }
    if ((unsigned)item >= (unsigned)nitems || (unsigned)head >= (unsigned)H) continue;
    // the item: (segment, query tile, the segment's start, its length)
    const u32x4 it4 = *(const u32x4*)(p.items + 4 * item);
    const int seg = (int)it4[0], qt = (int)it4[1], s0 = (int)it4[2], L = (int)it4[3];
    if ((unsigned)seg >= (unsigned)nseg) continue;
    if (s0 < 0 || L <= 0 || (int64_t)s0 + L > T || qt < 0 || qt * BQ >= L) continue;

    // the wave's 32 query rows (segment-relative); in a half item waves w and w + 4 name the same rows
    const int row0 = qt * BQ + (half < 0 ? 32 * wv : 128 * half + 32 * (wv & 3));
    // the segment's flag, read now and tested once K(0) and Q have landed (its latency overlaps theirs)
    const int flag = p.segflag[seg];
    const int ntiles = (L + FROWS - 1) / FROWS;
    const int rem = L - (ntiles - 1) * FROWS;  // valid keys of the last tile, 1..FROWS
    const uint16_t* kbase = p.khat + ((int64_t)head * T + s0) * HD;
    const uint16_t* vbase = p.v16 + ((int64_t)head * T + s0) * HD;

    // Every wave has finished reading LDS for the previous item before it is overwritten (LDS
    // only: the previous item's output stores need not have landed).
    lds_barrier();
    ftile_to_lds<NWAVES>(kbase, L, lds, wv, k_lane_off);  // K(0)
    const bool idle = half >= 0 && grp == 1;  // waves 4..7 of a half item: copies and barriers only
    const int qrow = row0 + l32;
    const bool qvalid = qrow < L;
    bf16x8 qf[8];
    if (!idle) load_q(p, s0, qrow, qvalid, head, hh, qf);
    __builtin_amdgcn_s_waitcnt(0xF70);  // K(0), Q and the flag have landed
    // the counter's reply arrived with them (vmcnt counts all): post the next unit now, so the
    // unit's end waits for no memory operation
    if (!one_round && tid == 0) {
      s_unit[it & 1] = nslots + fetched;
      posted = true;
    }
    if (flag != 0) {
      // This segment holds a value that cannot enter the products (or invalid position ids): its
      // rows are NaN; every other segment is computed as usual.
      const int qr = row0 + l32;
      if (qr < L && (half < 0 || grp == 0)) {
        const int64_t r = (int64_t)(s0 + qr) * H + head;
        const u32x2 nan2 = {0x7FC07FC0u, 0x7FC07FC0u};
#pragma unroll
        for (int d = 0; d < HD / 2; d += 4) *(u32x2*)(p.out + r * HD + 2 * d + 4 * hh) = nan2;
        if (p.lse && hh == 0) p.lse[r] = __builtin_nanf("");
        if (p.o32) {
          const f32x4 nanf4 = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
#pragma unroll
          for (int d = 0; d < HD / 2; d += 4) *(f32x4*)(p.o32 + r * HD + 2 * d + 4 * hh) = nanf4;
        }
      }
      continue;
    }

    // K(m+1) and V(m) go into the buffers of K(m-1) and V(m-2), which were last read in slot 2m-1.
    // The buffer parity MP = m & 1 is a compile-time constant at every call, so the compiler can
    // see that a copy never writes the buffers being read and needs no wait for it.
    // trailing waves, even slot t = 2m: K(m+1) (two slots to land)
    auto issue_k = [&](int t, auto mp) {
      constexpr int MP = decltype(mp)::value;
      const int m = t >> 1;
      if (m + 1 < ntiles)
        ftile_to_lds_o<4>(kbase + (int64_t)(m + 1) * FROWS * HD, L - (m + 1) * FROWS, lds + (1 - MP) * FTILE, wv & 3,
                          coffs);
    };
    // leading waves, odd slot t = 2m+1: V(m) (one slot to land)
    auto issue_v = [&](int t, auto mp) {
      constexpr int MP = decltype(mp)::value;
      const int m = t >> 1;
      if (m < ntiles)
        ftile_to_lds_o<4>(vbase + (int64_t)m * FROWS * HD, L - m * FROWS, lds + (2 + MP) * FTILE, wv & 3, coffs);
    };

    if (idle) {
      // waves 4..7 of a half item: the trailing group's K copies and barriers, and no arithmetic
      const int tau_idle = 2 * ntiles;
      auto idle_phase = [&](int tau, auto tm) {
        constexpr int TM = decltype(tm)::value;
        const int t = tau + 1;
        if (!(t & 1)) __builtin_amdgcn_s_waitcnt(0xF70);
        phase_barrier();
        if constexpr ((TM & 1) == 1) issue_k(t, Par<(TM == 1 ? 1 : 0)>{});
      };
      __builtin_amdgcn_s_waitcnt(0xF70);
      phase_barrier();
      issue_k(0, Par<0>{});
      int tau = 0;
      for (; tau + 3 <= tau_idle; tau += 4) {
        idle_phase(tau, Par<0>{});
        idle_phase(tau + 1, Par<1>{});
        idle_phase(tau + 2, Par<2>{});
        idle_phase(tau + 3, Par<3>{});
      }
      if (tau <= tau_idle) idle_phase(tau, Par<0>{});
      if (tau + 1 <= tau_idle) idle_phase(tau + 1, Par<1>{});
      if (tau + 2 <= tau_idle) idle_phase(tau + 2, Par<2>{});
      continue;
    }

    f32x16 S[NKB];  // scores of the tile whose softmax is next
    f16x8 pf[NKS];  // P of the tile whose P.V is next
    f32x16 O[4];
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int i = 0; i < 16; i++) O[d][i] = 0.0f;
    float lsum = 0.0f;
    float m_run = -__builtin_inff();

    // Phase tau of this wave runs in slot t = tau + grp.  Even tau: G(k), k = tau/2 - 1 (scores of
    // tile k+1 from K buffer (k+1)&1, P.V of tile k from V buffer k&1).  Odd tau: V(k),
    // k = (tau-1)/2 - 1 (softmax of tile k+1).  TM = tau % 4 fixes the buffers at compile time.
    auto phase = [&](int tau, auto tm) {
      constexpr int TM = decltype(tm)::value;
      const int t = tau + grp;
      // copies issued at slot t-2 or t-1 are read from slot t on: wait for them (vmcnt(0)) before the barrier
      if (!(t & 1) && t >= 2) __builtin_amdgcn_s_waitcnt(0xF70);
      phase_barrier();
      // copies only in vector phases (odd tau); m = t / 2 has the parity below
      if constexpr ((TM & 1) == 1) {
        if (grp == 1) issue_k(t, Par<(TM == 1 ? 1 : 0)>{});  // t = 4n + TM + 1: m = 2n + 1 or 2n + 2
        else issue_v(t, Par<(TM == 1 ? 0 : 1)>{});           // t = 4n + TM: m = 2n or 2n + 1
      }
      if constexpr ((TM & 1) == 0) {
        const int k = tau / 2 - 1;
        constexpr int KBUF = TM == 0 ? 0 : 1;  // K(k+1): k = 2n-1 -> K(2n); k = 2n -> K(2n+1)
        constexpr int VBUF = TM == 0 ? 1 : 0;  // V(k)
        if (k + 1 < ntiles) fscores<4>(lds + KBUF * FTILE, qf, l32, hh, S);
        if (k >= 0) ftr_gemm<VBUF>(vb, pf, O);
      } else {
        const int k = (tau - 1) / 2 - 1;
        if (k + 1 < ntiles) {
          if (k + 1 == ntiles - 1 && rem < FROWS) {
            // The key limit enters as an opaque per-lane value, so the 48 compares stay in this
            // last-tile branch: hoisted out of the loop they were 48 SGPR masks, and the SGPR
            // spills they caused were reloaded on every phase.
            int r = rem - 4 * hh;
            asm volatile("" : "+v"(r));
            fmask_tail_rel(S, r);
          }
          float ts = exp_pack_sum(S, c, m_run, pf);
          // rare (the first tile, where m is -inf, or a tile whose p would pass the limit): move m
          if (__builtin_expect(__ballot(!(ts <= P_SUM_LIMIT)) != 0, 0)) {
            float ta, tb;
            swap_halves(ts, ta, tb);
            const bool need = !(ta <= P_SUM_LIMIT) || !(tb <= P_SUM_LIMIT);
            const float mt = tile_max(S) * c;
            const float m_new = need ? __builtin_fmaxf(mt, m_run) : m_run;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            lsum *= alpha;
#pragma unroll
            for (int d = 0; d < 4; d++)
#pragma unroll
              for (int i = 0; i < 16; i++) O[d][i] *= alpha;
            m_run = m_new;
            ts = exp_pack_sum(S, c, m_run, pf);
          }
          lsum += ts;
        }
      }
    };

    if (grp == 1) {                     // slot 0 of the trailing waves: barrier and copies only
      phase_barrier();
      issue_k(0, Par<0>{});
    }
    const int tau_last = 2 * ntiles + 1 - grp;
    int tau = 0;
    for (; tau + 3 <= tau_last; tau += 4) {
      phase(tau, Par<0>{});
      phase(tau + 1, Par<1>{});
      phase(tau + 2, Par<2>{});
      phase(tau + 3, Par<3>{});
    }
    if (tau <= tau_last) phase(tau, Par<0>{});
    if (tau + 1 <= tau_last) phase(tau + 1, Par<1>{});
    if (tau + 2 <= tau_last) phase(tau + 2, Par<2>{});

    // ---------------- epilogue: one division per row, one bf16 rounding per element
    float la, lb;
    swap_halves(lsum, la, lb);
    const float l = la + lb;
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
      if (p.o32) {
        float* o32p = p.o32 + ((int64_t)(s0 + qrow) * H + head) * HD;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
          for (int g = 0; g < 4; g++) {
            const f32x4 f = {O[db][4 * g] * inv, O[db][4 * g + 1] * inv, O[db][4 * g + 2] * inv, O[db][4 * g + 3] * inv};
            *(f32x4*)(o32p + 32 * db + 8 * g + 4 * hh) = f;
          }
      }
      if (p.lse && hh == 0) p.lse[(int64_t)(s0 + qrow) * H + head] = (m_run + __builtin_amdgcn_logf(l)) * LN2;
    }
    } while (0);
    if (one_round) break;
    // the counter hands out the units from nslots on (the first nslots are the slots themselves)
    if (tid == 0 && !posted) s_unit[it & 1] = nslots + fetched;
    lds_barrier();
    u = s_unit[it & 1];
    it++;
  }

  // The last workgroup to leave zeroes the counters, so that the next launch on this workspace (the
  // staged entry points may attend several times per plan) starts from the first unit again.  Every
  // workgroup has made its last fetch, and had its result, before it counts itself out.
  if (!one_round && tid == 0 && atomicAdd(&p.sched[SCHED_DONE], 1) == (int)gridDim.x - 1) {
    for (int x = 0; x < 8; x++) atomicExch(&p.sched[SCHED_STRIDE * x], 0);
    atomicExch(&p.sched[SCHED_DONE], 0);
  }
}

hipError_t launch_attend(const void* q, bool normed, int64_t T, int32_t H, float scale, void* out, float* lse,
                         float* o32, int32_t* status_out, void* ws, int grid_cap, hipStream_t stream) {
  const WsLayout Lw = ws_layout(T, H);
  char* base = (char*)ws;
  AttnParams p;
  p.q = normed ? (const uint16_t*)(base + Lw.qhat) : (const uint16_t*)q;
  p.q_rs = normed ? HD : (int64_t)H * HD;
  p.q_hs = normed ? T * HD : HD;
  p.khat = (const uint16_t*)(base + Lw.khat);
  p.v16 = (const uint16_t*)(base + Lw.v16);
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.o32 = o32;
  p.status_out = status_out;
  p.hdr = (const WsHeader*)base;
  p.segtab = (const int32_t*)(base + Lw.segtab);
  p.items = (const int32_t*)(base + Lw.items);
  p.segflag = (const int32_t*)(base + Lw.segflag);
  p.sched = (int32_t*)(base + Lw.sched);
  p.bkt = (const int32_t*)(base + Lw.bkt);
  p.T = T;
  p.H = H;
  p.c = (float)((double)scale * 1.4426950408889634074);
  // a multiple of 8 workgroups (one slot per XCD each), at most grid_cap and no more than the work
  const int64_t max_work = Lw.max_items * H;
  int64_t grid = grid_cap < max_work ? grid_cap : max_work;
  grid = (grid + 7) & ~(int64_t)7;
  p.xcd_slots = (int32_t)(grid / 8);
  hipLaunchKernelGGL(k_attn_fwd, dim3((unsigned)grid), dim3(64 * NWAVES), 0, stream, p);
  return hipGetLastError();
}

}  // namespace h3
