// Segment decode: per-token int32 segment ids -> segment table (start, length) and the list of
// attention work items, plus the status word.  An item is (segment, tile, the segment's start, its
// length), so the attention kernels read one 16-byte entry per unit.
//
// Packed layouts ("ws1_one_h3_block" page, Summary: several sequences share one token axis) are
// described to the library by one id per token; a segment is a maximal run of equal ids, and ids
// must not decrease.  The decode runs in one 1024-thread workgroup: each thread walks a contiguous
// run of tokens (then of segments), and one block-wide exclusive scan per pass places every run's
// results, so the whole decode costs two scans and three barriers whatever T is.  For runs of more
// than two tokens (T in (2048, PLAN_STAGE]) the ids are first copied to LDS with coalesced loads
// that are all in flight at once, so the walks read LDS instead of waiting on one global load per
// token (8349 tokens: 12.5 -> 10.3 us per call; at T <= 2048 the extra barrier costs more than it
// saves).
#include "h3_common.h"
#include "h3_bwd.h"
#include "h3_launch.h"
#include "h3_tiles.h"

namespace h3 {

constexpr int TILE_ROWS_PLAN = 64;  // inner-loop tile of the backward kernels (their cost unit)
constexpr int PLAN_STAGE = 16384;   // tokens whose ids the decode stages in LDS (64 KB)

// Exclusive scan of one int per thread over a 1024-thread block; also returns the block total.
__device__ __forceinline__ int block_excl_scan(int v, int* lds_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds_wave[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 16; w++) {
    const int s = lds_wave[w];
    before += (w < wave) ? s : 0;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

// Items are grouped by the cost class of their segment, floor(log2(ceil(L / 64))), most expensive
// class first (the order inside a class is free: it only decides which workgroup runs an item,
// never a result; a segment's tiles stay together, in order), and bkt[2b], bkt[2b+1] = first item
// and item count of the b-th non-empty class; the work counters are reset.
// tok2seg: the segment index of every token; segflag: the per-segment error flags, cleared for the
// call's nseg segments; dmax (backward only, else NULL): the per-(segment, head) maxima of |dO|,
// zeroed for the nseg * H slots the call uses; sched (forward only, else NULL): the attention
// kernel's work counters, zeroed.
__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ seg, int64_t T, WsHeader* hdr,
                                              int32_t* __restrict__ segtab, int32_t* __restrict__ items, int tile,
                                              int32_t* __restrict__ bkt, int32_t* __restrict__ tok2seg,
                                              int32_t* __restrict__ segflag, uint32_t* __restrict__ dmax,
                                              int32_t H, int32_t* __restrict__ sched) {
  __shared__ int lds_wave[16];
  __shared__ int s_bad;
  __shared__ int s_cnt[NBKT], s_run[NBKT];
  __shared__ int s_nbkt;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // pass 1: segment starts at every token whose id differs from its predecessor's.  Each thread owns
  // a contiguous run of ceil(T / 1024) tokens: it counts the starts in its run, one block-wide scan
  // gives every run its first segment index, and a second walk over the run writes the starts and
  // every token's segment.
  const int64_t per = (T + 1023) / 1024;
  const int64_t t0 = min(T, (int64_t)tid * per), t1 = min(T, t0 + per);
  int cnt = 0, bad = 0;
  int nseg;
  if (T > 2048 && T <= PLAN_STAGE) {
    // ids staged in LDS; the second walk overwrites each id with its token's segment index, which
    // is then stored coalesced
    __shared__ int32_t s_ids[PLAN_STAGE];
#pragma unroll
    for (int k = 0; k < PLAN_STAGE / 1024; k++) {
      const int t = k * 1024 + tid;
      if (t < T) s_ids[t] = seg[t];
    }
    __syncthreads();
    const int32_t prev0 = t0 > 0 ? s_ids[t0 - 1] : 0;  // read before any thread overwrites it
    {
      int32_t prev = prev0;
      for (int t = (int)t0; t < (int)t1; t++) {
        const int32_t cur = s_ids[t];
        cnt += (t == 0 || cur != prev) ? 1 : 0;
        bad |= (t > 0 && cur < prev) ? 1 : 0;
        prev = cur;
      }
    }
    const int first = block_excl_scan(cnt, lds_wave, nseg);  // its barriers order prev0 before the writes
    {
      int si = first - 1;
      int32_t prev = prev0;
      for (int t = (int)t0; t < (int)t1; t++) {
        const int32_t cur = s_ids[t];
        if (t == 0 || cur != prev) segtab[2 * (++si)] = t;
        s_ids[t] = si;
        prev = cur;
      }
    }
    __syncthreads();
    for (int t = tid; t < (int)T; t += 1024) tok2seg[t] = s_ids[t];
  } else {
    {
      int32_t prev = t0 > 0 ? seg[t0 - 1] : 0;
      for (int64_t t = t0; t < t1; t++) {
        const int32_t cur = seg[t];
        cnt += (t == 0 || cur != prev) ? 1 : 0;
        bad |= (t > 0 && cur < prev) ? 1 : 0;
        prev = cur;
      }
    }
    const int first = block_excl_scan(cnt, lds_wave, nseg);
    {
      int si = first - 1;  // the segment of token t0 - 1 (the run's tokens before its first start)
      int32_t prev = t0 > 0 ? seg[t0 - 1] : 0;
      for (int64_t t = t0; t < t1; t++) {
        const int32_t cur = seg[t];
        if (t == 0 || cur != prev) segtab[2 * (++si)] = (int32_t)t;
        tok2seg[t] = si;
        prev = cur;
      }
    }
  }
  if (bad) atomicOr(&s_bad, 1);
  for (int i = tid; i < nseg; i += 1024) segflag[i] = 0;
  if (dmax)
    for (int64_t i = tid; i < (int64_t)nseg * H; i += 1024) dmax[i] = 0u;
  if (sched)
    for (int i = tid; i < (int)(SCHED_BYTES / 4); i += 1024) sched[i] = 0;
  __syncthreads();

  // pass 2: lengths
  for (int s = tid; s < nseg; s += 1024) {
    const int32_t st = segtab[2 * s];
    const int32_t en = (s + 1 < nseg) ? segtab[2 * (s + 1)] : (int32_t)T;
    segtab[2 * s + 1] = en - st;
  }
  __syncthreads();

  // pass 3: work items, ceil(L / tile) tiles per segment
  int nitems = 0;
  int nbkt = 0;
  {  // by cost class, most expensive first (the class counts and offsets live in LDS, so the
     // barriers below guard LDS only and do not wait for the table's global stores)
    if (tid < NBKT) s_cnt[tid] = 0;
    lds_barrier();
    for (int s = tid; s < nseg; s += 1024) {
      const int L = segtab[2 * s + 1];
      const int b = 31 - __builtin_clz((unsigned)((L + TILE_ROWS_PLAN - 1) / TILE_ROWS_PLAN));
      atomicAdd(&s_cnt[b], (L + tile - 1) / tile);
    }
    lds_barrier();
    if (tid < 64) {  // one wave: lane l takes class NBKT - 1 - l (most expensive first)
      const int c = NBKT - 1 - tid;
      const int n = tid < NBKT ? s_cnt[c] : 0;
      int x = n;  // inclusive prefix sum of the counts over the lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (tid >= o) x += y;
      }
      const uint64_t nonempty = __ballot(n > 0);
      if (tid < NBKT) s_run[c] = x - n;
      if (n > 0) {
        const int idx = __builtin_popcountll(nonempty & ((1ull << tid) - 1));
        bkt[2 * idx] = x - n;
        bkt[2 * idx + 1] = n;
      }
      if (tid == 63) {
        s_nbkt = __builtin_popcountll(nonempty);
        lds_wave[0] = x;
      }
    }
    lds_barrier();
    nbkt = s_nbkt;
    nitems = lds_wave[0];
    for (int s = tid; s < nseg; s += 1024) {
      const int L = segtab[2 * s + 1];
      const int b = 31 - __builtin_clz((unsigned)((L + TILE_ROWS_PLAN - 1) / TILE_ROWS_PLAN));
      const int nt = (L + tile - 1) / tile;
      const int off = atomicAdd(&s_run[b], nt);
      const int st = segtab[2 * s];
      for (int j = 0; j < nt; j++) {
        const u32x4 e = {(uint32_t)s, (uint32_t)j, (uint32_t)st, (uint32_t)L};
        *(u32x4*)(items + 4 * (off + j)) = e;
      }
    }
  }

  if (tid == 0) {
    const int b = s_bad;
    hdr->nseg = b ? 0 : nseg;
    hdr->nitems = b ? 0 : nitems;
    hdr->nbkt = b ? 0 : nbkt;
    hdr->next[0] = 0;
    hdr->next[1] = 0;
    hdr->status = b ? STATUS_SEG_BIT : 0;
  }
}

hipError_t launch_plan(const int32_t* seg, int64_t T, void* ws, int32_t H, hipStream_t stream) {
  const WsLayout L = ws_layout(T, H);
  char* base = (char*)ws;
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, stream, seg, T, (WsHeader*)base, (int32_t*)(base + L.segtab),
                     (int32_t*)(base + L.items), BQ, (int32_t*)(base + L.bkt), (int32_t*)(base + L.tok2seg),
                     (int32_t*)(base + L.segflag), nullptr, H, (int32_t*)(base + L.sched));
  return hipGetLastError();
}

hipError_t launch_plan_bwd(const int32_t* seg, int64_t T, void* ws, int32_t H, hipStream_t stream) {
  const BwdLayout L = bwd_layout(T, H);
  char* base = (char*)ws;
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, stream, seg, T, (WsHeader*)base, (int32_t*)(base + L.segtab),
                     (int32_t*)(base + L.items), BT, (int32_t*)(base + L.bkt), (int32_t*)(base + L.tok2seg),
                     (int32_t*)(base + L.segflag), (uint32_t*)(base + L.dmax), H, nullptr);
  return hipGetLastError();
}

}  // namespace h3
