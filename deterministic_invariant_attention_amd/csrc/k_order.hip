// Position ids -> staged rows, checked.  Token t of a segment starting at s0 with length L and
// position pos[t] is staged at row s0 + pos[t]; the ids of a segment must be a permutation of
// 0..L-1 (the positions restart at zero in each packed sequence).  Two kernels, no float work:
//   k_order_slots  (one thread per token) finds the token's segment by binary search over the
//                  segment starts, writes slot[t] and scatters inv[slot[t]] = t; an id outside
//                  0..L-1 stages the token at its own row and sets STATUS_POS_BIT.
//   k_order_check  (one thread per staged row s) accepts s when t = inv[s] is a token with
//                  slot[t] == s.  A row that no token claims this call fails the check even if inv
//                  holds a stale value from an earlier call (that token's slot is elsewhere now),
//                  and L tokens that each land in their own segment's L rows cover them all only
//                  if no two share a row; so the check passes exactly for permutations.
// Every index stays inside [0, T) whatever the ids are, and inside the token's own segment; a failed
// check flags that segment, whose outputs the attention and backward kernels then fill with NaN
// instead of using the order (the other segments are computed as usual).
#include "h3_common.h"
#include "h3_launch.h"
#include "h3_order.h"

namespace h3 {

__device__ __forceinline__ void flag_status(WsHeader* hdr, bool bad, int32_t bit) {
  const uint64_t any = __ballot(bad);
  if (any && (threadIdx.x & 63) == __builtin_ctzll(any)) atomicOr(&hdr->status, bit);
}

__global__ __launch_bounds__(256) void k_order_slots(const int32_t* __restrict__ pos, int64_t T, WsHeader* hdr,
                                                    const int32_t* __restrict__ segtab, int32_t* __restrict__ slot,
                                                    int32_t* __restrict__ inv, int32_t* __restrict__ segflag) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nseg = (int)min((int64_t)max(hdr->nseg, 0), T);  // 0 after a segment-id error
  bool bad = false;
  int bad_seg = -1;
  if (t < T) {
    int32_t s = (int32_t)t;
    if (nseg > 0) {
      int lo = 0, hi = nseg - 1;  // the last segment whose start is <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (segtab[2 * mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      const int64_t s0 = segtab[2 * lo], len = segtab[2 * lo + 1];
      const int64_t p = pos[t];
      if (p >= 0 && p < len && s0 + p < T) {
        s = (int32_t)(s0 + p);
        inv[s] = (int32_t)t;
      } else {
        bad = true;
        bad_seg = lo;
      }
    }
    slot[t] = s;
  }
  if (bad) flag_segment(segflag, bad_seg, nseg);
  flag_status(hdr, bad, STATUS_POS_BIT);
}

// A staged row s lies in the rows of the segment that token s belongs to (segments are contiguous
// runs in both orders), so tok2seg[s] names the segment to flag.
__global__ __launch_bounds__(256) void k_order_check(int64_t T, WsHeader* hdr, const int32_t* __restrict__ slot,
                                                    const int32_t* __restrict__ inv,
                                                    const int32_t* __restrict__ tok2seg,
                                                    int32_t* __restrict__ segflag) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  bool bad = false;
  const int nseg = hdr->nseg;
  if (s < T && nseg > 0) {
    const int32_t t = inv[s];
    bad = !(t >= 0 && t < T && slot[t] == s);
    if (bad) flag_segment(segflag, tok2seg[s], nseg);
  }
  flag_status(hdr, bad, STATUS_POS_BIT);
}

hipError_t launch_order(const int32_t* pos, int64_t T, void* ws, const int32_t* segtab, const int32_t* tok2seg,
                        int32_t* segflag, int32_t* slot, int32_t* inv, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const unsigned grid = (unsigned)((T + 255) / 256);
  WsHeader* hdr = (WsHeader*)ws;
  hipLaunchKernelGGL(k_order_slots, dim3(grid), dim3(256), 0, stream, pos, T, hdr, segtab, slot, inv, segflag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_order_check, dim3(grid), dim3(256), 0, stream, T, hdr, (const int32_t*)slot,
                     (const int32_t*)inv, tok2seg, segflag);
  return hipGetLastError();
}

}  // namespace h3
