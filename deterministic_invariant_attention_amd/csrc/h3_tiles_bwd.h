// LDS tile machinery of the backward kernels: the unified tile layout (one swizzle for row reads and
// transposed reads of the same tile), the barrier that publishes global-to-LDS copies, and products
// whose LDS reads are issued as inline assembly with explicit lgkmcnt waits (so independent work can
// sit between the MFMAs).
#pragma once

#include "h3_tiles.h"

namespace h3 {

// One layout for tiles that are read both ways (by rows with 16-byte reads and transposed with
// ds_read_b64_tr_b16): row r, chunk c at slot c ^ u_swz(r), u_swz(r) = 4 (r & 3) + ((r >> 2) & 3).
// A half-wave of row reads (32 rows, one chunk) then touches 16 distinct slots per 16 rows, and a
// transposed read (4 consecutive rows from a 4-aligned row, 4 consecutive chunks from a 4-aligned
// chunk) touches 16 distinct slots: both are free of bank conflicts.
__device__ __forceinline__ int u_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int u_off(int r, int d) { return r * HD + (((d >> 3) ^ u_swz(r)) << 3) + (d & 7); }


// tile_lane_offset for the unified layout.
__device__ __forceinline__ int tile_lane_offset_u(int wv, int lane) {
  const int r = 4 * wv + (lane >> 4);
  return r * 256 + ((lane & 15) ^ u_swz(r)) * 16;
}


// Barrier after which every wave sees every global-to-LDS copy issued before it.  A copy lands in
// LDS when the issuing wave's vmcnt drops; the compiler waits for that only before that wave's own
// reads that may alias the copy, and the workgroup fence of __syncthreads does not wait for it, so
// without the explicit wait another wave may read a tile that is still being written.
__device__ __forceinline__ void copies_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  __syncthreads();
}


// The same products with a hook between the MFMAs: hook(Par<T>) runs right after step T's MFMA is
// issued, so independent vector work (the next tile's softmax) executes while the matrix core is
// busy.  Waits are explicit counts, so the hook must not issue LDS reads.
template <int N>
__device__ __forceinline__ void lgkm_wait_tied(u32x2& x, u32x2& y) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "i"(N));
}
template <int V>
struct StepIdx {
  static constexpr int value = V;
};

// NP products of 16 steps each, product p over tile TILES[p] (unified layout) with B operands bop[p]
// into acc[p]; reads run 4 steps ahead across product boundaries.  vb: tr_bases_u.
template <int T0, int T1>
struct TilePair {
  static constexpr int tile(int p) { return p == 0 ? T0 : T1; }
};
template <typename Tiles, int NP, int S>
__device__ __forceinline__ void trh_read(const uint32_t* vb, u32x2 (&va)[32][2]) {
  constexpr int p = S >> 4, T = S & 15;
  constexpr int ks = T >> 2, db = T & 3;
  constexpr int off = Tiles::tile(p) * TILE_ELEMS * 2 + 16 * ks * HD * 2;
  va[S][0] = tr_read_asm<off>(vb[db]);
  va[S][1] = tr_read_asm<off>(vb[4 + db]);
}
template <typename Tiles, int NP, int S, typename Hook>
__device__ __forceinline__ void trh_step(const uint32_t* vb, const f16x8* const* bop, f32x16* const* acc,
                                         u32x2 (&va)[32][2], Hook& hook) {
  constexpr int NS = 16 * NP;
  if constexpr (S + 4 < NS) trh_read<Tiles, NP, S + 4>(vb, va);
  constexpr int ahead = (S + 4 < NS ? 4 : NS - 1 - S);
  lgkm_wait_tied<2 * ahead>(va[S][0], va[S][1]);
  constexpr int p = S >> 4, T = S & 15;
  const f16x4 lo = __builtin_bit_cast(f16x4, va[S][0]), hi = __builtin_bit_cast(f16x4, va[S][1]);
  const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  acc[p][T & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bop[p][T >> 2], acc[p][T & 3], 0, 0, 0);
  hook(StepIdx<S>{});
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (S + 1 < NS) trh_step<Tiles, NP, S + 1>(vb, bop, acc, va, hook);
}
template <typename Tiles, int NP, typename Hook>
__device__ __forceinline__ void tr_gemm_hooked(const uint32_t* vb, const f16x8* const* bop, f32x16* const* acc,
                                               Hook hook) {
  static_assert(NP == 1 || NP == 2, "one or two products");
  u32x2 va[32][2];
  trh_read<Tiles, NP, 0>(vb, va);
  trh_read<Tiles, NP, 1>(vb, va);
  trh_read<Tiles, NP, 2>(vb, va);
  trh_read<Tiles, NP, 3>(vb, va);
  trh_step<Tiles, NP, 0>(vb, bop, acc, va, hook);
}

// Row-read products with assembly reads: S[kb] = sum over m of tile rows
// 32kb + l32's 16-dim slice m times the B operand b[m] (bf16 or fp16, the tile holds the same
// type), reads NPRE steps ahead, explicit waits, and hook(StepIdx<s>) after step s's MFMA (the hook
// must not issue LDS reads).  The lane's read address for slice m is its slice-0 address XOR
// (m << 5), so one base register serves every slice; RowBases.lo addresses tiles 0..3 and .hi tiles
// 4..7 (the ds offset field is 16 bits).
template <int N>
__device__ __forceinline__ void lgkm_wait_tied4(u32x4& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128_asm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
struct RowBases {
  uint32_t lo, hi;  // lane's slice-0 address of tile 0 and of tile 4
};
// The lane's row-read bases in the unified layout (slice m's slot is the slice-0 slot XOR 2m).
__device__ __forceinline__ RowBases row_bases_u(const uint16_t* lds, int l32, int hh) {
  RowBases b;
  b.lo = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint16_t*)(lds + u_off(l32, 8 * hh));
  b.hi = b.lo + 4 * TILE_ELEMS * 2;
  return b;
}
// Step s covers row block kb and dim slice m: interleaved (kb = s % 2, the two accumulators
// alternate) or, with KM, block-major (kb = s / 8: block 0's eight steps first, so its result is
// complete halfway through).
template <int s, bool KM>
struct RowStep {
  static constexpr int kb = KM ? (s >> 3) : (s & 1), m = KM ? (s & 7) : (s >> 1);
};
template <int TILE, int s, bool KM = false>
__device__ __forceinline__ u32x4 rows_read(const RowBases& rb) {
  constexpr int kb = RowStep<s, KM>::kb, m = RowStep<s, KM>::m;
  constexpr int off = (TILE & 3) * TILE_ELEMS * 2 + kb * 32 * HD * 2;
  return ds_read_b128_asm<off>((TILE >= 4 ? rb.hi : rb.lo) ^ (uint32_t)(m << 5));
}
__device__ __forceinline__ f32x16 mfma_rows(const u32x4& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_rows(const u32x4& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), b, c, 0, 0, 0);
}
// init == nullptr: the accumulators start at zero; else S[kb] starts at init[kb] (the first MFMA of
// each accumulator takes it as its addend).
template <int TILE, int NPRE, int s, bool KM, typename BT, typename Hook>
__device__ __forceinline__ void rows_step(const RowBases& rb, const BT* b, f32x16* S, u32x4 (&ka)[16], Hook& hook,
                                          const f32x16* init) {
  constexpr int kb = RowStep<s, KM>::kb, m = RowStep<s, KM>::m;
  if constexpr (s + NPRE < 16) ka[s + NPRE] = rows_read<TILE, s + NPRE, KM>(rb);
  constexpr int ahead = (s + NPRE < 16 ? NPRE : 15 - s);
  lgkm_wait_tied4<ahead>(ka[s]);
  if constexpr (m == 0) S[kb] = mfma_rows(ka[s], b[m], init ? init[kb] : S[kb]);
  else S[kb] = mfma_rows(ka[s], b[m], S[kb]);
  hook(StepIdx<s>{});
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (s + 1 < 16) rows_step<TILE, NPRE, s + 1, KM>(rb, b, S, ka, hook, init);
}
template <int TILE, int NPRE = 4, bool KM = false, typename BT, typename Hook>
__device__ __forceinline__ void gemm_rows(const RowBases& rb, const BT* b, f32x16* S, Hook hook,
                                          const f32x16* init = nullptr) {
  static_assert(TILE >= 0 && TILE <= 7 && NPRE >= 1 && NPRE <= 8, "tile and prefetch depth");
  if (!init) {
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int i = 0; i < 16; i++) S[kb][i] = 0.0f;
  }
  u32x4 ka[16];
  ka[0] = rows_read<TILE, 0, KM>(rb);
  if constexpr (NPRE > 1) ka[1] = rows_read<TILE, 1, KM>(rb);
  if constexpr (NPRE > 2) ka[2] = rows_read<TILE, 2, KM>(rb);
  if constexpr (NPRE > 3) ka[3] = rows_read<TILE, 3, KM>(rb);
  if constexpr (NPRE > 4) ka[4] = rows_read<TILE, 4, KM>(rb);
  if constexpr (NPRE > 5) ka[5] = rows_read<TILE, 5, KM>(rb);
  if constexpr (NPRE > 6) ka[6] = rows_read<TILE, 6, KM>(rb);
  if constexpr (NPRE > 7) ka[7] = rows_read<TILE, 7, KM>(rb);
  rows_step<TILE, NPRE, 0, KM>(rb, b, S, ka, hook, init);
}

// The lane's eight transposed-read base addresses in tile 0 of the unified layout: vb[4u + db] for
// the read of rows 8u + 4hh + ((lane & 15) >> 2) (+16ks: the swizzle repeats every 16 rows, so the
// row slices are constant offsets), columns 32db + the lane's 4-column group.
__device__ __forceinline__ void tr_bases_u(const uint16_t* lds, int lane, uint32_t* vb) {
  const int hh = lane >> 5;
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int u = 0; u < 2; u++)
#pragma unroll
    for (int db = 0; db < 4; db++)
      vb[4 * u + db] = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint16_t*)(
          lds + u_off(tr_row + 8 * u, 32 * db + tr_col));
}


}  // namespace h3
