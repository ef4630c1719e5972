// LDS tile machinery shared by the attention kernels: 64-row tiles of 128 16-bit columns copied
// from head-major global arrays into XOR-swizzled LDS with buffer_load ... lds, the two read
// patterns (16-byte row reads, transposed 8-byte reads), half-wave exchanges and fixed sum trees.
#pragma once

#include "h3_common.h"

namespace h3 {

constexpr int TILE_ROWS = 64;                // rows (keys or queries) per LDS tile
constexpr int TILE_ELEMS = TILE_ROWS * HD;   // 16-bit elements per tile (16 KB)

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Element offsets of a 16-bit value (row r, column d) inside a swizzled tile.
__device__ __forceinline__ int k_off(int r, int d) { return r * HD + ((((d >> 3) ^ (r & 15))) << 3) + (d & 7); }
__device__ __forceinline__ int v_off(int r, int d) { return r * HD + ((((d >> 3) ^ ((r & 3) << 2))) << 3) + (d & 7); }
// One layout for tiles that are read both ways (by rows with 16-byte reads and transposed with
// ds_read_b64_tr_b16): row r, chunk c at slot c ^ u_swz(r), u_swz(r) = 4 (r & 3) + ((r >> 2) & 3).
// A half-wave of row reads (32 rows, one chunk) then touches 16 distinct slots per 16 rows, and a
// transposed read (4 consecutive rows from a 4-aligned row, 4 consecutive chunks from a 4-aligned
// chunk) touches 16 distinct slots: both are free of bank conflicts.
__device__ __forceinline__ int u_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int u_off(int r, int d) { return r * HD + (((d >> 3) ^ u_swz(r)) << 3) + (d & 7); }

// Copy one 64-row tile of a head-major [rows][128] 16-bit array into a swizzled LDS tile with
// buffer_load_dwordx4 ... lds.  The buffer resource covers only the tile's rows inside the segment
// (`valid` rows), so the rows past the segment end read as zeros: nothing outside the segment can
// reach the products.  NW waves share the 16 blocks of 1 KB (4 rows each); each lane's 16 bytes land
// at LDS base + lane * 16, so the lane fetches the global chunk that belongs in that slot.  The slot
// pattern repeats every 16 rows, so one lane offset serves all of a wave's blocks.
__device__ __forceinline__ int tile_lane_offset(bool is_v, int wv, int lane) {
  const int r = 4 * wv + (lane >> 4);  // tile row of the lane's slot in block wv (rows 4wv..4wv+3)
  const int slot = lane & 15;
  const int c = is_v ? (slot ^ ((r & 3) << 2)) : (slot ^ (r & 15));
  return r * 256 + c * 16;  // bytes
}

// The same for the unified layout.
__device__ __forceinline__ int tile_lane_offset_u(int wv, int lane) {
  const int r = 4 * wv + (lane >> 4);
  return r * 256 + ((lane & 15) ^ u_swz(r)) * 16;
}

template <int NW>
__device__ __forceinline__ void tile_to_lds(const uint16_t* gtile, int valid, uint16_t* lds_tile, int wv,
                                            int lane_off) {
  static_assert(TILE_ROWS % (4 * NW) == 0, "whole 1 KB blocks per wave");
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)gtile, (short)0, (valid < TILE_ROWS ? valid : TILE_ROWS) * 256, 0x00020000);
  // The wave's block offset is opaque here, so each copy forms its LDS address (M0) next to its
  // use instead of keeping one hoisted SGPR per buffer and block alive across the whole loop.
  int wofs = wv * 4 * HD;
  asm volatile("" : "+s"(wofs));
#pragma unroll
  for (int i = 0; i < TILE_ROWS / (4 * NW); i++)  // block NW*i + wv = rows 4*NW*i + 4wv .. +3
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_tile + NW * i * 4 * HD + wofs), 16,
                                             lane_off + i * NW * 1024, 0, 0, 0);
}

// Transposed LDS read (ds_read_b64_tr_b16, gfx950): within each 16-lane group, lane s supplies the
// address of 4 consecutive 16-bit elements C_s; lane s receives {C_{s/4}[s%4], C_{4+s/4}[s%4],
// C_{8+s/4}[s%4], C_{12+s/4}[s%4]}.  With C_s = V[key0 + s/4][dim0 + 4(s%4) .. +3] lane s gets
// V[key0 + i][dim0 + s], i = 0..3: four consecutive keys of one dim, the A-operand layout of a P.V
// MFMA.  (Issued as inline assembly below: tr_read_asm.)

// Every lane receives (x of lane l % 32, x of lane l % 32 + 32) in some fixed order; callers only
// combine the pair with commutative operations (max, +), which give the same bits either way.
__device__ __forceinline__ void swap_halves(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  a = __builtin_bit_cast(float, (uint32_t)r[0]);
  b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

template <int N>
__device__ __forceinline__ float tree_sum(const float* x) {
  if constexpr (N == 1) {
    return x[0];
  } else {
    return tree_sum<N / 2>(x) + tree_sum<N / 2>(x + N / 2);
  }
}

// p -> packed fp16 B operand (8 keys), round to nearest even.
__device__ __forceinline__ f16x8 pack_p(const float* p) {
  u32x4 w4;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const f32x2 two = {p[2 * i], p[2 * i + 1]};
    w4[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(two, f16x2));
  }
  return __builtin_bit_cast(f16x8, w4);
}

// Workgroup barrier between phases, without the memory fence of __syncthreads: where the compiler
// cannot tell a copy's LDS target from a later read, that fence makes every wave wait for all of
// its outstanding global-to-LDS copies at every phase, while a copy only has to land two phases
// after it is issued (the explicit vmcnt wait in the phase loop).  Every LDS read before the
// barrier has been consumed, so waited for, by then; the empty asm statements keep the compiler
// from moving memory operations across the barrier.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier after which every wave sees every global-to-LDS copy issued before it.  A copy lands in
// LDS when the issuing wave's vmcnt drops; the compiler waits for that only before that wave's own
// reads that may alias the copy, and the workgroup fence of __syncthreads does not wait for it, so
// without the explicit wait another wave may read a tile that is still being written.
__device__ __forceinline__ void copies_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  __syncthreads();
}

// ds_read_b64_tr_b16 as inline assembly.  The builtin carries no memory operand, so the compiler's
// wait insertion assumes it may read what an outstanding global-to-LDS copy writes and waits for
// every copy before it, which serialises the copies with the matrix phase.  The assembly form is
// invisible to that analysis, so the caller waits for the results itself (LGKM_WAIT_TIED).  base is
// an LDS byte address, OFF a constant byte offset (the instruction's 16-bit offset field).
template <int OFF>
__device__ __forceinline__ u32x2 tr_read_asm(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(base), "i"(OFF));
  return r;
}

// Wait until at most N LDS operations are outstanding; x and y are tied to the wait, so nothing
// that reads them can be scheduled before it.
#define LGKM_WAIT_TIED(N, x, y) asm volatile("s_waitcnt lgkmcnt(" #N ")" : "+v"(x), "+v"(y))

// Products whose A operand is read transposed from a row-major LDS tile (rows = the contracted
// index: keys for P.V, queries in the backward): ACC^T[dim][n] += X^T[dim][row] B[row][n] over the
// tile's 64 rows, with B held as packed fp16 (bop[ks] = rows 16ks + {4hh..4hh+3, 8+4hh..8+4hh+3}).

// A operand of step T = 4ks + db from LDS tile TILE (0..3): rows 16ks + {0..7} and 16ks + 8 + {0..7}.
// vb[db] is the lane's LDS byte address of (row tr_row, column 32db + tr_col) in tile 0; the
// swizzle of a row depends on row & 3 only, so the other rows and tiles are constant offsets.
template <int TILE, int T>
__device__ __forceinline__ void tr_read_step(const uint32_t* vb, u32x2 (&va)[16][2]) {
  constexpr int ks = T >> 2, db = T & 3;
  constexpr int off = TILE * TILE_ELEMS * 2 + 16 * ks * HD * 2;
  va[T][0] = tr_read_asm<off>(vb[db]);
  va[T][1] = tr_read_asm<off + 8 * HD * 2>(vb[db]);
}

// Step T = 4ks + db, so every ACC[db] sums its row slices in order.  Operands are read 4 steps
// ahead; before step T's MFMA the reads of the steps after it (two each, at most 4 steps) may still
// be in flight, and no other LDS operation is (the caller has consumed every earlier LDS read).
template <int TILE, int T>
__device__ __forceinline__ void tr_gemm_step(const uint32_t* vb, const f16x8* pf, f32x16* O, u32x2 (&va)[16][2]) {
  if constexpr (T + 4 < 16) tr_read_step<TILE, T + 4>(vb, va);
  constexpr int ahead = (T + 4 < 16 ? T + 4 : 15) - T;  // later steps already issued
  if constexpr (ahead == 4) LGKM_WAIT_TIED(8, va[T][0], va[T][1]);
  else if constexpr (ahead == 3) LGKM_WAIT_TIED(6, va[T][0], va[T][1]);
  else if constexpr (ahead == 2) LGKM_WAIT_TIED(4, va[T][0], va[T][1]);
  else if constexpr (ahead == 1) LGKM_WAIT_TIED(2, va[T][0], va[T][1]);
  else LGKM_WAIT_TIED(0, va[T][0], va[T][1]);
  const f16x4 lo = __builtin_bit_cast(f16x4, va[T][0]), hi = __builtin_bit_cast(f16x4, va[T][1]);
  const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  O[T & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[T >> 2], O[T & 3], 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (T + 1 < 16) tr_gemm_step<TILE, T + 1>(vb, pf, O, va);
}

template <int TILE>
__device__ __forceinline__ void tr_gemm(const uint32_t* vb, const f16x8* pf, f32x16* O) {
  static_assert(TILE >= 0 && TILE <= 3, "the ds offset field reaches the first four tiles");
  u32x2 va[16][2];
  tr_read_step<TILE, 0>(vb, va);
  tr_read_step<TILE, 1>(vb, va);
  tr_read_step<TILE, 2>(vb, va);
  tr_read_step<TILE, 3>(vb, va);
  tr_gemm_step<TILE, 0>(vb, pf, O, va);
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

// Row-read products (the gemm_scores shape) with assembly reads: S[kb] = sum over m of tile rows
// 32kb + l32's 16-dim slice m times the B operand b[m] (bf16 or fp16, the tile holds the same type), reads NPRE steps ahead, explicit waits, and
// hook(StepIdx<s>) after step s's MFMA (the hook must not issue LDS reads).  The lane's read address
// for slice m is its slice-0 address XOR (m << 5) (K swizzle), so one base register serves every
// slice; kbase[0] addresses tiles 0..3 and kbase[1] tiles 4..7 (the ds offset field is 16 bits).
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
__device__ __forceinline__ RowBases row_bases(const uint16_t* lds, int l32, int hh) {
  RowBases b;
  b.lo = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint16_t*)(lds + k_off(l32, 8 * hh));
  b.hi = b.lo + 4 * TILE_ELEMS * 2;
  return b;
}
// The same for tiles in the unified layout (slice m's slot is again the slice-0 slot XOR 2m).
__device__ __forceinline__ RowBases row_bases_u(const uint16_t* lds, int l32, int hh) {
  RowBases b;
  b.lo = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint16_t*)(lds + u_off(l32, 8 * hh));
  b.hi = b.lo + 4 * TILE_ELEMS * 2;
  return b;
}
template <int TILE, int s>
__device__ __forceinline__ u32x4 rows_read(const RowBases& rb) {
  constexpr int kb = s & 1, m = s >> 1;
  constexpr int off = (TILE & 3) * TILE_ELEMS * 2 + kb * 32 * HD * 2;
  return ds_read_b128_asm<off>((TILE >= 4 ? rb.hi : rb.lo) ^ (uint32_t)(m << 5));
}
__device__ __forceinline__ f32x16 mfma_rows(const u32x4& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_rows(const u32x4& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), b, c, 0, 0, 0);
}
template <int TILE, int NPRE, int s, typename BT, typename Hook>
__device__ __forceinline__ void rows_step(const RowBases& rb, const BT* b, f32x16* S, u32x4 (&ka)[16], Hook& hook) {
  if constexpr (s + NPRE < 16) ka[s + NPRE] = rows_read<TILE, s + NPRE>(rb);
  constexpr int ahead = (s + NPRE < 16 ? NPRE : 15 - s);
  lgkm_wait_tied4<ahead>(ka[s]);
  S[s & 1] = mfma_rows(ka[s], b[s >> 1], S[s & 1]);
  hook(StepIdx<s>{});
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (s + 1 < 16) rows_step<TILE, NPRE, s + 1>(rb, b, S, ka, hook);
}
template <int TILE, int NPRE = 4, typename BT, typename Hook>
__device__ __forceinline__ void gemm_rows(const RowBases& rb, const BT* b, f32x16* S, Hook hook) {
  static_assert(TILE >= 0 && TILE <= 7 && NPRE >= 1 && NPRE <= 8, "tile and prefetch depth");
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++) S[kb][i] = 0.0f;
  u32x4 ka[16];
  ka[0] = rows_read<TILE, 0>(rb);
  if constexpr (NPRE > 1) ka[1] = rows_read<TILE, 1>(rb);
  if constexpr (NPRE > 2) ka[2] = rows_read<TILE, 2>(rb);
  if constexpr (NPRE > 3) ka[3] = rows_read<TILE, 3>(rb);
  if constexpr (NPRE > 4) ka[4] = rows_read<TILE, 4>(rb);
  if constexpr (NPRE > 5) ka[5] = rows_read<TILE, 5>(rb);
  if constexpr (NPRE > 6) ka[6] = rows_read<TILE, 6>(rb);
  if constexpr (NPRE > 7) ka[7] = rows_read<TILE, 7>(rb);
  rows_step<TILE, NPRE, 0>(rb, b, S, ka, hook);
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

// The lane's four tr_gemm base addresses (tile 0, row tr_row, column 32db + tr_col).
__device__ __forceinline__ void tr_bases(const uint16_t* lds, int lane, uint32_t* vb) {
  const int hh = lane >> 5;
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int db = 0; db < 4; db++)
    vb[db] = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint16_t*)(lds + v_off(tr_row, 32 * db + tr_col));
}

// Keys at or past `rem` (the valid keys of the segment's last tile) get -inf.  S[kb] holds keys
// 32kb + 8(i/4) + 4hh + (i%4) of the lane's query.
__device__ __forceinline__ void mask_tail(f32x16* S, int rem, int hh) {
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++)
      if (32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3) >= rem) S[kb][i] = -__builtin_inff();
}
// The same with the lane's limit given as rel = rem - 4hh.
__device__ __forceinline__ void mask_tail_rel(f32x16* S, int rel) {
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++)
      if (32 * kb + 8 * (i >> 2) + (i & 3) >= rel) S[kb][i] = -__builtin_inff();
}

// Products whose A operand is a 64-row LDS tile read by rows (16-byte reads, K swizzle) and whose B
// operand is 32 rows held in registers: S[kb][i] = tile row 32kb + 8(i/4) + 4hh + (i%4) dotted with
// the lane's register row (in the forward: the scores of one 64-key tile for the lane's query).
// Each accumulator sums its k-slices m = 0..7 in order.
template <int NPRE>
__device__ __forceinline__ void gemm_scores(const uint16_t* Kb, const bf16x8* qf, int l32, int hh, f32x16* S) {
  bf16x8 ka[16];
  auto kread = [&](int s) { ka[s] = *(const bf16x8*)(Kb + k_off(32 * (s & 1) + l32, 16 * (s >> 1) + 8 * hh)); };
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++) S[kb][i] = 0.0f;
#pragma unroll
  for (int s = 0; s < NPRE; s++) kread(s);
#pragma unroll
  for (int s = 0; s < 16; s++) {  // step s = 2m + kb
    if (s + NPRE < 16) kread(s + NPRE);
    S[s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qf[s >> 1], S[s & 1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace h3
