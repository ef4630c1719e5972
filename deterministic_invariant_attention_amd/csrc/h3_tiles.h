// LDS tile machinery shared by the attention kernels: tiles of 128 16-bit columns copied
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

// Workgroup barrier for LDS hazards only: this wave's LDS operations are complete (lgkmcnt(0));
// outstanding global loads and stores are not waited for (unlike __syncthreads, whose fence waits
// for them).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// Keys at or past `rem` (the valid keys of the segment's last tile) get -inf.  S[kb] holds keys
// 32kb + 8(i/4) + 4hh + (i%4) of the lane's query.
__device__ __forceinline__ void mask_tail(f32x16* S, int rem, int hh) {
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++)
      if (32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3) >= rem) S[kb][i] = -__builtin_inff();
}

}  // namespace h3
