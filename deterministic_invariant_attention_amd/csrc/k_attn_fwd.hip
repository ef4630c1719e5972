// Forward attention of the H3 node: non-causal softmax attention inside each packed segment
// ("ws1_one_h3_block" page, Bindings table: attention with causal=False over packed layouts), with
// the q RMSNorm fused into the Q load prologue, FP32 accumulation and one bf16 rounding of the
// output ("33B forward/backward" page, Scope: strict mode).
//
// Work item = (segment, 128-query tile, head); a persistent grid walks the items.  Each wave owns 32
// queries.  The product is computed transposed so that one lane owns one query:
//   S^T[key][query] = Khat . Qhat^T   (A = 32 keys x 16 dims from LDS, B = the wave's normed Q held
//                                      in registers; v_mfma_f32_32x32x16_bf16)
//   O^T[dim][query] += V^T . P^T      (A = 32 dims x 16 keys, read from the row-major V tile with
//                                      ds_read_b64_tr_b16; B = P in fp16; v_mfma_f32_32x32x16_f16)
// With that layout the softmax row max and row sum are lane-local over 32 scores plus one exchange
// with lane ^ 32 (the other half of the query's keys).
//
// Determinism and batch invariance: tiles are anchored at the segment's first key and walked in
// ascending order; keys past the segment end are zero in LDS and masked to -inf; every reduction
// tree is fixed; the code path depends only on the segment length.  So each output row is a
// function of its own segment's bytes, never of the batch, the offset, neighbours or the grid.
//
// Online softmax with a lazy maximum: the running maximum m (log2 units) moves only when a tile's
// maximum exceeds it by more than 8, so p = exp2(s*c - m) <= 2^8 stays well inside fp16, and the
// O/l rescale is skipped on most tiles.  Lanes whose m does not move take alpha = 1 exactly.
#include "h3_common.h"
#include "h3_launch.h"

namespace h3 {

constexpr int KPITCH = 136;  // 16-bit elements per K row in LDS (272 B: 16-byte rows shift 4 banks)
constexpr int VPITCH = 160;  // 16-bit elements per V row in LDS (320 B: transposed reads stay conflict-free)
constexpr float LN2 = 0.69314718055994530942f;
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units

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
};

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposed LDS read (gfx950): within each 16-lane group, lane s supplies the address of 4
// consecutive 16-bit elements C_s; lane s receives {C_{s/4}[s%4], C_{4+s/4}[s%4], C_{8+s/4}[s%4],
// C_{12+s/4}[s%4]}.  With C_s = V[key0 + s/4][dim0 + 4(s%4) .. +3] lane s gets V[key0 + i][dim0 + s],
// i = 0..3: four consecutive keys of one dim, the A-operand layout of a P.V MFMA.
__device__ __forceinline__ i16x4 tr_read(const uint16_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uint16_t*)lds_ptr);
}

__device__ __forceinline__ float max3(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }

template <int N>
__device__ __forceinline__ float tree_sum(const float* x) {
  if constexpr (N == 1) {
    return x[0];
  } else {
    return tree_sum<N / 2>(x) + tree_sum<N / 2>(x + N / 2);
  }
}

__global__ __launch_bounds__(256, 2) void k_attn_fwd(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BK * KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BK * VPITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
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
  const int nwork = (int)min((int64_t)max(p.hdr->nitems, 0), max_items) * H;
  // staging map: thread covers 16-byte chunk (tid & 15) of rows (tid >> 4) + 16*i, i = 0..3
  const int st_c = tid & 15;
  const int st_r = tid >> 4;

  for (int w = blockIdx.x; w < nwork; w += gridDim.x) {
    const int item = w / H;
    const int head = w - item * H;
    const int seg = p.items[2 * item];
    const int qt = p.items[2 * item + 1];
    if ((unsigned)seg >= (unsigned)nseg) continue;
    const int s0 = p.segtab[2 * seg];
    const int L = p.segtab[2 * seg + 1];
    if (s0 < 0 || L <= 0 || (int64_t)s0 + L > T || qt < 0 || qt * BQ >= L) continue;

    // ---------------- Q prologue: load, RMSNorm (2 lanes per row), round to bf16 B-operands
    const int qrow = qt * BQ + wv * 32 + l32;
    const bool qvalid = qrow < L;
    bf16x8 qf[8];
    {
      float x[8][8];
      const uint16_t* qp = p.q + ((int64_t)(s0 + (qvalid ? qrow : 0)) * H + head) * HD;
#pragma unroll
      for (int m = 0; m < 8; m++) {
        u32x4 v = {0, 0, 0, 0};
        if (qvalid) v = *(const u32x4*)(qp + 16 * m + 8 * hh);
        unpack8_bf16(v, x[m]);
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

    // ---------------- KV walk
    const int ntiles = (L + BK - 1) / BK;
    const uint16_t* kbase = p.khat + ((int64_t)head * T + s0) * HD;
    const uint16_t* vbase = p.v16 + ((int64_t)head * T + s0) * HD;
    u32x4 kreg[4], vreg[4];
    auto prefetch = [&](int j) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int key = j * BK + st_r + 16 * i;
        kreg[i] = u32x4{0, 0, 0, 0};
        vreg[i] = u32x4{0, 0, 0, 0};
        if (key < L) {
          kreg[i] = *(const u32x4*)(kbase + (int64_t)key * HD + st_c * 8);
          vreg[i] = *(const u32x4*)(vbase + (int64_t)key * HD + st_c * 8);
        }
      }
    };

    f32x16 O[4];
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int i = 0; i < 16; i++) O[d][i] = 0.0f;
    float m_run = -__builtin_inff();
    float lsum = 0.0f;

    prefetch(0);
    for (int j = 0; j < ntiles; j++) {
      __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
      for (int i = 0; i < 4; i++) {
        *(u32x4*)(Ks + (st_r + 16 * i) * KPITCH + st_c * 8) = kreg[i];
        *(u32x4*)(Vs + (st_r + 16 * i) * VPITCH + st_c * 8) = vreg[i];
      }
      __syncthreads();
      if (j + 1 < ntiles) prefetch(j + 1);

      // S^T for keys [32kb, 32kb+32) of the tile
      f32x16 S[2];
#pragma unroll
      for (int kb = 0; kb < 2; kb++) {
#pragma unroll
        for (int i = 0; i < 16; i++) S[kb][i] = 0.0f;
#pragma unroll
        for (int m = 0; m < 8; m++) {
          const bf16x8 a = *(const bf16x8*)(Ks + (32 * kb + l32) * KPITCH + 16 * m + 8 * hh);
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[m], S[kb], 0, 0, 0);
        }
      }
      // lane holds keys 32kb + 8(i/4) + 4hh + (i%4) of its query
      if (j == ntiles - 1) {
        const int rem = L - j * BK;
        if (rem < BK) {
#pragma unroll
          for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int i = 0; i < 16; i++)
              if (32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3) >= rem) S[kb][i] = -__builtin_inff();
        }
      }

      // ---- online softmax (one query per lane pair)
      float mx[8];
#pragma unroll
      for (int g = 0; g < 8; g++) {
        const int kb = g >> 2, i0 = (g & 3) * 4;
        mx[g] = __builtin_fmaxf(max3(S[kb][i0], S[kb][i0 + 1], S[kb][i0 + 2]), S[kb][i0 + 3]);
      }
      float tmax = __builtin_fmaxf(max3(mx[0], mx[1], mx[2]), max3(mx[3], mx[4], mx[5]));
      tmax = max3(tmax, mx[6], mx[7]);
      tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mt = tmax * p.c;
      const bool need = mt > m_run + RESCALE_THRESHOLD;
      if (__ballot(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < 4; d++)
#pragma unroll
          for (int i = 0; i < 16; i++) O[d][i] *= alpha;
        m_run = m_new;
      }
      float pr[32];
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) pr[16 * kb + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][i], p.c, -m_run));
      lsum += tree_sum<32>(pr);

      f16x8 pf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        u32x4 w4;
#pragma unroll
        for (int i = 0; i < 4; i++) w4[i] = pack_f16(pr[8 * ks + 2 * i], pr[8 * ks + 2 * i + 1]);
        pf[ks] = __builtin_bit_cast(f16x8, w4);
      }

      // ---- O^T += V^T P^T ; A rows = dims 32db + l32, A k-slots = keys 16ks + {4hh..4hh+3, 8+4hh..8+4hh+3}
      const int tr_row = 4 * hh + ((lane & 15) >> 2);
      const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const uint16_t* base = Vs + (16 * ks + tr_row) * VPITCH + 32 * db + tr_col;
          const i16x4 lo = tr_read(base);
          const i16x4 hi = tr_read(base + 8 * VPITCH);
          const f16x4 flo = __builtin_bit_cast(f16x4, lo), fhi = __builtin_bit_cast(f16x4, hi);
          const f16x8 a = {flo[0], flo[1], flo[2], flo[3], fhi[0], fhi[1], fhi[2], fhi[3]};
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], O[db], 0, 0, 0);
        }
      }
    }

    // ---------------- epilogue: one division per row, one bf16 rounding per element
    const float l = lsum + __shfl_xor(lsum, 32, 64);
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
  const int64_t max_work = Lw.max_items * H;
  const int grid = (int)(max_work < grid_cap ? max_work : grid_cap);
  hipLaunchKernelGGL(k_attn_fwd, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace h3
