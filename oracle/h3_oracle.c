/*
 * FP64 CPU oracle for the deterministic, batch-invariant H3 full attention node with its per-head
 * q/k RMSNorm.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls this file; only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg do.  It shares no code, header,
 * table or constant with the HIP library: it is written from the pages' description of the node,
 * not from the kernels.
 *
 * What it follows (the RL-Kernel pull-request pages on MiniMax-H3):
 *  - "ws1_one_h3_block + full-model qualification", Bindings table: the block runs
 *    q_norm/k_norm -> rope -> attention(causal=False); q_norm/k_norm is an RMSNorm over each
 *    128-wide head that is bitwise equal to nn.RMSNorm, and its output (the node's output) is bf16.
 *  - same page, Results: the q-norm weight is a 128-element tensor shared by all heads.
 *  - same page, Summary: several sequences are packed on one token axis (packed layouts); each
 *    token attends only to the tokens of its own sequence, non-causally.
 *  - "33B forward/backward and rollout-vs-train control", Scope: FP32 accumulation with one final
 *    rounding.  The oracle is the exact (FP64) value that such a kernel approximates.
 *
 * Readings where the pages are silent:
 *  - segments: int32 ids per token, non-decreasing; a segment is a maximal run of equal ids;
 *  - norm: y = x * (mean(x^2) + eps)^(-1/2) * w over the 128 channels of one (token, head), computed
 *    in FP64 and rounded ONCE, round-to-nearest-even, directly from FP64 to bf16 (the q_norm node's
 *    output dtype); with no weights the inputs are taken as already normalised (no norm at all);
 *  - attention: exact two-pass softmax in FP64 over the keys of the query's own segment,
 *    s_ij = scale * <qhat_i, khat_j>,  O_i = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i),
 *    LSE_i = m_i + ln(sum_j exp(s_ij - m_i)); O is returned in FP64, NOT rounded.
 *
 * Layouts: q, k, v, out are [T, H, 128] (token-major, then head, then channel); lse is [T, H].
 * bf16 values are passed as their uint16 bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HD 128

enum { ORACLE_OK = 0, ORACLE_ERR_ARGS = 1, ORACLE_ERR_SEGMENTS = 2, ORACLE_ERR_NOMEM = 3 };

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---------------------------------------------------------------- bf16 <-> FP64 */

double oracle_bf16_to_f64(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* Round an FP64 value to bf16 in ONE step, round-to-nearest, ties to even.  bf16 keeps 8
 * significant bits and float's exponent range (normals down to 2^-126, subnormals in steps of
 * 2^-133).  x / ulp is exact (ulp is a power of two), nearbyint rounds half to even in the default
 * rounding mode, and the rounded value has at most 8 significant bits, so converting it to float is
 * exact and its top 16 bits are the bf16 pattern. */
uint16_t oracle_f64_to_bf16(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
  double a = fabs(x);
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);          /* a in [2^(e-1), 2^e) */
  int E = e - 1;         /* unbiased exponent */
  if (E < -126) E = -126; /* subnormal range shares the smallest normal's ulp */
  double ulp = ldexp(1.0, E - 7);
  double r = nearbyint(a / ulp) * ulp;
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u); /* overflow to infinity */
  float f = (float)r;
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

/* Element-wise array form of oracle_f64_to_bf16. */
void oracle_f64_to_bf16_array(const double* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; i++) y[i] = oracle_f64_to_bf16(x[i]);
}

/* ---------------------------------------------------------------- segments */

/* Maximal runs of equal ids.  Ids must be non-decreasing; a decrease is an error.
 * starts/lens have room for T entries.  Returns ORACLE_OK or ORACLE_ERR_SEGMENTS. */
int oracle_segments(const int32_t* seg, int64_t T, int64_t* starts, int64_t* lens, int64_t* nseg) {
  int64_t n = 0;
  for (int64_t t = 0; t < T; t++) {
    if (t > 0 && seg[t] < seg[t - 1]) { *nseg = 0; return ORACLE_ERR_SEGMENTS; }
    if (t == 0 || seg[t] != seg[t - 1]) { starts[n] = t; n++; }
  }
  for (int64_t s = 0; s < n; s++) lens[s] = (s + 1 < n ? starts[s + 1] : T) - starts[s];
  *nseg = n;
  return ORACLE_OK;
}

/* ---------------------------------------------------------------- RMSNorm */

/* One (token, head) row, unrounded: y_d = x_d * (mean(x^2) + eps)^(-1/2) * w_d. */
static void norm_row_f64(const uint16_t* x, const uint16_t* w, double eps, double* y) {
  double ss = 0.0;
  double xv[HD];
  for (int d = 0; d < HD; d++) {
    xv[d] = oracle_bf16_to_f64(x[d]);
    ss += xv[d] * xv[d];
  }
  double ms = ss / HD;
  double r = 1.0 / sqrt(ms + eps);
  for (int d = 0; d < HD; d++) y[d] = xv[d] * r * oracle_bf16_to_f64(w[d]);
}

/* Unrounded FP64 norm of every row of x [T, H, 128]; w is [128]. */
int oracle_rmsnorm_f64(const uint16_t* x, const uint16_t* w, double* y, int64_t T, int32_t H, double eps) {
  if (T < 0 || H < 1 || (T > 0 && (!x || !w || !y))) return ORACLE_ERR_ARGS;
  int64_t rows = T * (int64_t)H;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) norm_row_f64(x + r * HD, w, eps, y + r * HD);
  return ORACLE_OK;
}

/* The q_norm / k_norm node: the FP64 norm rounded once to bf16.  y may alias x. */
int oracle_qknorm(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t T, int32_t H, double eps) {
  if (T < 0 || H < 1 || (T > 0 && (!x || !w || !y))) return ORACLE_ERR_ARGS;
  int64_t rows = T * (int64_t)H;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    double yr[HD];
    norm_row_f64(x + r * HD, w, eps, yr);
    for (int d = 0; d < HD; d++) y[r * HD + d] = oracle_f64_to_bf16(yr[d]);
  }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------- attention */

/* ---------------------------------------------------------------- MM-RoPE (partial) */

/* The rope node between q_norm/k_norm and attention ("ws1_one_h3_block" page, Bindings table:
 * rope_q, rope_k; Tests: MM-RoPE rotates 96 of 128 channels).  The pages give neither the axis
 * split nor the frequencies, so the rotation is table-driven: the caller supplies, per token, the
 * cosine and sine of each of the 48 rotated pairs (cos_t, sin_t: [T][48], float32), having composed
 * the three axes itself.  Pairing (a reading): channels (2i, 2i+1) for i < 48 form pair i and are
 * rotated by that pair's angle; channels 96..127 pass through unchanged:
 *   y_2i = x_2i cos - x_2i+1 sin,   y_2i+1 = x_2i sin + x_2i+1 cos.
 * Evaluated in FP64 (the products of bf16 and float32 values are exact), unrounded here. */
#define ROPE_PAIRS 48

static void rope_row_f64(const double* x, const float* c, const float* sn, double* y) {
  for (int i = 0; i < ROPE_PAIRS; i++) {
    const double a = x[2 * i], b = x[2 * i + 1];
    const double ci = (double)c[i], si = (double)sn[i];
    y[2 * i] = a * ci - b * si;
    y[2 * i + 1] = a * si + b * ci;
  }
  for (int d = 2 * ROPE_PAIRS; d < HD; d++) y[d] = x[d];
}

/* The transpose of the rotation (its gradient): dx_2i = dy_2i cos + dy_2i+1 sin,
 * dx_2i+1 = -dy_2i sin + dy_2i+1 cos; channels 96..127 unchanged. */
static void rope_row_transpose_f64(const double* dy, const float* c, const float* sn, double* dx) {
  for (int i = 0; i < ROPE_PAIRS; i++) {
    const double a = dy[2 * i], b = dy[2 * i + 1];
    const double ci = (double)c[i], si = (double)sn[i];
    dx[2 * i] = a * ci + b * si;
    dx[2 * i + 1] = b * ci - a * si;
  }
  for (int d = 2 * ROPE_PAIRS; d < HD; d++) dx[d] = dy[d];
}

/* Unrounded FP64 rotation of every 128-wide row of x [T, H, 128] (bf16 bits) by its token's table. */
int oracle_rope_f64(const uint16_t* x, const float* cos_t, const float* sin_t, double* y, int64_t T, int32_t H) {
  if (T < 0 || H < 1 || (T > 0 && (!x || !cos_t || !sin_t || !y))) return ORACLE_ERR_ARGS;
  int64_t rows = T * (int64_t)H;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    const int64_t t = r / H;
    double xr[HD];
    for (int d = 0; d < HD; d++) xr[d] = oracle_bf16_to_f64(x[r * HD + d]);
    rope_row_f64(xr, cos_t + t * ROPE_PAIRS, sin_t + t * ROPE_PAIRS, y + r * HD);
  }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------- attention */

/* The operands entering Q.K^T, as FP64 in head-major order [H][T][128] (one head's rows contiguous).
 * With weights: the norm node's output, rounded once to bf16 (the node's output dtype) when `round`;
 * then, with rope tables, the rope node on that output, rounded once more to bf16 when `round` (the
 * block's q_norm -> rope -> attention sequence, each node emitting bf16).  Without weights: the
 * inputs themselves (already normalised by the caller; no rope).  round == 0 keeps every step exact
 * (a smooth function, for the finite-difference and "pure" checks). */
static double* operand(const uint16_t* x, const uint16_t* w, const float* cos_t, const float* sin_t, int64_t T,
                       int32_t H, double eps, int round) {
  int64_t n = T * (int64_t)H * HD;
  double* out = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  if (!out) return NULL;
  int64_t rows = T * (int64_t)H;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    const int64_t t = r / H, h = r % H;
    double* o = out + (h * T + t) * HD;
    if (w) {
      double yr[HD];
      norm_row_f64(x + r * HD, w, eps, yr);
      for (int d = 0; d < HD; d++) o[d] = round ? oracle_bf16_to_f64(oracle_f64_to_bf16(yr[d])) : yr[d];
      if (cos_t) {
        rope_row_f64(o, cos_t + t * ROPE_PAIRS, sin_t + t * ROPE_PAIRS, yr);
        for (int d = 0; d < HD; d++) o[d] = round ? oracle_bf16_to_f64(oracle_f64_to_bf16(yr[d])) : yr[d];
      }
    } else {
      for (int d = 0; d < HD; d++) o[d] = oracle_bf16_to_f64(x[r * HD + d]);
    }
  }
  return out;
}

/* Exact softmax attention of query token i (head h) over its segment [s0, s0+L).
 * qh, kh: normed operands, vd: v; all FP64 head-major [H][T][128]. */
static void attend_one(const double* qh, const double* kh, const double* vd, int64_t T, int h, int64_t i,
                       int64_t s0, int64_t L, double scale, double* scores, double* o, double* lse) {
  const double* qi = qh + (h * T + i) * HD;
  double m = -INFINITY;
  for (int64_t j = 0; j < L; j++) {
    const double* kj = kh + (h * T + s0 + j) * HD;
    /* four interleaved partial sums (channels d = 4i + r), added in a fixed order */
    double part[4] = {0.0, 0.0, 0.0, 0.0};
    for (int d = 0; d < HD; d += 4)
      for (int r = 0; r < 4; r++) part[r] += qi[d + r] * kj[d + r];
    const double dot = (part[0] + part[1]) + (part[2] + part[3]);
    scores[j] = scale * dot;
    if (scores[j] > m) m = scores[j];
  }
  double l = 0.0;
  double acc[HD];
  for (int d = 0; d < HD; d++) acc[d] = 0.0;
  for (int64_t j = 0; j < L; j++) {
    double e = exp(scores[j] - m);
    l += e;
    const double* vj = vd + (h * T + s0 + j) * HD;
    for (int d = 0; d < HD; d++) acc[d] += e * vj[d];
  }
  for (int d = 0; d < HD; d++) o[d] = acc[d] / l;
  *lse = m + log(l);
}

/* Shared driver.  rows == NULL: every token; else only the listed query tokens (n_rows of them),
 * with out/lse laid out [n_rows, H, 128] / [n_rows, H]. */
static int fwd_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seg, const uint16_t* wq,
                    const uint16_t* wk, const float* cos_t, const float* sin_t, int round, int64_t T, int32_t H,
                    double eps, double scale, const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  if (T < 0 || H < 1) return ORACLE_ERR_ARGS;
  if ((wq == NULL) != (wk == NULL)) return ORACLE_ERR_ARGS;
  if ((cos_t == NULL) != (sin_t == NULL) || (cos_t && !wq)) return ORACLE_ERR_ARGS; /* rope needs the norm */
  if (T == 0) return ORACLE_OK;
  if (!q || !k || !v || !seg || !out) return ORACLE_ERR_ARGS;
  int64_t* starts = (int64_t*)malloc((size_t)T * sizeof(int64_t));
  int64_t* lens = (int64_t*)malloc((size_t)T * sizeof(int64_t));
  int64_t* seg_of = (int64_t*)malloc((size_t)T * sizeof(int64_t));
  if (!starts || !lens || !seg_of) { free(starts); free(lens); free(seg_of); return ORACLE_ERR_NOMEM; }
  int64_t nseg = 0;
  int rc = oracle_segments(seg, T, starts, lens, &nseg);
  if (rc != ORACLE_OK) { free(starts); free(lens); free(seg_of); return rc; }
  for (int64_t s = 0; s < nseg; s++)
    for (int64_t t = starts[s]; t < starts[s] + lens[s]; t++) seg_of[t] = s;
  int64_t maxlen = 0;
  for (int64_t s = 0; s < nseg; s++) if (lens[s] > maxlen) maxlen = lens[s];

  double* qh = operand(q, wq, cos_t, sin_t, T, H, eps, round);
  double* kh = operand(k, wk, cos_t, sin_t, T, H, eps, round);
  double* vd = operand(v, NULL, NULL, NULL, T, H, eps, 1); /* no weights: the exact values of v */
  if (!qh || !kh || !vd) {
    free(qh); free(kh); free(vd); free(starts); free(lens); free(seg_of);
    return ORACLE_ERR_NOMEM;
  }

  int64_t nq = rows ? n_rows : T;
  for (int64_t r = 0; r < nq; r++)
    if (rows && (rows[r] < 0 || rows[r] >= T)) { rc = ORACLE_ERR_ARGS; break; }
  if (rc == ORACLE_OK) {
    int64_t units = nq * (int64_t)H;
#pragma omp parallel
    {
      double* scores = (double*)malloc((size_t)(maxlen > 0 ? maxlen : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
      for (int64_t u = 0; u < units; u++) { /* head-major: neighbouring units share one head's rows */
        int h = (int)(u / nq);
        int64_t r = u % nq;
        int64_t i = rows ? rows[r] : r;
        int64_t s = seg_of[i];
        double lse_val;
        attend_one(qh, kh, vd, T, h, i, starts[s], lens[s], scale, scores, out + (r * H + h) * HD, &lse_val);
        if (lse) lse[r * H + h] = lse_val;
      }
      free(scores);
    }
  }
  free(qh); free(kh); free(vd); free(starts); free(lens); free(seg_of);
  return rc;
}

/* Forward of the whole node: out [T,H,128] FP64, lse [T,H] FP64 (may be NULL).
 * wq and wk both NULL means q and k are already normalised; exactly one NULL is an error. */
int oracle_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seg, const uint16_t* wq,
               const uint16_t* wk, int64_t T, int32_t H, double eps, double scale, double* out, double* lse) {
  return fwd_impl(q, k, v, seg, wq, wk, NULL, NULL, 1, T, H, eps, scale, NULL, 0, out, lse);
}

/* Forward for selected query tokens only (for sampling full-size workloads). */
int oracle_fwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seg, const uint16_t* wq,
                    const uint16_t* wk, int64_t T, int32_t H, double eps, double scale, const int64_t* rows,
                    int64_t n_rows, double* out, double* lse) {
  if (n_rows < 0 || (n_rows > 0 && !rows)) return ORACLE_ERR_ARGS;
  if (n_rows == 0) return ORACLE_OK;
  return fwd_impl(q, k, v, seg, wq, wk, NULL, NULL, 1, T, H, eps, scale, rows, n_rows, out, lse);
}

/* The forward with every option: rope tables (cos_t, sin_t: [T][48] float32, both or neither; only
 * with weights), the operand rounding (round_operands == 0: the exact FP64 norm and rope outputs),
 * and optionally selected query rows (rows == NULL: every token). */
int oracle_fwd_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seg, const uint16_t* wq,
                  const uint16_t* wk, const float* cos_t, const float* sin_t, int round_operands, int64_t T, int32_t H,
                  double eps, double scale, const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  if (rows && n_rows == 0) return ORACLE_OK;
  if (n_rows < 0) return ORACLE_ERR_ARGS;
  return fwd_impl(q, k, v, seg, wq, wk, cos_t, sin_t, round_operands ? 1 : 0, T, H, eps, scale, rows, n_rows, out,
                  lse);
}

/* ---------------------------------------------------------------- backward */

/* Gradients of the node's composite -- q_norm / k_norm, their bf16 rounding, attention(causal=False)
 * over packed segments -- for an upstream gradient dO ("33B forward/backward" page: the node runs in
 * the training step's backward as well; "ws1_one_h3_block" page, Bindings: the norm and attention
 * nodes).  Everything in FP64.
 *
 * The bf16 rounding of the normed operands is treated as the identity (straight-through): P and the
 * products use the rounded q̂ and k̂, exactly the operands of the forward, and the gradient with
 * respect to q̂ flows unchanged to the unrounded norm output.  round_operands == 0 drops that
 * rounding (q̂, k̂ exact FP64 norm outputs), which makes the result the exact gradient of a smooth
 * function; the tests use that form against finite differences.
 *
 * For one segment and head, with s_ij = scale * q̂_i . k̂_j and P_ij = softmax_j(s_ij):
 *   dV_j = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j,  D_i = sum_j P_ij dP_ij,  dS_ij = P_ij (dP_ij - D_i)
 *   dq̂_i = scale sum_j dS_ij k̂_j,   dk̂_j = scale sum_i dS_ij q̂_i
 * then, per (token, head) row x with r = (mean(x^2) + eps)^(-1/2) and g = w * dŷ (dŷ = dq̂ or dk̂):
 *   dx = r g - (r^3 / 128) x (g . x),    dw += dŷ * x * r   (summed over every token and head).
 * Without weights (wq = wk = NULL) dq = dq̂ and dk = dk̂, and dwq / dwk are not produced. */

static double dot128(const double* a, const double* b) {
  double part[4] = {0.0, 0.0, 0.0, 0.0};
  for (int d = 0; d < HD; d += 4)
    for (int r = 0; r < 4; r++) part[r] += a[d + r] * b[d + r];
  return (part[0] + part[1]) + (part[2] + part[3]);
}

/* One segment of one head: accumulates dq̂ [L][128], dk̂ [L][128], dV [L][128] (zeroed by the caller)
 * for the segment's rows; qh/kh/vd/go are head-major [H][T][128], the segment starts at token s0. */
static void bwd_segment(const double* qh, const double* kh, const double* vd, const double* go, int64_t T, int h,
                        int64_t s0, int64_t L, double scale, double* dqh, double* dkh, double* dvh, double* P,
                        double* dP) {
  for (int64_t i = 0; i < L; i++) {
    const double* qi = qh + (h * T + s0 + i) * HD;
    const double* gi = go + (h * T + s0 + i) * HD;
    double m = -INFINITY;
    for (int64_t j = 0; j < L; j++) {
      P[j] = scale * dot128(qi, kh + (h * T + s0 + j) * HD);
      if (P[j] > m) m = P[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < L; j++) {
      P[j] = exp(P[j] - m);
      l += P[j];
    }
    double Di = 0.0;
    for (int64_t j = 0; j < L; j++) {
      P[j] /= l;
      dP[j] = dot128(gi, vd + (h * T + s0 + j) * HD);
      Di += P[j] * dP[j];
    }
    double* dqi = dqh + i * HD;
    for (int64_t j = 0; j < L; j++) {
      const double dS = P[j] * (dP[j] - Di);
      const double* kj = kh + (h * T + s0 + j) * HD;
      double* dkj = dkh + j * HD;
      double* dvj = dvh + j * HD;
      for (int d = 0; d < HD; d++) {
        dvj[d] += P[j] * gi[d];
        dqi[d] += scale * dS * kj[d];
        dkj[d] += scale * dS * qi[d];
      }
    }
  }
}

/* Norm backward of one row; adds this row's dw contribution to dw_row (caller-owned [128]). */
static void norm_bwd_row(const uint16_t* x_bits, const uint16_t* w_bits, double eps, const double* dy, double* dx,
                         double* dw_row) {
  double x[HD], g[HD];
  double ss = 0.0;
  for (int d = 0; d < HD; d++) {
    x[d] = oracle_bf16_to_f64(x_bits[d]);
    ss += x[d] * x[d];
  }
  const double r = 1.0 / sqrt(ss / HD + eps);
  double gx = 0.0;
  for (int d = 0; d < HD; d++) {
    g[d] = oracle_bf16_to_f64(w_bits[d]) * dy[d];
    gx += g[d] * x[d];
  }
  for (int d = 0; d < HD; d++) {
    dx[d] = r * g[d] - (r * r * r / HD) * x[d] * gx;
    dw_row[d] = dy[d] * x[d] * r;
  }
}

/* Backward of the whole node.  dout, q, k, v: bf16 bits [T,H,128]; outputs dq, dk, dv FP64 [T,H,128];
 * dwq, dwk FP64 [128] (required when weights are given, ignored otherwise).  With rope tables the
 * gradient with respect to the rotated operand goes back through the transposed rotation before
 * the norm backward (the rope node's rounding, like the norm's, is the identity for gradients). */
int oracle_bwd_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seg, const uint16_t* wq,
                  const uint16_t* wk, const float* cos_t, const float* sin_t, const uint16_t* dout, int64_t T,
                  int32_t H, double eps, double scale, int round_operands, double* dq, double* dk, double* dv,
                  double* dwq, double* dwk) {
  if (T < 0 || H < 1) return ORACLE_ERR_ARGS;
  if ((wq == NULL) != (wk == NULL)) return ORACLE_ERR_ARGS;
  if ((cos_t == NULL) != (sin_t == NULL) || (cos_t && !wq)) return ORACLE_ERR_ARGS;
  if (wq && (!dwq || !dwk)) return ORACLE_ERR_ARGS;
  if (wq)
    for (int d = 0; d < HD; d++) dwq[d] = dwk[d] = 0.0;
  if (T == 0) return ORACLE_OK;
  if (!q || !k || !v || !seg || !dout || !dq || !dk || !dv) return ORACLE_ERR_ARGS;
  int64_t* starts = (int64_t*)malloc((size_t)T * sizeof(int64_t));
  int64_t* lens = (int64_t*)malloc((size_t)T * sizeof(int64_t));
  if (!starts || !lens) { free(starts); free(lens); return ORACLE_ERR_NOMEM; }
  int64_t nseg = 0;
  int rc = oracle_segments(seg, T, starts, lens, &nseg);
  if (rc != ORACLE_OK) { free(starts); free(lens); return rc; }
  int64_t maxlen = 0;
  for (int64_t s = 0; s < nseg; s++) if (lens[s] > maxlen) maxlen = lens[s];

  const int64_t n = T * (int64_t)H * HD;
  double* qh = operand(q, wq, cos_t, sin_t, T, H, eps, round_operands);
  double* kh = operand(k, wk, cos_t, sin_t, T, H, eps, round_operands);
  double* vd = operand(v, NULL, NULL, NULL, T, H, eps, 1);
  double* go = operand(dout, NULL, NULL, NULL, T, H, eps, 1);
  double* dqh = (double*)calloc((size_t)n, sizeof(double)); /* head-major [H][T][128] */
  double* dkh = (double*)calloc((size_t)n, sizeof(double));
  double* dvh = (double*)calloc((size_t)n, sizeof(double));
  if (!qh || !kh || !vd || !go || !dqh || !dkh || !dvh) {
    rc = ORACLE_ERR_NOMEM;
  } else {
    const int64_t units = nseg * (int64_t)H;
#pragma omp parallel
    {
      double* P = (double*)malloc((size_t)(maxlen > 0 ? maxlen : 1) * sizeof(double));
      double* dP = (double*)malloc((size_t)(maxlen > 0 ? maxlen : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
      for (int64_t u = 0; u < units; u++) { /* (segment, head) units write disjoint rows */
        const int h = (int)(u % H);
        const int64_t s = u / H;
        const int64_t off = (h * T + starts[s]) * HD;
        bwd_segment(qh, kh, vd, go, T, h, starts[s], lens[s], scale, dqh + off, dkh + off, dvh + off, P, dP);
      }
      free(P);
      free(dP);
    }
    /* back to token-major, with the norm backward; dw summed over rows in (token, head) order */
    double* dwq_rows = wq ? (double*)malloc((size_t)T * H * HD * sizeof(double)) : NULL;
    double* dwk_rows = wq ? (double*)malloc((size_t)T * H * HD * sizeof(double)) : NULL;
    if (wq && (!dwq_rows || !dwk_rows)) {
      rc = ORACLE_ERR_NOMEM;
    } else {
      const int64_t rows = T * (int64_t)H;
#pragma omp parallel for schedule(static)
      for (int64_t r = 0; r < rows; r++) {
        const int64_t t = r / H, h = r % H;
        const int64_t src = (h * T + t) * HD;
        for (int d = 0; d < HD; d++) dv[r * HD + d] = dvh[src + d];
        if (wq) {
          double gq[HD], gk[HD];
          if (cos_t) {
            rope_row_transpose_f64(dqh + src, cos_t + t * ROPE_PAIRS, sin_t + t * ROPE_PAIRS, gq);
            rope_row_transpose_f64(dkh + src, cos_t + t * ROPE_PAIRS, sin_t + t * ROPE_PAIRS, gk);
          } else {
            memcpy(gq, dqh + src, sizeof(gq));
            memcpy(gk, dkh + src, sizeof(gk));
          }
          norm_bwd_row(q + r * HD, wq, eps, gq, dq + r * HD, dwq_rows + r * HD);
          norm_bwd_row(k + r * HD, wk, eps, gk, dk + r * HD, dwk_rows + r * HD);
        } else {
          for (int d = 0; d < HD; d++) {
            dq[r * HD + d] = dqh[src + d];
            dk[r * HD + d] = dkh[src + d];
          }
        }
      }
      if (wq)
        for (int64_t r = 0; r < rows; r++)
          for (int d = 0; d < HD; d++) {
            dwq[d] += dwq_rows[r * HD + d];
            dwk[d] += dwk_rows[r * HD + d];
          }
    }
    free(dwq_rows);
    free(dwk_rows);
  }
  free(qh); free(kh); free(vd); free(go); free(dqh); free(dkh); free(dvh);
  free(starts); free(lens);
  return rc;
}

int oracle_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seg, const uint16_t* wq,
               const uint16_t* wk, const uint16_t* dout, int64_t T, int32_t H, double eps, double scale,
               int round_operands, double* dq, double* dk, double* dv, double* dwq, double* dwk) {
  return oracle_bwd_ex(q, k, v, seg, wq, wk, NULL, NULL, dout, T, H, eps, scale, round_operands, dq, dk, dv, dwq,
                       dwk);
}

/* Forward with the operand rounding optional (round_operands == 0: exact FP64 norm outputs), for the
 * finite-difference checks of the backward and the "pure" reference of the parity report. */
int oracle_fwd_opt(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seg, const uint16_t* wq,
                   const uint16_t* wk, int64_t T, int32_t H, double eps, double scale, int round_operands,
                   double* out) {
  return fwd_impl(q, k, v, seg, wq, wk, NULL, NULL, round_operands ? 1 : 0, T, H, eps, scale, NULL, 0, out, NULL);
}
