/*
 * h3attn -- deterministic, batch-invariant full attention of the MiniMax-H3 block with its fused
 * per-head q/k RMSNorm, for AMD Instinct MI355X (gfx950).  C ABI of libh3attn.so.
 *
 * The operation (RL-Kernel MiniMax-H3 pull-request pages):
 *   - "ws1_one_h3_block + full-model qualification", Bindings table: q_norm/k_norm is an RMSNorm over
 *     each 128-wide head (bitwise nn.RMSNorm semantics), then attention with causal=False;
 *     Results: the norm weight is one 128-element tensor shared by all heads; Summary: sequences are
 *     packed on one token axis, and a token attends only to its own sequence.
 *   - "33B forward/backward and rollout-vs-train control", Scope (strict mode): no fast-math, no
 *     split-K, FP32 accumulation with one final rounding; unsupported shapes, dtypes and devices
 *     raise instead of falling back.
 *   - same page, dual-trajectory results: a row must give the same bits whether it runs alone
 *     (rollout) or inside a batch (training).
 *
 * Definitions used by every entry point below:
 *   T = tokens >= 0, H = heads >= 1, head_dim must be 128.
 *   q, k, v, out: bf16 [T, H, 128], contiguous, token-major (element (t, h, d) at (t*H + h)*128 + d).
 *   seg_ids: int32 [T], non-decreasing; a segment is a maximal run of equal ids.  Every token attends
 *     to all tokens of its own segment (non-causal) and to nothing else.  A batch of packed rows is
 *     the concatenation of the rows with distinct ids at row boundaries.
 *   wq, wk: bf16 [128] RMSNorm weights.  Norm of one (token, head) row x, evaluated in FP64 because
 *     its bf16 output is a rounding decision: ms = (sum_d x_d^2) / 128 summed in a fixed tree,
 *     r = 1 / sqrt(ms + eps) (correctly rounded sqrt and division), y_d = (x_d * r) * w_d, then ONE
 *     round-to-nearest-even from FP64 to bf16.  The normed q and k enter Q.K^T as bf16.
 *   Attention: S = scale * Qn.Kn^T in FP32 (bf16 MFMA, FP32 accumulate); an online softmax over the
 *     segment's keys in fixed 96-key tiles, walked in ascending order from the segment's first key;
 *     O = (sum_j p_ij v_j) / l_i, rounded once to bf16.  P.V runs on fp16 MFMA with V converted
 *     exactly to fp16 (bf16 P would miss the accuracy bound).
 *   lse (optional, may be NULL): fp32 [T, H], natural-log log-sum-exp of each row's scaled scores.
 *   Determinism: every output row is a function of its own segment's bytes, the weights, eps and
 *     scale only -- not of the batch, the segment's offset in the batch, neighbouring segments,
 *     the grid size or occupancy.  Repeated calls give identical bits.
 *
 * Ownership and threading: the caller allocates every buffer (device memory unless stated) and keeps
 * it alive until the enqueued work completes.  The library never allocates or frees device memory,
 * never synchronises except in h3attn_status_read, and keeps no mutable global state beyond a
 * per-device cache of device properties.  All work is enqueued on `stream` (a hipStream_t; NULL =
 * the default stream) of the current device.  Entry points are thread-safe.
 *
 * Errors are fail-closed, never a fallback.  Argument errors are returned synchronously before any
 * work is enqueued.  Data errors that only the device can see are recorded in the workspace's
 * status word, which h3attn_status_read reports, and the affected outputs are filled with NaN so
 * they cannot be mistaken for valid results:
 *   - decreasing segment ids: no segmentation exists, every output of the call is NaN;
 *   - a value that cannot enter an fp16 product (a finite |v| > 65504; in the backward also a normed
 *     q or k), or position ids that are not a permutation of 0..L-1: only the rows of that value's
 *     segment are NaN.  Every other segment is computed as usual and keeps the bits it has alone,
 *     so a row's output never depends on another segment's bytes.  (The backward's dwq / dwk are
 *     sums over the whole batch and are NaN after any data error.)
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3ATTN_VERSION 3

enum {
  H3ATTN_OK = 0,
  H3ATTN_ERR_NULL = 1,      /* a required pointer is NULL, or exactly one of wq/wk is NULL */
  H3ATTN_ERR_SHAPE = 2,     /* tokens < 0, heads < 1, head_dim != 128, or sizes overflow */
  H3ATTN_ERR_ALIGN = 3,     /* a tensor is not 16-byte aligned (seg_ids/lse: 4; workspace: 256) */
  H3ATTN_ERR_ALIAS = 4,     /* an output overlaps an input or the workspace */
  H3ATTN_ERR_WORKSPACE = 5, /* workspace_bytes < h3attn_workspace_bytes(tokens, heads) */
  H3ATTN_ERR_DEVICE = 6,    /* no current device, or it is not gfx950 */
  H3ATTN_ERR_LAUNCH = 7,    /* the HIP runtime rejected a launch */
  H3ATTN_ERR_SEGMENTS = 8,  /* device status: segment ids decrease somewhere */
  H3ATTN_ERR_RANGE = 9,     /* device status: a finite value > 65504 cannot enter an fp16 product (its segment is NaN) */
  H3ATTN_ERR_POSITIONS = 10, /* device status: position ids are not a permutation of 0..L-1 in a segment (NaN there) */
  H3ATTN_ERR_SCRATCH = 11    /* h3attn_fwd_noalloc: the workspace would exceed its 256 MiB static scratch */
};

/* H3ATTN_VERSION of the loaded library. */
int h3attn_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* h3attn_strerror(int status);

/* Bytes of device workspace that h3attn_fwd, h3attn_fwd_pos and the staged calls need for
 * `tokens` x `heads`: a 256-byte header (status word, counts), the segment table and work list
 * (O(tokens) int32), the normed Q and K and the fp16 V in head-major layout
 * (3 * tokens * heads * 256 bytes) and the two int32 [tokens] maps of the position order.
 * Returns 0 for invalid sizes. */
size_t h3attn_workspace_bytes(int64_t tokens, int32_t heads);

/* The q_norm / k_norm node on its own: y = RMSNorm(x) * w per (token, head) row, as defined above,
 * bitwise identical to the norm fused into h3attn_fwd.  x, y: bf16 [T, H, 128]; w: bf16 [128].
 * y may equal x (in place); any other overlap is H3ATTN_ERR_ALIAS.  eps > 0 (the H3 node uses 1e-6). */
int h3attn_qknorm(const void* x, const void* w, void* y, int64_t tokens, int32_t heads, int32_t head_dim,
                  float eps, void* stream);

/* Full forward of the attention node with its fused q/k norm:
 *   plan (segment decode) -> Q and K norm + fp16 V staging -> attention.
 * wq and wk both NULL means q and k are already normalised (no norm is applied); exactly one NULL
 * is H3ATTN_ERR_NULL.  scale is the softmax scale (the H3 node uses 1/sqrt(128)); it must be finite
 * and > 0.  out must not overlap q, k, v, seg_ids, lse or the workspace.  workspace: device memory
 * of at least h3attn_workspace_bytes(tokens, heads), 256-byte aligned, used as scratch and for the
 * status word; its prior contents do not matter.  tokens == 0 is a no-op returning H3ATTN_OK. */
int h3attn_fwd(const void* q, const void* k, const void* v, const int32_t* seg_ids, const void* wq,
               const void* wk, int64_t tokens, int32_t heads, int32_t head_dim, float eps, float scale, void* out,
               float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* h3attn_fwd with the keys of each segment walked in position order instead of packed order.  The
 * "ws1_one_h3_block + full-model qualification" page (Results, control H-C3) reports that permuting
 * the packed rows together with their positions changes output bits, because attention adds keys
 * in packed order, and leaves that to the attention.  Here the order of the
 * sums follows the positions, so permuting the tokens of a segment together with their position
 * ids permutes the output rows and changes no bit of them.
 *   pos_ids: int32 [T] device memory, 4-byte aligned: the position of each token within its
 *     segment; the ids of a segment of L tokens must be a permutation of 0..L-1.  Anything else
 *     sets H3ATTN_ERR_POSITIONS in the status word and NaN-fills that segment's outputs (checked on
 *     the device).
 * With pos_ids[t] = t - (start of t's segment) the result is bitwise that of h3attn_fwd.  Other
 * arguments as for h3attn_fwd; out and lse must not overlap pos_ids either. */
int h3attn_fwd_pos(const void* q, const void* k, const void* v, const int32_t* seg_ids, const int32_t* pos_ids,
                   const void* wq, const void* wk, int64_t tokens, int32_t heads, int32_t head_dim, float eps,
                   float scale, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* The forward with every option: pos_ids NULL walks keys in packed order (h3attn_fwd), else in
 * position order (h3attn_fwd_pos); o32 (optional, fp32 [T, H, 128] device memory, 16-byte aligned)
 * receives each output element before its one bf16 rounding, for the backward's D = dO . O (see
 * h3attn_bwd_ex).  o32 must not overlap any input, out, lse or the workspace.
 * rope_cos, rope_sin (optional, both or neither, only with wq/wk): the MM-RoPE node that the block
 * runs between q_norm/k_norm and the attention ("ws1_one_h3_block + full-model qualification" page,
 * Bindings table: rope_q, rope_k; Tests: MM-RoPE rotates 96 of 128 channels).  The pages give
 * neither its axis split nor its frequencies, so the rotation is table-driven: float32 [T, 48]
 * device arrays (16-byte aligned, token-major, packed token order) holding, for every token, the
 * cosine and sine of the angle of each of the 48 rotated pairs -- the caller composes the three
 * axes.  Pair i is channels (2i, 2i+1): y_2i = x_2i cos - x_2i+1 sin, y_2i+1 = x_2i sin +
 * x_2i+1 cos; channels 96..127 pass through.  It acts on the normed bf16 q and k, in FP64 with one
 * rounding back to bf16 (each node of the block emits bf16), before Q.K^T.  No output and not the
 * workspace may overlap the tables.  Everything else as for h3attn_fwd; out, lse and o32 carry the
 * same bits whatever pos_ids is; an identity table (cos 1, sin 0) gives the bits of no rope. */
int h3attn_fwd_ex(const void* q, const void* k, const void* v, const int32_t* seg_ids, const int32_t* pos_ids,
                  const void* wq, const void* wk, const float* rope_cos, const float* rope_sin, int64_t tokens,
                  int32_t heads, int32_t head_dim, float eps, float scale, void* out, float* lse, float* o32,
                  void* workspace, size_t workspace_bytes, void* stream);

/* h3attn_fwd for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): it takes no workspace and calls no allocating
 * routine, running on a static scratch array of 256 MiB inside the library instead (each GPU the
 * library runs on holds it until the process ends; the first call on a device resolves its
 * address).  Accepts sizes with h3attn_workspace_bytes(tokens, heads) <= 256 MiB (e.g. 8349 tokens
 * x 40 heads); larger ones return H3ATTN_ERR_SCRATCH before anything is enqueued.  Same kernels and
 * bits as h3attn_fwd with the same arguments.  status: optional device int32 (4-byte aligned) that
 * receives the call's data-error code (H3ATTN_OK, H3ATTN_ERR_SEGMENTS, H3ATTN_ERR_POSITIONS or
 * H3ATTN_ERR_RANGE), since the scratch's status word is not the caller's to read; NULL = not
 * reported (the NaN rows still mark failed segments).  Every call on one GPU uses the same scratch:
 * calls that overlap in time on one GPU (other streams, other threads) race and must not be issued;
 * calls in order on one stream are safe.  Everything the kernels need zeroed is cleared by the
 * call itself, whatever an earlier call left. */
int h3attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* seg_ids, const void* wq,
                       const void* wk, int64_t tokens, int32_t heads, int32_t head_dim, float eps, float scale,
                       void* out, float* lse, int32_t* status, void* stream);

/* The three stages of h3attn_fwd, for callers that reuse one segment plan across layers (the 50
 * blocks of the model share the packed layout) or time the stages.  They must be enqueued in this
 * order on one stream with one workspace: h3attn_plan (resets the status word), h3attn_prep_qkv,
 * h3attn_attend.  h3attn_fwd is exactly these three calls.  h3attn_prep_qkv norms q and k into the
 * workspace (wq, wk both given) and converts v; h3attn_attend takes the same q and wq: with wq it
 * reads the normed Q of the workspace (q and eps are then only checked), without it it reads q. */
int h3attn_plan(const int32_t* seg_ids, int64_t tokens, int32_t heads, void* workspace, size_t workspace_bytes,
                void* stream);
int h3attn_prep_qkv(const void* q, const void* k, const void* v, const void* wq, const void* wk, int64_t tokens,
                    int32_t heads, int32_t head_dim, float eps, void* workspace, size_t workspace_bytes, void* stream);
int h3attn_attend(const void* q, const void* wq, int64_t tokens, int32_t heads, int32_t head_dim, float eps,
                  float scale, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace that h3attn_bwd and h3attn_bwd_pos need for `tokens` x `heads`: the
 * header, the segment table and work list (128-token tiles), four head-major fp16 staged operands
 * (normed q and k, v, dO: 4 * tokens * heads * 256 bytes), the log-sum-exp and D rows
 * (2 * tokens * heads * 4 bytes), the fp32 gradients with respect to the normed q and k
 * (2 * tokens * heads * 512 bytes), the norm-weight gradient partials and the two int32 [tokens]
 * maps of the position order.  0 if invalid. */
size_t h3attn_bwd_workspace_bytes(int64_t tokens, int32_t heads);

/* Backward of the node: gradients of sum(dout * out) with respect to q, k, v and the two norm
 * weights ("33B forward/backward" page: the node inside the training step's backward).  The bf16
 * rounding of the normed q and k is the identity for gradients (straight-through); P is recomputed
 * from the forward's log-sum-exp `lse` (fp32 [T, H], natural log, as h3attn_fwd writes it), and
 * D_i = sum_j P_ij dP_ij is recomputed in FP32 (not taken from the rounded forward output).
 *   dout, q, k, v: bf16 [T, H, 128] (q, k, v as given to h3attn_fwd); seg_ids as for h3attn_fwd.
 *   dq, dk, dv: bf16 [T, H, 128] outputs, each rounded once.
 *   dwq, dwk: fp32 [128] outputs, required when wq/wk are given (ignored otherwise): sums over every
 *     token and head of dy * x * r, added in a fixed order (bitwise repeatable).
 * Determinism: no atomics on data; every gradient row of q, k and v is a function of its own
 * segment's bytes only (the same bits alone or batched); dwq/dwk are sums over the whole batch.
 * Every product runs on fp16 MFMA with FP32 accumulation: P and dS are rounded to fp16 (as P is in
 * the forward), and the normed q, k and v are converted to fp16, which is exact for magnitudes
 * from 2^-17 to 65504 (below 2^-17 the error is at most 2^-25); a finite value beyond 65504 in any of
 * them sets H3ATTN_ERR_RANGE in the status word and NaN-fills its segment's outputs.  dO may take any
 * bf16 value: each (segment, head) of dO is multiplied by the power of two 2^s that brings its
 * largest |dO| into [4, 8) before the fp16 conversion (N(0,1) gradients get s = 0), and the
 * gradients are multiplied by 2^-s on output, both exactly; within one (segment, head), elements
 * more than 2^17 times smaller than the largest lose precision to fp16's subnormals, elements more
 * than 2^27 times smaller are dropped -- a relative error far below the accuracy bound.
 * Outputs must not overlap any input, the workspace or each other. */
int h3attn_bwd(const void* dout, const void* q, const void* k, const void* v, const float* lse,
               const int32_t* seg_ids, const void* wq, const void* wk, int64_t tokens, int32_t heads,
               int32_t head_dim, float eps, float scale, void* dq, void* dk, void* dv, float* dwq, float* dwk,
               void* workspace, size_t workspace_bytes, void* stream);

/* h3attn_bwd in position order (see h3attn_fwd_pos): the operands are staged by position, so the
 * sums over keys (dq), over queries (dk, dv) and over rows (dwq, dwk) run in position order.
 * Permuting the tokens of a segment together with their position ids permutes the gradient rows
 * of q, k and v and changes no bit of them or of dwq and dwk.  pos_ids as for h3attn_fwd_pos (an
 * invalid set gives H3ATTN_ERR_POSITIONS and NaN outputs); lse is the forward's, in packed token
 * order as either forward writes it.  With pos_ids[t] = t - (start of t's segment) the result is
 * bitwise that of h3attn_bwd.  Outputs must not overlap pos_ids either. */
int h3attn_bwd_pos(const void* dout, const void* q, const void* k, const void* v, const float* lse,
                   const int32_t* seg_ids, const int32_t* pos_ids, const void* wq, const void* wk, int64_t tokens,
                   int32_t heads, int32_t head_dim, float eps, float scale, void* dq, void* dk, void* dv, float* dwq,
                   float* dwk, void* workspace, size_t workspace_bytes, void* stream);

/* The backward with every option.  pos_ids as for h3attn_fwd_ex (NULL: packed order).  o32: NULL,
 * or the o32 that h3attn_fwd_ex wrote for the same inputs (and the same pos_ids, which change no bit
 * of it).  With o32, D_i = dO_i . O_i is formed from it once per row (FP64 products and sums,
 * one fp32 rounding) instead of being recomputed from P and dP over every key, which saves two
 * of the dq kernel's five products per (query, key) pair.  O_i in fp32 differs from the exact O_i
 * only by the forward's fp16 rounding of P, unlike the bf16 output, whose rounding alone moves D
 * beyond the gradients' accuracy bound.  Results meet the same bound either way; they are
 * bitwise repeatable and batch-invariant for each choice, and the two choices differ in the last
 * bits.  o32 must not overlap an output or the workspace.  rope_cos, rope_sin: the tables given
 * to h3attn_fwd_ex (or NULL): the products use the rotated operands, and the gradient with respect
 * to each rotated q or k goes back through the transposed rotation before the norm backward (the
 * rope's rounding, like the norm's, is the identity for gradients). */
int h3attn_bwd_ex(const void* dout, const void* q, const void* k, const void* v, const float* lse, const float* o32,
                  const int32_t* seg_ids, const int32_t* pos_ids, const void* wq, const void* wk,
                  const float* rope_cos, const float* rope_sin, int64_t tokens, int32_t heads, int32_t head_dim,
                  float eps, float scale, void* dq, void* dk, void* dv, float* dwq, float* dwk, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Wait for `stream`, then copy the workspace's device status word to *device_status (host memory):
 * H3ATTN_OK, H3ATTN_ERR_SEGMENTS, H3ATTN_ERR_POSITIONS or H3ATTN_ERR_RANGE (in this order of
 * precedence when several are recorded).  Returns the HIP copy's status (H3ATTN_OK or
 * H3ATTN_ERR_LAUNCH). */
int h3attn_status_read(const void* workspace, int32_t* device_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H */
