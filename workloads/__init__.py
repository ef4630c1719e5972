"""Seeded synthetic inputs for the H3 attention node.

Shared by the oracle tests, the GPU parity tests, the smoke check and the benchmark.  This module
holds none of the method's arithmetic: only the workload shapes, seeded random draws, the cast of
those draws to bf16, and the per-token segment ids of a packed batch.

Recipe (the same for every workload): a CPU ``torch.Generator`` seeded with ``seed`` draws fp32
normals in the order q, k, v, q-norm-weight noise, k-norm-weight noise, then (for gradients) dO;
each draw is cast to bf16 by torch (round to nearest even).  q/k may be multiplied by a constant
before the cast; norm weights are ``bf16(w_scale * (1 + 0.1 * N(0, 1)))``.

Segment ids: one int32 per token, non-decreasing; each segment of each packed row gets the next id,
so a batch of rows is just more segments on the token axis.
"""
from __future__ import annotations

import dataclasses
import hashlib

import torch

HEAD_DIM = 128
# The norm's eps (1e-6) as the float32 value the C ABI receives, so that the oracle and the library
# are handed the same number.
EPS = 9.999999974752427e-07


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    rows: tuple          # one tuple of segment lengths per packed row
    heads: int
    qk_scale: float = 1.0  # multiplier on the q and k draws before the bf16 cast
    w_scale: float = 1.0   # multiplier on the norm weights (sharp-softmax companions)
    normed: bool = True    # False: no norm weights (q/k are taken as already normalised)
    eps: float = EPS
    seed: int = 0
    description: str = ""

    @property
    def seg_lens(self) -> tuple:
        return tuple(L for row in self.rows for L in row)

    @property
    def tokens(self) -> int:
        return sum(self.seg_lens)

    @property
    def scale(self) -> float:
        return HEAD_DIM ** -0.5

    def flops(self) -> float:
        """Nominal forward FLOPs: Q.K^T and P.V over every (query, key) pair inside a segment."""
        return 4.0 * sum(L * L for L in self.seg_lens) * self.heads * HEAD_DIM

    def algorithmic_bytes(self, with_lse: bool = False) -> int:
        """q, k, v read once and out written once (bf16), segment ids, the two norm weights."""
        T, H = self.tokens, self.heads
        b = 4 * T * H * HEAD_DIM * 2 + 4 * T + (2 * HEAD_DIM * 2 if self.normed else 0)
        return b + (4 * T * H if with_lse else 0)


WORKLOADS = {
    # 12 tokens, two segments, 4 heads: small enough for brute force.
    "tiny": Workload("tiny", ((5, 7),), 4, description="1 row of 12 tokens, segments 5+7, 4 heads"),
    # 925 tokens, three segments, 24 heads: short, bandwidth-bound.
    "short3": Workload("short3", ((300, 300, 325),), 24, description="1 row of 925 tokens, segments 300+300+325, 24 heads"),
    # two packed rows of 4253 tokens: row 0 one segment, row 1 three.
    "batch2": Workload("batch2", ((4253,), (2000, 2000, 253)), 40,
                       description="2 rows x 4253 tokens (4253 | 2000+2000+253), 40 heads"),
    # one row of 8349 tokens, one segment, q/k drawn x3: the throughput workload.
    "long": Workload("long", ((8349,),), 40, qk_scale=3.0,
                     description="1 row of 8349 tokens, one segment, 40 heads, q/k = bf16(3 N(0,1))"),
    # sharp-softmax companions of "long" (the norm cancels the x3 of q/k; these sharpen through w).
    "long_w3": Workload("long_w3", ((8349,),), 40, qk_scale=3.0, w_scale=3.0, description="long with norm weights x3"),
    "long_w8": Workload("long_w8", ((8349,),), 40, qk_scale=3.0, w_scale=8.0, description="long with norm weights x8"),
    "long_w25": Workload("long_w25", ((8349,),), 40, qk_scale=3.0, w_scale=25.0, description="long with norm weights x25"),
    "long_raw": Workload("long_raw", ((8349,),), 40, qk_scale=3.0, normed=False,
                         description="long without the norm (q/k = bf16(3 N(0,1)) enter Q.K^T directly)"),
}


def segment_ids(seg_lens) -> torch.Tensor:
    """int32 [T]: token t of the s-th segment (in packing order) gets id s."""
    ids = [torch.full((L,), s, dtype=torch.int32) for s, L in enumerate(seg_lens)]
    return torch.cat(ids) if ids else torch.zeros(0, dtype=torch.int32)


def position_ids(seg_lens) -> torch.Tensor:
    """int32 [T]: each token's position within its segment, 0..L-1 in packing order."""
    ids = [torch.arange(L, dtype=torch.int32) for L in seg_lens]
    return torch.cat(ids) if ids else torch.zeros(0, dtype=torch.int32)


def shuffle_within_segments(seg_lens, seed: int) -> torch.Tensor:
    """int64 [T]: a seeded permutation p of the token axis that keeps every token in its segment;
    row i of the shuffled batch is row p[i] of the original (take q[p], k[p], v[p], positions[p])."""
    g = torch.Generator().manual_seed(seed)
    parts, t0 = [], 0
    for L in seg_lens:
        parts.append(t0 + torch.randperm(L, generator=g))
        t0 += L
    return torch.cat(parts) if parts else torch.zeros(0, dtype=torch.int64)


def make_inputs(w: Workload, with_grad: bool = False) -> dict:
    """CPU tensors: q, k, v bf16 [T, H, 128]; seg int32 [T]; wq, wk bf16 [128] or None; dout if asked."""
    g = torch.Generator().manual_seed(w.seed)
    T, H = w.tokens, w.heads
    shape = (T, H, HEAD_DIM)
    q = (torch.randn(shape, generator=g) * w.qk_scale).to(torch.bfloat16)
    k = (torch.randn(shape, generator=g) * w.qk_scale).to(torch.bfloat16)
    v = torch.randn(shape, generator=g).to(torch.bfloat16)
    wq_noise = torch.randn(HEAD_DIM, generator=g)
    wk_noise = torch.randn(HEAD_DIM, generator=g)
    out = dict(q=q, k=k, v=v, seg=segment_ids(w.seg_lens), wq=None, wk=None)
    if w.normed:
        out["wq"] = (w.w_scale * (1.0 + 0.1 * wq_noise)).to(torch.bfloat16)
        out["wk"] = (w.w_scale * (1.0 + 0.1 * wk_noise)).to(torch.bfloat16)
    if with_grad:
        out["dout"] = torch.randn(shape, generator=g).to(torch.bfloat16)
    return out


def random_inputs(seg_lens, heads, seed=0, qk_scale=1.0, normed=True, w_scale=1.0, with_grad=False) -> dict:
    """Same recipe as make_inputs for an ad-hoc list of segment lengths."""
    wl = Workload("adhoc", (tuple(seg_lens),), heads, qk_scale=qk_scale, w_scale=w_scale, normed=normed, seed=seed)
    return make_inputs(wl, with_grad=with_grad)


ROPE_PAIRS = 48  # MM-RoPE: 48 rotated pairs (96 of the 128 channels)


def rope_tables(seg_lens, kind: str = "grid", seed: int = 0):
    """float32 [T, 48] cosine and sine tables of the partial MM-RoPE, per token (packed order).

    kind "grid": a synthetic 3-axis layout standing in for video tokens: each segment's tokens fill a
    frames x 8 x 8 grid in order, pairs 0-15 take the frame index, 16-31 the row, 32-47 the column,
    with angle = position * 10000^(-j/16) for the j-th pair of an axis.  kind "random": uniform
    angles in [0, 2 pi).  kind "identity": cos 1, sin 0.  (The pages give neither the axis split nor
    the frequencies; these are inputs, not part of the method.)"""
    T = sum(seg_lens)
    if kind == "identity":
        return torch.ones(T, ROPE_PAIRS), torch.zeros(T, ROPE_PAIRS)
    if kind == "random":
        g = torch.Generator().manual_seed(seed)
        ang = torch.rand(T, ROPE_PAIRS, generator=g, dtype=torch.float64) * (2 * torch.pi)
    else:
        pos = torch.cat([torch.arange(L, dtype=torch.float64) for L in seg_lens]) if T else torch.zeros(0)
        f, rem = torch.div(pos, 64, rounding_mode="floor"), torch.remainder(pos, 64)
        y, x = torch.div(rem, 8, rounding_mode="floor"), torch.remainder(rem, 8)
        freq = 10000.0 ** (-torch.arange(16, dtype=torch.float64) / 16)
        ang = torch.cat([f[:, None] * freq, y[:, None] * freq, x[:, None] * freq], 1)
    return torch.cos(ang).float().contiguous(), torch.sin(ang).float().contiguous()


def row_slices(w: Workload):
    """Token ranges [(t0, t1)] of each packed row of the workload."""
    out, t = [], 0
    for row in w.rows:
        n = sum(row)
        out.append((t, t + n))
        t += n
    return out


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()
