"""The backward (h3attn_bwd) on the GPU: parity of dq, dk, dv and the norm-weight gradients with the
FP64 oracle, and its bitwise properties (repeat, one row alone vs batched, segment offset).

Bound (whole gradient tensors, bf16 upcast exactly): relative L2 <= 2e-3 and max abs <= 2e-2 *
max(1, max |oracle|) for dq, dk, dv; relative L2 <= 2e-3 for dwq, dwk (fp32).  The max-abs bound is
the forward's (whose outputs are O(1)) scaled by the gradient's largest magnitude: gradients of a
sharp softmax reach ~40, where one bf16 rounding alone moves a value by up to 0.125.  The oracle
evaluates the gradients at the rounded normed operands with the rounding as the identity
(straight-through), the definition the kernels implement.  The full config-5 shape (2 x 4253 tokens, 40 heads) is checked on a subset of
heads, which are independent; its weight gradients (sums over all heads) are compared on the
smaller workloads."""
import numpy as np
import pytest
import torch

import deterministic_invariant_attention_amd as h3
import oracle
import workloads
from gpu_util import EPS, MAX_ABS_BOUND, REL_L2_BOUND, bitwise_equal, digest, f64, metrics, run_fwd, say, to_dev

pytestmark = pytest.mark.gpu
SCALE = 128 ** -0.5


def run_bwd(g, weights=True, eps=EPS, scale=SCALE):
    wq, wk = (g["wq"], g["wk"]) if weights else (None, None)
    _, lse = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], wq, wk, eps=eps, scale=scale, want_lse=True)
    res = h3.h3attn_bwd(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], wq, wk, eps=eps, scale=scale)
    torch.cuda.synchronize()
    return res


def _check(name, x, heads=None, weights=True, eps=EPS, scale=SCALE):
    g = to_dev(x)
    T, H = x["q"].shape[0], x["q"].shape[1]
    say(f"[bwd parity] {name}: T={T} H={H} heads={'all' if heads is None else heads}")
    dq, dk, dv, dwq, dwk = run_bwd(g, weights=weights, eps=eps, scale=scale)
    hs = slice(None) if heads is None else list(heads)
    sub = {n: (x[n][:, hs].contiguous() if n in ("q", "k", "v", "dout") else x[n]) for n in x}
    wq, wk = (x["wq"], x["wk"]) if weights else (None, None)
    ref = oracle.bwd(sub["q"], sub["k"], sub["v"], x["seg"].numpy(), sub["dout"], wq, wk, eps, scale)
    res, mag = {}, {}
    for nm, a, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        a = a[:, hs]
        assert np.all(np.isfinite(f64(a))), nm
        res[nm] = metrics(a, r)
        mag[nm] = max(1.0, float(np.abs(r).max())) if r.size else 1.0
    if weights and heads is None:
        for nm, a, r in (("dwq", dwq, ref[3]), ("dwk", dwk, ref[4])):
            res[nm] = (float(np.linalg.norm(a.cpu().double().numpy() - r) / np.linalg.norm(r)), 0.0)
    say(f"[bwd parity] {name}: " + " ".join(f"{k}: rel_l2={v[0]:.3e} max_abs={v[1]:.3e}" for k, v in res.items()))
    for nm, (rel, mx) in res.items():
        assert rel <= REL_L2_BOUND, nm
        assert mx <= MAX_ABS_BOUND * mag.get(nm, 1.0), nm
    return dq, dk, dv


def test_bwd_parity_tiny():
    _check("tiny", workloads.make_inputs(workloads.WORKLOADS["tiny"], with_grad=True))


def test_bwd_parity_ragged():
    """Segment lengths around the 64-row tiles and the 128-row work items, single-token segments."""
    lens = [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 3, 1, 257]
    _check("ragged", workloads.random_inputs(lens, 3, seed=31, with_grad=True))


def test_bwd_parity_short3():
    _check("short3", workloads.make_inputs(workloads.WORKLOADS["short3"], with_grad=True))


def test_bwd_parity_without_weights():
    _check("no-norm", workloads.random_inputs([150, 77], 2, seed=12, normed=False, with_grad=True), weights=False)


def test_bwd_parity_sharp_softmax():
    """Norm weights x3 (max logit ~50): the case where D from the rounded forward output would fail."""
    _check("sharp-w3", workloads.random_inputs([500, 130], 2, seed=13, w_scale=3.0, with_grad=True))


def test_bwd_parity_many_segments():
    """300 segments of random lengths 1..100 (every cost class of the work order, many items per
    class), 2 heads, against the oracle."""
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(1, 101, 300)]
    _check("many-segments", workloads.random_inputs(lens, 2, seed=42, with_grad=True))


def test_bwd_parity_other_scale_and_eps():
    x = workloads.random_inputs([150, 90], 2, seed=9, with_grad=True)
    _check("scale0.2-eps1e-3", x, eps=float(np.float32(1e-3)), scale=0.2)


def test_bwd_empty_input_is_a_noop():
    x = workloads.random_inputs([4], 2, seed=1, with_grad=True)
    g = to_dev(x)
    e = {n: (t[:0].contiguous() if n in ("q", "k", "v", "dout", "seg") else t) for n, t in g.items()}
    lse = torch.empty(0, 2, dtype=torch.float32, device=g["q"].device)
    dq, dk, dv, dwq, dwk = h3.h3attn_bwd(e["dout"], e["q"], e["k"], e["v"], lse, e["seg"], e["wq"], e["wk"], eps=EPS)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and dk.numel() == 0 and dv.numel() == 0


def test_bwd_parity_batch2_heads():
    """Config 5 (2 x 4253 tokens, 40 heads) at full size, heads 0, 17 and 39 against the oracle."""
    _check("batch2", workloads.make_inputs(workloads.WORKLOADS["batch2"], with_grad=True), heads=(0, 17, 39))


def test_bwd_repeat_bitwise():
    g = to_dev(workloads.make_inputs(workloads.WORKLOADS["short3"], with_grad=True))
    say("[bwd bitwise] short3 repeat x5")
    ref = [digest(t) for t in run_bwd(g)]
    for _ in range(4):
        assert [digest(t) for t in run_bwd(g)] == ref


def test_bwd_repeat_bitwise_batch2():
    """Full config-5 size, all five outputs: many tiles per item, so a wave that read a 64-row tile
    before another wave's copy of it had landed would show up as differing bits."""
    g = to_dev(workloads.make_inputs(workloads.WORKLOADS["batch2"], with_grad=True))
    say("[bwd bitwise] batch2 repeat x3")
    ref = [digest(t) for t in run_bwd(g)]
    for _ in range(2):
        assert [digest(t) for t in run_bwd(g)] == ref


def test_bwd_batch2_alone_equals_batched():
    """Each packed row's dq, dk, dv are the same bits alone as inside the batch (rollout vs train)."""
    wl = workloads.WORKLOADS["batch2"]
    g = to_dev(workloads.make_inputs(wl, with_grad=True))
    say("[bwd bitwise] batch2 alone vs batched")
    bq, bk, bv, _, _ = run_bwd(g)
    for (t0, t1) in workloads.row_slices(wl):
        alone = {n: (g[n][t0:t1].contiguous() if n in ("q", "k", "v", "seg", "dout") else g[n]) for n in g}
        q, k, v, _, _ = run_bwd(alone)
        assert bitwise_equal(q, bq[t0:t1]) and bitwise_equal(k, bk[t0:t1]) and bitwise_equal(v, bv[t0:t1])


@pytest.mark.parametrize("pad", [1, 64, 127])
def test_bwd_leading_segment_offset_invariance(pad):
    x = workloads.random_inputs([300, 129, 64], 3, seed=17, with_grad=True)
    g = to_dev(x)
    say(f"[bwd bitwise] offset shift by a {pad}-token leading segment")
    base = run_bwd(g)[:3]
    d = workloads.random_inputs([pad], 3, seed=99, with_grad=True)
    sh = {n: torch.cat([d[n].to(g[n].device), g[n]]) for n in ("q", "k", "v", "dout")}
    sh["seg"] = torch.cat([torch.full((pad,), -1, dtype=torch.int32), x["seg"]]).to(g["seg"].device)
    sh["wq"], sh["wk"] = g["wq"], g["wk"]
    shifted = run_bwd(sh)[:3]
    for a, b in zip(shifted, base):
        assert bitwise_equal(a[pad:], b)


def test_bwd_nan_neighbour_does_not_leak():
    x = workloads.random_inputs([40, 70, 33], 2, seed=5, with_grad=True)
    g = to_dev(x)
    base = run_bwd(g)[:3]
    y = {n: g[n].clone() for n in g}
    for n in ("q", "k", "v", "dout"):
        y[n][40:110] = float("nan")
    got = run_bwd(y)[:3]
    for a, b in zip(got, base):
        assert bitwise_equal(a[:40], b[:40]) and bitwise_equal(a[110:], b[110:])


def test_bwd_dout_out_of_fp16_range_sets_status():
    x = workloads.random_inputs([20], 2, seed=6, with_grad=True)
    g = to_dev(x)
    g["dout"][3, 1, 7] = 1e6
    _, lse = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], g["wq"], g["wk"], eps=EPS, want_lse=True)
    T, H = x["q"].shape[:2]
    ws = h3.bwd_workspace(T, H, g["q"].device)
    dq, dk, dv, dwq, dwk = h3.h3attn_bwd(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], g["wq"], g["wk"], eps=EPS,
                                         workspace_buf=ws)
    torch.cuda.synchronize()
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_ERR_RANGE
    for t in (dq, dk, dv, dwq, dwk):
        assert torch.isnan(t.float()).all()
