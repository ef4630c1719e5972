"""Pins of the FP64 backward oracle to things other than itself (CPU only).

The oracle's gradients (dq, dk, dv, dwq, dwk of the node for an upstream gradient dO) are checked
against torch's FP64 autograd of an independently written composite (a library routine), against
central finite differences of a smooth FP64 forward, and against exact properties of softmax
attention: single-key segments, sum rules, linearity in dO and segment locality.  A dropped term
of dS, a wrong sign or scale, a transposed product or a mistaken norm backward fails one of them.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

D = 128


def _f64(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _t64(bits):
    return torch.from_numpy(oracle.bf16_to_f64(bits))


def _round_bf16(x):
    """bf16 rounding of FP64 values (the pinned oracle rounding), as a constant."""
    return torch.from_numpy(oracle.bf16_to_f64(oracle.f64_to_bf16(x.detach().numpy())))


def _torch_node(q, k, v, seg, wq, wk, eps, scale, straight_through=True):
    """FP64 torch composite: RMSNorm -> (straight-through) bf16 rounding -> per-segment softmax attention.
    q, k, v: FP64 [T,H,128] tensors (leaves may require grad); wq, wk FP64 [128] or None."""
    def norm(x, w):
        if w is None:
            return x
        y = x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * w
        return y + (_round_bf16(y) - y).detach() if straight_through else y
    qn, kn = norm(q, wq), norm(k, wk)
    starts, lens = oracle.segments(seg)
    outs = []
    for s0, L in zip(starts, lens):
        sl = slice(int(s0), int(s0 + L))
        qs, ks, vs = qn[sl].transpose(0, 1), kn[sl].transpose(0, 1), v[sl].transpose(0, 1)  # [H, L, 128]
        p = torch.softmax(scale * qs @ ks.transpose(1, 2), dim=-1)
        outs.append((p @ vs).transpose(0, 1))
    return torch.cat(outs, 0)


def _inputs(lens, H, seed, normed=True, w_scale=1.0):
    x = workloads.random_inputs(lens, H, seed=seed, normed=normed, w_scale=w_scale, with_grad=True)
    return {n: (_f64(t) if t is not None and t.dtype == torch.bfloat16 else t) for n, t in x.items()}


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.mark.parametrize("normed", [True, False])
def test_bwd_matches_torch_autograd(normed):
    x = _inputs([5, 7, 1, 33], 3, seed=3, normed=normed)
    eps, scale = workloads.EPS, D ** -0.5
    q = _t64(x["q"]).requires_grad_()
    k = _t64(x["k"]).requires_grad_()
    v = _t64(x["v"]).requires_grad_()
    wq = _t64(x["wq"]).requires_grad_() if normed else None
    wk = _t64(x["wk"]).requires_grad_() if normed else None
    out = _torch_node(q, k, v, x["seg"].numpy(), wq, wk, eps, scale)
    go = _t64(x["dout"])
    (out * go).sum().backward()
    dq, dk, dv, dwq, dwk = oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"], x["wq"], x["wk"], eps, scale)
    for name, a, b in (("dq", dq, q.grad), ("dk", dk, k.grad), ("dv", dv, v.grad)):
        assert _rel(a, b.numpy()) < 1e-12, name
    if normed:
        assert _rel(dwq, wq.grad.numpy()) < 1e-12 and _rel(dwk, wk.grad.numpy()) < 1e-12
    else:
        assert dwq is None and dwk is None


def test_bwd_finite_differences_smooth():
    """round_operands=False: the exact gradient of a smooth FP64 function, checked by central
    differences of an independent torch forward along random directions."""
    x = _inputs([9, 6, 13], 2, seed=11, w_scale=2.0)
    eps, scale = workloads.EPS, 0.3
    seg = x["seg"].numpy()
    dq, dk, dv, dwq, dwk = oracle.bwd(x["q"], x["k"], x["v"], seg, x["dout"], x["wq"], x["wk"], eps, scale,
                                      round_operands=False)
    base = {n: _t64(x[n]) for n in ("q", "k", "v", "wq", "wk")}
    go = _t64(x["dout"])
    grads = {"q": dq, "k": dk, "v": dv, "wq": dwq, "wk": dwk}
    rng = np.random.default_rng(0)

    def loss(p):
        with torch.no_grad():
            o = _torch_node(p["q"], p["k"], p["v"], seg, p["wq"], p["wk"], eps, scale, straight_through=False)
            return float((o * go).sum())

    for name in grads:
        for _ in range(3):
            u = torch.from_numpy(rng.standard_normal(base[name].shape))
            h = 1e-5
            pp = dict(base)
            pp[name] = base[name] + h * u
            lp = loss(pp)
            pp[name] = base[name] - h * u
            lm = loss(pp)
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(grads[name] * u.numpy()))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_bwd_single_key_segments_closed_form():
    """P = 1 for a one-key segment: dV = dO and dS = 0, so dq = dk = 0 and the weights get nothing."""
    x = _inputs([1, 1, 1, 1], 3, seed=4)
    dq, dk, dv, dwq, dwk = oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"], x["wq"], x["wk"])
    assert np.array_equal(dv, oracle.bf16_to_f64(x["dout"]))
    assert not np.any(dq) and not np.any(dk) and not np.any(dwq) and not np.any(dwk)


def test_bwd_sum_rules():
    """Without the norm: shifting every key of a segment by the same vector leaves P unchanged, so
    sum_j dk_j = 0; and sum_j dV_j = sum_i dO_i because every row of P sums to one."""
    x = _inputs([37, 1, 64], 2, seed=8, normed=False)
    dq, dk, dv, _, _ = oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"])
    go = oracle.bf16_to_f64(x["dout"])
    starts, lens = oracle.segments(x["seg"].numpy())
    for s0, L in zip(starts, lens):
        sl = slice(int(s0), int(s0 + L))
        scale_k = np.abs(dk[sl]).sum(0) + 1e-300
        assert np.all(np.abs(dk[sl].sum(0)) <= 1e-12 * scale_k)
        assert np.allclose(dv[sl].sum(0), go[sl].sum(0), rtol=1e-12, atol=1e-12)


def test_bwd_linear_in_dout_exactly():
    x = _inputs([20, 11], 2, seed=5)
    seg = x["seg"].numpy()
    a = oracle.bwd(x["q"], x["k"], x["v"], seg, x["dout"], x["wq"], x["wk"])
    d2 = oracle.f64_to_bf16(2.0 * oracle.bf16_to_f64(x["dout"]))  # exact: a power of two
    b = oracle.bwd(x["q"], x["k"], x["v"], seg, d2, x["wq"], x["wk"])
    for u, w in zip(a, b):
        assert np.array_equal(2.0 * u, w)


def test_bwd_segment_locality():
    """Gradients of one segment do not depend on another segment's q, k, v or dO."""
    x = _inputs([30, 17], 2, seed=6)
    seg = x["seg"].numpy()
    a = oracle.bwd(x["q"], x["k"], x["v"], seg, x["dout"], x["wq"], x["wk"])
    y = {n: x[n].copy() for n in ("q", "k", "v", "dout")}
    rng = np.random.default_rng(1)
    for n in y:
        y[n][30:] = oracle.f64_to_bf16(rng.standard_normal(y[n][30:].shape))
    b = oracle.bwd(y["q"], y["k"], y["v"], seg, y["dout"], x["wq"], x["wk"])
    for u, w in zip(a[:3], b[:3]):
        assert np.array_equal(u[:30], w[:30])


def test_bwd_operand_rounding_is_straight_through():
    """Rounded and unrounded operands give gradients that differ only at the bf16 rounding level."""
    x = _inputs([40, 24], 2, seed=9)
    seg = x["seg"].numpy()
    a = oracle.bwd(x["q"], x["k"], x["v"], seg, x["dout"], x["wq"], x["wk"])
    b = oracle.bwd(x["q"], x["k"], x["v"], seg, x["dout"], x["wq"], x["wk"], round_operands=False)
    for u, w in zip(a, b):
        r = _rel(u, w)
        assert 0 < r < 2e-2


def test_bwd_errors():
    x = _inputs([4], 1, seed=1)
    with pytest.raises(oracle.OracleError):
        oracle.bwd(x["q"], x["k"], x["v"], np.array([1, 0, 0, 0], np.int32), x["dout"], x["wq"], x["wk"])
    with pytest.raises(oracle.OracleError):
        oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"], x["wq"], None)
