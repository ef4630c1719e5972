"""Pins of the oracle's MM-RoPE step (CPU only).

The rope node between the norm and the attention rotates 96 of 128 channels ("ws1_one_h3_block +
full-model qualification" page, Bindings table: rope_q/rope_k; Tests: "MM-RoPE rotates 96 of 128
channels").  The pages give neither the axis split nor the frequencies, so the node is table-driven
(per-token cosines and sines of the 48 rotated pairs) and pairs channels (2i, 2i+1).  It is pinned
here to torch's complex multiplication (a library routine), to the invariants of a rotation (pair
norms, relative position), to the identity table, and, for the backward, to torch FP64 autograd and
central differences of an independently written composite.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

D = 128
NP = 48


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _t64(bits):
    return torch.from_numpy(oracle.bf16_to_f64(bits))


def tables(T, seed, kind="random"):
    """float32 [T, 48] cosine and sine tables."""
    g = torch.Generator().manual_seed(seed)
    if kind == "identity":
        return torch.ones(T, NP), torch.zeros(T, NP)
    if kind == "quarter":  # angles that are multiples of pi/2: exact 0/+-1 entries
        k = torch.randint(0, 4, (T, NP), generator=g)
        c = torch.tensor([1.0, 0.0, -1.0, 0.0])[k]
        s = torch.tensor([0.0, 1.0, 0.0, -1.0])[k]
        return c, s
    ang = torch.rand(T, NP, generator=g, dtype=torch.float64) * 2 * math.pi
    return torch.cos(ang).float(), torch.sin(ang).float()


def torch_rope(x, c, s):
    """Rotation by complex multiplication: channels (2i, 2i+1) as the complex number x_2i + i x_2i+1,
    times cos + i sin; channels 96..127 unchanged.  x FP64 [T, H, 128]; c, s [T, 48]."""
    T, H, _ = x.shape
    xc = torch.view_as_complex(x[..., :2 * NP].reshape(T, H, NP, 2).contiguous())
    e = torch.complex(c.double(), s.double())[:, None, :]
    y = torch.view_as_real(xc * e).reshape(T, H, 2 * NP)
    return torch.cat([y, x[..., 2 * NP:]], -1)


def test_rope_matches_torch_complex_multiplication():
    x = workloads.random_inputs([37, 5], 3, seed=2)
    c, s = tables(42, seed=3)
    got = oracle.rope_f64(x["q"], c, s)
    ref = torch_rope(x["q"].double(), c, s).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-15 * max(1.0, np.max(np.abs(ref)))
    assert np.array_equal(got[..., 96:], x["q"].double().numpy()[..., 96:])  # 32 channels pass through
    assert not np.allclose(got[..., :96], x["q"].double().numpy()[..., :96])


def test_rope_scales_pair_norms_by_the_table_norm():
    x = workloads.random_inputs([30], 2, seed=4)
    c, s = tables(30, seed=5)
    y = oracle.rope_f64(x["k"], c, s)
    xd = x["k"].double().numpy()
    nx = xd[..., :96:2] ** 2 + xd[..., 1:96:2] ** 2
    ny = y[..., :96:2] ** 2 + y[..., 1:96:2] ** 2
    k = (c.double() ** 2 + s.double() ** 2).numpy()[:, None, :]  # 1 up to float32 rounding
    assert np.allclose(ny, nx * k, rtol=1e-13, atol=1e-300)


def test_identity_table_is_the_plain_node():
    x = workloads.random_inputs([50, 21, 1], 2, seed=6, with_grad=True)
    seg = x["seg"].numpy()
    c, s = tables(72, 0, "identity")
    a, la = oracle.fwd_ex(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], workloads.EPS, D ** -0.5, cos=c, sin=s)
    b, lb = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], workloads.EPS, D ** -0.5)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    ga = oracle.bwd(x["q"], x["k"], x["v"], seg, x["dout"], x["wq"], x["wk"], workloads.EPS, D ** -0.5, cos=c, sin=s)
    gb = oracle.bwd(x["q"], x["k"], x["v"], seg, x["dout"], x["wq"], x["wk"], workloads.EPS, D ** -0.5)
    for u, w in zip(ga, gb):
        assert np.array_equal(u, w)


def test_rotation_makes_scores_depend_on_relative_position_only():
    """With a 1-axis table theta_t,i = (t + shift) * omega_i in quarter turns (exact entries), moving
    every token of a segment by the same shift leaves the attention unchanged: only angle differences
    reach Q.K^T.  A mix-up of the rotation's signs or pairs breaks this."""
    L = 24
    x = workloads.random_inputs([L], 2, seed=8)
    omega = torch.randint(1, 4, (NP,), generator=torch.Generator().manual_seed(9))

    def tab(shift):
        k = ((torch.arange(L)[:, None] + shift) * omega[None, :]) % 4
        return torch.tensor([1.0, 0.0, -1.0, 0.0])[k], torch.tensor([0.0, 1.0, 0.0, -1.0])[k]

    outs = [oracle.fwd_ex(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], workloads.EPS, D ** -0.5,
                          cos=c, sin=s)[0] for c, s in (tab(0), tab(1), tab(3))]
    assert np.max(np.abs(outs[1] - outs[0])) < 1e-13 and np.max(np.abs(outs[2] - outs[0])) < 1e-13
    plain, _ = oracle.fwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], workloads.EPS, D ** -0.5)
    assert np.max(np.abs(outs[0] - plain)) > 1e-3  # the rotation does change the attention


def test_rope_forward_is_norm_then_rope_then_attention_each_rounded():
    """The operands are bf16(rope(bf16(norm(x)))): rebuilt here from the pinned norm, torch's complex
    rotation and the pinned bf16 rounding, then torch FP64 softmax attention."""
    lens = [17, 40]
    x = workloads.random_inputs(lens, 2, seed=12, w_scale=2.0)
    c, s = tables(sum(lens), seed=13)
    got, _ = oracle.fwd_ex(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], workloads.EPS, D ** -0.5,
                           cos=c, sin=s)

    def operand(t, w):
        n = _t64(oracle.qknorm(t, w, workloads.EPS))
        return _t64(oracle.f64_to_bf16(torch_rope(n, c, s).numpy()))

    qh, kh, v = operand(x["q"], x["wq"]), operand(x["k"], x["wk"]), x["v"].double()
    t0, ref = 0, []
    for L in lens:
        sl = slice(t0, t0 + L)
        p = torch.softmax(D ** -0.5 * qh[sl].transpose(0, 1) @ kh[sl].transpose(0, 1).transpose(1, 2), -1)
        ref.append((p @ v[sl].transpose(0, 1)).transpose(0, 1))
        t0 += L
    assert np.max(np.abs(got - torch.cat(ref).numpy())) < 1e-12


def _torch_node_rope(q, k, v, seg, wq, wk, c, s, eps, scale, straight_through=True):
    """FP64 composite: RMSNorm -> bf16 -> rope -> bf16 -> per-segment softmax attention, the roundings
    straight-through (identity for gradients), written independently of the oracle."""
    def st(y):
        if not straight_through:
            return y
        r = torch.from_numpy(oracle.bf16_to_f64(oracle.f64_to_bf16(y.detach().numpy())))
        return y + (r - y).detach()

    def node(x, w):
        y = st(x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * w)
        return st(torch_rope(y, c, s))

    qn, kn = node(q, wq), node(k, wk)
    starts, lens = oracle.segments(seg)
    outs = []
    for s0, L in zip(starts, lens):
        sl = slice(int(s0), int(s0 + L))
        qs, ks, vs = qn[sl].transpose(0, 1), kn[sl].transpose(0, 1), v[sl].transpose(0, 1)
        p = torch.softmax(scale * qs @ ks.transpose(1, 2), dim=-1)
        outs.append((p @ vs).transpose(0, 1))
    return torch.cat(outs, 0)


def test_rope_bwd_matches_torch_autograd():
    lens = [5, 7, 1, 33]
    x = workloads.random_inputs(lens, 3, seed=21, with_grad=True)
    c, s = tables(sum(lens), seed=22)
    eps, scale = workloads.EPS, D ** -0.5
    q = _t64(_bits(x["q"])).requires_grad_()
    k = _t64(_bits(x["k"])).requires_grad_()
    v = _t64(_bits(x["v"])).requires_grad_()
    wq = _t64(_bits(x["wq"])).requires_grad_()
    wk = _t64(_bits(x["wk"])).requires_grad_()
    out = _torch_node_rope(q, k, v, x["seg"].numpy(), wq, wk, c, s, eps, scale)
    (out * _t64(_bits(x["dout"]))).sum().backward()
    got = oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"], x["wq"], x["wk"], eps, scale, cos=c, sin=s)
    for name, a, b in zip(("dq", "dk", "dv", "dwq", "dwk"), got, (q.grad, k.grad, v.grad, wq.grad, wk.grad)):
        b = b.numpy()
        assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-12, name
    plain = oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"], x["wq"], x["wk"], eps, scale)
    assert np.linalg.norm(got[0] - plain[0]) / np.linalg.norm(plain[0]) > 1e-2  # the rotation matters


def test_rope_bwd_finite_differences_smooth():
    lens = [9, 6]
    x = workloads.random_inputs(lens, 2, seed=31, with_grad=True)
    c, s = tables(sum(lens), seed=32)
    eps, scale = workloads.EPS, 0.3
    seg = x["seg"].numpy()
    grads = oracle.bwd(x["q"], x["k"], x["v"], seg, x["dout"], x["wq"], x["wk"], eps, scale, round_operands=False,
                       cos=c, sin=s)
    base = {n: _t64(_bits(x[n])) for n in ("q", "k", "v", "wq", "wk")}
    go = _t64(_bits(x["dout"]))
    rng = np.random.default_rng(33)

    def f(pt):
        with torch.no_grad():
            return float((_torch_node_rope(pt["q"], pt["k"], pt["v"], seg, pt["wq"], pt["wk"], c, s, eps, scale,
                                           straight_through=False) * go).sum())

    for name, g in zip(("q", "k", "v", "wq", "wk"), grads):
        d = torch.from_numpy(rng.standard_normal(tuple(base[name].shape)))
        h = 1e-6
        plus = dict(base, **{name: base[name] + h * d})
        minus = dict(base, **{name: base[name] - h * d})
        fd = (f(plus) - f(minus)) / (2 * h)
        an = float((torch.from_numpy(g) * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), name


def test_rope_argument_errors():
    x = workloads.random_inputs([4], 1, seed=1, normed=False)
    c, s = tables(4, 0)
    with pytest.raises(oracle.OracleError):  # rope needs the norm weights (the fused q_norm -> rope chain)
        oracle.fwd_ex(x["q"], x["k"], x["v"], x["seg"].numpy(), None, None, cos=c, sin=s)
    with pytest.raises(ValueError):
        oracle.rope_f64(x["q"], c[:3], s[:3])
