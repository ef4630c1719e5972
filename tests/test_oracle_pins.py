"""Pins of the FP64 oracle to things other than itself (CPU only).

Every check here is independent of the oracle's own code: library routines (torch FP64 rms_norm and
scaled_dot_product_attention), a 50-digit mpmath brute force, closed forms of the softmax, and
invariants of the method (segment locality, key-permutation invariance, linearity in V).  Together
they are chosen so that a plausible slip in the oracle -- a dropped norm weight, a wrong mean
divisor or eps, a wrong softmax scale, a transposed operand, an off-by-one segment boundary, a wrong
LSE -- fails at least one of them.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
import workloads

D = 128


def f64(bits):
    return oracle.bf16_to_f64(bits)


# ----------------------------------------------------------------------------- bf16 rounding

def _bf16_vals(bits):
    return f64(np.asarray(bits, np.uint16))


def test_bf16_roundtrip_every_finite_pattern():
    b = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    finite = (b & 0x7F80) != 0x7F80
    b = b[finite]
    assert np.array_equal(oracle.f64_to_bf16(f64(b)), b)


def test_bf16_midpoints_tie_to_even():
    # positive finite patterns below the largest; the exact midpoint of b and b+1 is an FP64 value
    b = np.arange(1, 0x7F7F, dtype=np.uint16)
    lo, hi = _bf16_vals(b), _bf16_vals(b + 1)
    mid = (lo + hi) / 2.0
    r = oracle.f64_to_bf16(mid)
    expect = np.where(b % 2 == 0, b, b + 1).astype(np.uint16)
    assert np.array_equal(r, expect)
    # just above / below the midpoint go up / down regardless of parity
    assert np.array_equal(oracle.f64_to_bf16(np.nextafter(mid, np.inf)), (b + 1).astype(np.uint16))
    assert np.array_equal(oracle.f64_to_bf16(np.nextafter(mid, 0)), b)
    # negative values mirror
    assert np.array_equal(oracle.f64_to_bf16(-mid), expect | 0x8000)


def test_bf16_nearest_on_random_doubles():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000))
    r = oracle.f64_to_bf16(x)
    a = np.abs(x)
    rb = r & 0x7FFF
    val = _bf16_vals(rb)
    up = _bf16_vals(np.minimum(rb + 1, 0x7F80))
    dn = _bf16_vals(np.where(rb > 0, rb - 1, 0))
    err = np.abs(a - val)
    assert np.all(err <= np.abs(a - up)) and np.all(err <= np.abs(a - dn))
    assert np.array_equal(r >> 15, (x < 0).astype(np.uint16))


def test_bf16_overflow_and_specials():
    big = _bf16_vals(np.array([0x7F7F], np.uint16))[0]
    half_ulp = 2.0 ** 119
    r = oracle.f64_to_bf16(np.array([big + half_ulp * 0.999, big + half_ulp, np.inf, -np.inf, 0.0, -0.0, np.nan]))
    assert list(r[:6]) == [0x7F7F, 0x7F80, 0x7F80, 0xFF80, 0x0000, 0x8000]
    assert (r[6] & 0x7F80) == 0x7F80 and (r[6] & 0x7F) != 0


# ----------------------------------------------------------------------------- segments

def test_segments_runs_and_errors():
    s, l = oracle.segments(np.array([3, 3, 3, 4, 9, 9], np.int32))
    assert list(s) == [0, 3, 4] and list(l) == [3, 1, 2]
    s, l = oracle.segments(np.zeros(0, np.int32))
    assert len(s) == 0
    with pytest.raises(oracle.OracleError):
        oracle.segments(np.array([0, 1, 0], np.int32))


# ----------------------------------------------------------------------------- RMSNorm

@pytest.fixture(scope="module")
def small():
    return workloads.make_inputs(workloads.WORKLOADS["short3"])


def test_norm_matches_torch_rms_norm_fp64(small):
    x, w = small["q"][:200], small["wq"]
    ref = torch.nn.functional.rms_norm(x.double(), (D,), w.double(), eps=1e-6).numpy()
    got = oracle.rmsnorm_f64(x, w, 1e-6)
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)) < 1e-14
    # a different eps must show up (eps is honoured, not hard-wired)
    ref2 = torch.nn.functional.rms_norm(x.double(), (D,), w.double(), eps=1e-1).numpy()
    assert np.max(np.abs(oracle.rmsnorm_f64(x, w, 1e-1) - ref2)) < 1e-13


def test_norm_invariant_mean_square(small):
    x, w = small["k"][:100], small["wk"]
    y = oracle.rmsnorm_f64(x, w, 1e-6)
    xd = x.double().numpy()
    ms = (xd ** 2).mean(-1)
    lhs = ((y / w.double().numpy()) ** 2).mean(-1)
    assert np.allclose(lhs, ms / (ms + 1e-6), rtol=1e-13, atol=0)


def test_qknorm_is_one_rounding_of_fp64_norm(small):
    x, w = small["q"][:300], small["wq"]
    exact = torch.nn.functional.rms_norm(x.double(), (D,), w.double(), eps=1e-6).numpy()
    got = f64(oracle.qknorm(x, w, 1e-6))
    # within half a bf16 ulp of the library's FP64 value (ulp = 2^(e-7) for |y| in [2^e, 2^(e+1)))
    e = np.floor(np.log2(np.abs(exact)))
    assert np.all(np.abs(got - exact) <= np.exp2(e - 8) * (1 + 1e-12))


def test_qknorm_zero_row_gives_zero():
    x = torch.zeros(3, 2, D, dtype=torch.bfloat16)
    w = torch.ones(D, dtype=torch.bfloat16)
    assert np.all(oracle.qknorm(x, w, 1e-6) == 0)


# ----------------------------------------------------------------------------- attention

def _sdpa_fp64(qh, kh, v, seg, scale):
    """torch's FP64 scaled_dot_product_attention with a block-diagonal mask (a library routine)."""
    seg_t = torch.as_tensor(seg)
    mask = seg_t[:, None] == seg_t[None, :]
    q = torch.as_tensor(qh).permute(1, 0, 2).contiguous()
    k = torch.as_tensor(kh).permute(1, 0, 2).contiguous()
    vv = torch.as_tensor(v).permute(1, 0, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, vv, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("name", ["tiny", "short3"])
def test_fwd_matches_torch_sdpa_fp64(name):
    wl = workloads.WORKLOADS[name]
    x = workloads.make_inputs(wl)
    out, lse = oracle.fwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], wl.eps, wl.scale)
    qh = f64(oracle.qknorm(x["q"], x["wq"], wl.eps))
    kh = f64(oracle.qknorm(x["k"], x["wk"], wl.eps))
    ref = _sdpa_fp64(qh, kh, x["v"].double().numpy(), x["seg"].numpy(), wl.scale)
    assert np.max(np.abs(out - ref)) < 1e-12
    assert out.shape == (wl.tokens, wl.heads, D) and lse.shape == (wl.tokens, wl.heads)


def test_fwd_ragged_segments_match_sdpa():
    lens = [1, 2, 63, 64, 65, 127, 129, 3]
    x = workloads.random_inputs(lens, 3, seed=7)
    seg = x["seg"].numpy()
    out, _ = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    qh = f64(oracle.qknorm(x["q"], x["wq"], 1e-6))
    kh = f64(oracle.qknorm(x["k"], x["wk"], 1e-6))
    ref = _sdpa_fp64(qh, kh, x["v"].double().numpy(), seg, D ** -0.5)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_fwd_without_weights_uses_inputs_directly():
    x = workloads.random_inputs([40, 24], 2, seed=3, normed=False, qk_scale=0.5)
    seg = x["seg"].numpy()
    out, _ = oracle.fwd(x["q"], x["k"], x["v"], seg, None, None, 1e-6, 0.3)
    ref = _sdpa_fp64(x["q"].double().numpy(), x["k"].double().numpy(), x["v"].double().numpy(), seg, 0.3)
    assert np.max(np.abs(out - ref)) < 1e-12
    with pytest.raises(oracle.OracleError):
        oracle.fwd(x["q"], x["k"], x["v"], seg, x["q"][0, 0], None, 1e-6, 0.3)


def test_lse_normalises_the_softmax():
    """sum_j exp(s_ij - LSE_i) = 1, with s computed here from the pinned normed operands."""
    wl = workloads.WORKLOADS["short3"]
    x = workloads.make_inputs(wl)
    seg = x["seg"].numpy()
    _, lse = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], wl.eps, wl.scale)
    qh = torch.as_tensor(f64(oracle.qknorm(x["q"], x["wq"], wl.eps)))
    kh = torch.as_tensor(f64(oracle.qknorm(x["k"], x["wk"], wl.eps)))
    starts, lens = oracle.segments(seg)
    for s0, L in zip(starts, lens):
        q_s, k_s = qh[s0:s0 + L].permute(1, 0, 2), kh[s0:s0 + L].permute(1, 0, 2)
        s = torch.matmul(q_s, k_s.transpose(1, 2)) * wl.scale            # [H, L, L]
        tot = torch.exp(s - torch.as_tensor(lse[s0:s0 + L]).T[:, :, None]).sum(-1)
        assert torch.max(torch.abs(tot - 1)).item() < 1e-13


def _round_bf16_mp(y):
    """Exact round-to-nearest-even of an mpmath value to bf16 (independent of the oracle's rounding)."""
    if y == 0:
        return mpmath.mpf(0)
    a = abs(y)
    e = int(mpmath.floor(mpmath.log(a, 2)))
    # guard against log rounding at exact powers of two
    if mpmath.mpf(2) ** e > a:
        e -= 1
    elif mpmath.mpf(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = mpmath.mpf(2) ** (e - 7)
    z = a / ulp
    f = mpmath.floor(z)
    d = z - f
    if d > 0.5 or (d == 0.5 and int(f) % 2 == 1):
        f += 1
    r = f * ulp
    return r if y > 0 else -r


def test_fwd_brute_force_mpmath_tiny():
    """Every step of the tiny workload at 50 digits: norm, one bf16 rounding, softmax, P.V."""
    wl = workloads.WORKLOADS["tiny"]
    x = workloads.make_inputs(wl)
    seg = x["seg"].numpy()
    out, lse = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], wl.eps, wl.scale)
    mpmath.mp.dps = 50
    T, H = wl.tokens, wl.heads
    q, k, v = (x[n].double().numpy() for n in ("q", "k", "v"))
    wq, wk = x["wq"].double().numpy(), x["wk"].double().numpy()
    eps, scale = mpmath.mpf(wl.eps), mpmath.mpf(wl.scale)

    def norm(row, w):
        ms = mpmath.fsum(mpmath.mpf(a) ** 2 for a in row) / D
        r = 1 / mpmath.sqrt(ms + eps)
        return [_round_bf16_mp(mpmath.mpf(a) * r * mpmath.mpf(b)) for a, b in zip(row, w)]

    qh = [[norm(q[t, h], wq) for h in range(H)] for t in range(T)]
    kh = [[norm(k[t, h], wk) for h in range(H)] for t in range(T)]
    starts, lens = oracle.segments(seg)
    worst = 0.0
    for s0, L in zip(starts, lens):
        for h in range(H):
            for i in range(s0, s0 + L):
                s = [scale * mpmath.fsum(a * b for a, b in zip(qh[i][h], kh[j][h])) for j in range(s0, s0 + L)]
                m = max(s)
                e = [mpmath.exp(sj - m) for sj in s]
                l = mpmath.fsum(e)
                for d in range(D):
                    o = mpmath.fsum(e[jj] * mpmath.mpf(v[s0 + jj, h, d]) for jj in range(L)) / l
                    # absolute error against O(1) terms (relative error is meaningless where o cancels to ~0)
                    worst = max(worst, abs(float(o) - out[i, h, d]) / max(abs(float(o)), 1.0))
                assert abs(float(m + mpmath.log(l)) - lse[i, h]) < 1e-14
    assert worst < 1e-14


def test_identical_keys_give_mean_of_v():
    x = workloads.random_inputs([37, 50], 2, seed=11)
    k = x["k"].clone()
    k[37:] = k[37]                      # every key of segment 1 identical (per head)
    seg = x["seg"].numpy()
    out, _ = oracle.fwd(x["q"], k, x["v"], seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    mean_v = x["v"][37:].double().numpy().mean(0)
    assert np.max(np.abs(out[37:] - mean_v[None])) < 1e-14
    # and a zero query row: uniform softmax over its own segment
    q = x["q"].clone()
    q[5] = 0
    out2, _ = oracle.fwd(q, x["k"], x["v"], seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    assert np.max(np.abs(out2[5] - x["v"][:37].double().numpy().mean(0))) < 1e-14


def test_single_key_segment_returns_its_v_exactly():
    x = workloads.random_inputs([4, 1, 6, 1], 3, seed=2)
    seg = x["seg"].numpy()
    out, lse = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    v = x["v"].double().numpy()
    assert np.array_equal(out[4], v[4]) and np.array_equal(out[11], v[11])
    qh = f64(oracle.qknorm(x["q"], x["wq"], 1e-6))
    kh = f64(oracle.qknorm(x["k"], x["wk"], 1e-6))
    assert np.allclose(lse[4], D ** -0.5 * (qh[4] * kh[4]).sum(-1), rtol=1e-14, atol=1e-15)


def test_key_permutation_within_segment_is_invariant():
    x = workloads.random_inputs([90, 70], 2, seed=4)
    seg = x["seg"].numpy()
    out, lse = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    perm = torch.cat([torch.randperm(90, generator=torch.Generator().manual_seed(1)), torch.arange(90, 160)])
    k2, v2 = x["k"].clone(), x["v"].clone()
    k2[:] = x["k"][perm]
    v2[:] = x["v"][perm]
    out2, lse2 = oracle.fwd(x["q"], k2, v2, seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    # FP64 sums in a different order: absolute error of order L * 1e-16 against O(1) terms
    assert np.max(np.abs(out2 - out)) < 1e-13
    assert np.max(np.abs(lse2 - lse)) < 1e-13


def test_no_attention_across_segments():
    x = workloads.random_inputs([33, 40, 29], 2, seed=6)
    seg = x["seg"].numpy()
    out, lse = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    y = {n: x[n].clone() for n in ("q", "k", "v")}
    for n in y:
        y[n][33:73] = torch.randn(40, 2, D).to(torch.bfloat16) * 7   # rewrite the middle segment
        y[n][40, 1, 3] = float("nan")
    out2, lse2 = oracle.fwd(y["q"], y["k"], y["v"], seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    assert np.array_equal(out2[:33], out[:33]) and np.array_equal(out2[73:], out[73:])
    assert np.array_equal(lse2[:33], lse[:33]) and np.array_equal(lse2[73:], lse[73:])


def test_linear_in_v_and_heads_independent():
    x = workloads.random_inputs([50, 21], 4, seed=8)
    seg = x["seg"].numpy()
    out, _ = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    out4, _ = oracle.fwd(x["q"], x["k"], x["v"] * 4, seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    assert np.array_equal(out4, out * 4)
    hp = torch.tensor([2, 0, 3, 1])
    outp, _ = oracle.fwd(x["q"][:, hp], x["k"][:, hp], x["v"][:, hp], seg, x["wq"], x["wk"], 1e-6, D ** -0.5)
    assert np.array_equal(outp, out[:, hp.numpy()])


def test_fwd_rows_equals_full_fwd():
    wl = workloads.WORKLOADS["short3"]
    x = workloads.make_inputs(wl)
    seg = x["seg"].numpy()
    out, lse = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], wl.eps, wl.scale)
    rows = np.array([0, 299, 300, 601, 924, 5])
    o2, l2 = oracle.fwd_rows(x["q"], x["k"], x["v"], seg, rows, x["wq"], x["wk"], wl.eps, wl.scale)
    assert np.array_equal(o2, out[rows]) and np.array_equal(l2, lse[rows])


def test_decreasing_ids_rejected_and_empty_ok():
    x = workloads.random_inputs([3, 3], 1, seed=1)
    bad = np.array([0, 0, 1, 1, 0, 1], np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.fwd(x["q"], x["k"], x["v"], bad, x["wq"], x["wk"])
    e = torch.zeros(0, 2, D, dtype=torch.bfloat16)
    out, lse = oracle.fwd(e, e, e, np.zeros(0, np.int32), x["wq"], x["wk"])
    assert out.shape == (0, 2, D) and lse.shape == (0, 2)


def test_tiny_golden_regression():
    """The oracle still reproduces its committed outputs for the tiny workload (inputs pinned by sha256)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    with open(path) as f:
        doc = json.load(f)
    wl = workloads.WORKLOADS["tiny"]
    x = workloads.make_inputs(wl)
    for n, h in doc["sha256"].items():
        assert workloads.sha256(x[n]) == h, f"input {n} changed"
    out, lse = oracle.fwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], wl.eps, wl.scale)
    assert np.max(np.abs(lse - np.array(doc["lse"]))) < 1e-15
    assert np.max(np.abs(out[:, :, :8] - np.array(doc["out_first8"]))) < 1e-15


@pytest.mark.parametrize("normed", [True, False])
def test_fwd_opt_unrounded_matches_sdpa_on_fp64_rms_norm(normed):
    """The "pure" forward (normed operands kept in FP64, not rounded to bf16) against torch's FP64
    rms_norm followed by its FP64 scaled_dot_product_attention with a block-diagonal mask (both
    library routines), on ragged segments; with round_operands it is the node-faithful forward."""
    lens = [1, 2, 63, 97, 130, 5, 64]
    x = workloads.random_inputs(lens, 3, seed=41, normed=normed, w_scale=2.0)
    seg = x["seg"].numpy()
    scale = D ** -0.5
    got = oracle.fwd_opt(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], 1e-6, scale, round_operands=False)
    if normed:
        qh = torch.nn.functional.rms_norm(x["q"].double(), (D,), x["wq"].double(), eps=1e-6).numpy()
        kh = torch.nn.functional.rms_norm(x["k"].double(), (D,), x["wk"].double(), eps=1e-6).numpy()
    else:
        qh, kh = x["q"].double().numpy(), x["k"].double().numpy()
    ref = _sdpa_fp64(qh, kh, x["v"].double().numpy(), seg, scale)
    assert np.max(np.abs(got - ref)) < 1e-12
    rounded = oracle.fwd_opt(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], 1e-6, scale, round_operands=True)
    full, _ = oracle.fwd(x["q"], x["k"], x["v"], seg, x["wq"], x["wk"], 1e-6, scale)
    assert np.array_equal(rounded, full)
    if normed:  # the two differ by the operands' rounding: the unrounded form is not a copy of fwd
        assert np.max(np.abs(got - full)) > 1e-6
    else:
        assert np.array_equal(got, full)
