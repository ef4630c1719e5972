"""The backward (h3attn_bwd) on the GPU: parity of dq, dk, dv and the norm-weight gradients with the
FP64 oracle, and its bitwise properties (repeat, one row alone vs batched, segment offset).

Bound (whole gradient tensors, bf16 upcast exactly): relative L2 <= 2e-3 and max abs <= 2e-2 *
max(1, max |oracle|) for dq, dk, dv; relative L2 <= 2e-3 for dwq, dwk (fp32).  The max-abs bound is
the forward's (whose outputs are O(1)) scaled by the gradient's largest magnitude: gradients of a
sharp softmax reach ~40, where one bf16 rounding alone moves a value by up to 0.125.  The oracle
evaluates the gradients at the rounded normed operands with the rounding as the identity
(straight-through), the definition the kernels implement.  The full config-5 shape (2 x 4253 tokens,
40 heads) is compared on every head and on both weight gradients, in both ways of forming D."""
import functools

import numpy as np
import pytest
import torch

import deterministic_invariant_attention_amd as h3
import oracle
import workloads
from gpu_util import EPS, MAX_ABS_BOUND, REL_L2_BOUND, bitwise_equal, digest, f64, metrics, run_fwd, say, to_dev

pytestmark = pytest.mark.gpu
SCALE = 128 ** -0.5
# How D_i = sum_j P_ij dP_ij is formed: recomputed by the dq kernel (h3attn_bwd), or dO . O from the
# forward's fp32 output (h3attn_fwd_ex / h3attn_bwd_ex with o32).  Every property holds for both.
DMODES = ["recompute", "o32"]


def run_bwd(g, weights=True, eps=EPS, scale=SCALE, dmode="recompute"):
    wq, wk = (g["wq"], g["wk"]) if weights else (None, None)
    if dmode == "o32":
        _, lse, o32 = h3.h3attn_fwd_ex(g["q"], g["k"], g["v"], g["seg"], None, wq, wk, eps=eps, scale=scale,
                                       want_lse=True, want_o32=True)
        res = h3.h3attn_bwd_ex(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], None, o32, wq, wk, eps=eps,
                               scale=scale)
    else:
        _, lse = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], wq, wk, eps=eps, scale=scale, want_lse=True)
        res = h3.h3attn_bwd(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], wq, wk, eps=eps, scale=scale)
    torch.cuda.synchronize()
    return res


@functools.lru_cache(maxsize=1)
def _oracle_workload_bwd(name):
    """The oracle's gradients of a configured workload (cached: both D modes compare against them)."""
    wl = workloads.WORKLOADS[name]
    x = workloads.make_inputs(wl, with_grad=True)
    say(f"[bwd parity] oracle gradients of {name} (T={wl.tokens} H={wl.heads}, all heads)")
    return oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"], x["wq"], x["wk"], wl.eps, wl.scale)


def _check(name, x, heads=None, weights=True, eps=EPS, scale=SCALE, dmode="recompute", ref=None, abs_rel=False):
    g = to_dev(x)
    T, H = x["q"].shape[0], x["q"].shape[1]
    say(f"[bwd parity] {name} ({dmode}): T={T} H={H} heads={'all' if heads is None else heads}")
    dq, dk, dv, dwq, dwk = run_bwd(g, weights=weights, eps=eps, scale=scale, dmode=dmode)
    hs = slice(None) if heads is None else list(heads)
    sub = {n: (x[n][:, hs].contiguous() if n in ("q", "k", "v", "dout") else x[n]) for n in x}
    wq, wk = (x["wq"], x["wk"]) if weights else (None, None)
    if ref is None:
        ref = oracle.bwd(sub["q"], sub["k"], sub["v"], x["seg"].numpy(), sub["dout"], wq, wk, eps, scale)
    res, mag = {}, {}
    for nm, a, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        a = a[:, hs]
        assert np.all(np.isfinite(f64(a))), nm
        res[nm] = metrics(a, r)
        mag[nm] = (float(np.abs(r).max()) if abs_rel else max(1.0, float(np.abs(r).max()))) if r.size else 1.0
    if weights and heads is None:
        for nm, a, r in (("dwq", dwq, ref[3]), ("dwk", dwk, ref[4])):
            res[nm] = (float(np.linalg.norm(a.cpu().double().numpy() - r) / np.linalg.norm(r)), 0.0)
    say(f"[bwd parity] {name}: " + " ".join(f"{k}: rel_l2={v[0]:.3e} max_abs={v[1]:.3e}" for k, v in res.items()))
    for nm, (rel, mx) in res.items():
        assert rel <= REL_L2_BOUND, nm
        assert mx <= MAX_ABS_BOUND * mag.get(nm, 1.0), nm
    return dq, dk, dv


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_parity_tiny(dmode):
    _check("tiny", workloads.make_inputs(workloads.WORKLOADS["tiny"], with_grad=True), dmode=dmode)


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_parity_ragged(dmode):
    """Segment lengths around the 64-row tiles and the 128-row work items, single-token segments."""
    lens = [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 3, 1, 257]
    _check("ragged", workloads.random_inputs(lens, 3, seed=31, with_grad=True), dmode=dmode)


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_parity_short3(dmode):
    _check("short3", workloads.make_inputs(workloads.WORKLOADS["short3"], with_grad=True), dmode=dmode)


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_parity_without_weights(dmode):
    _check("no-norm", workloads.random_inputs([150, 77], 2, seed=12, normed=False, with_grad=True), weights=False,
           dmode=dmode)


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_parity_sharp_softmax(dmode):
    """Norm weights x3 (max logit ~50): the case where D from the rounded forward output would fail."""
    _check("sharp-w3", workloads.random_inputs([500, 130], 2, seed=13, w_scale=3.0, with_grad=True), dmode=dmode)


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_parity_many_segments(dmode):
    """300 segments of random lengths 1..100 (every cost class of the work order, many items per
    class), 2 heads, against the oracle."""
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(1, 101, 300)]
    _check("many-segments", workloads.random_inputs(lens, 2, seed=42, with_grad=True), dmode=dmode)


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_parity_other_scale_and_eps(dmode):
    x = workloads.random_inputs([150, 90], 2, seed=9, with_grad=True)
    _check("scale0.2-eps1e-3", x, eps=float(np.float32(1e-3)), scale=0.2, dmode=dmode)


def test_bwd_empty_input_is_a_noop():
    x = workloads.random_inputs([4], 2, seed=1, with_grad=True)
    g = to_dev(x)
    e = {n: (t[:0].contiguous() if n in ("q", "k", "v", "dout", "seg") else t) for n, t in g.items()}
    lse = torch.empty(0, 2, dtype=torch.float32, device=g["q"].device)
    dq, dk, dv, dwq, dwk = h3.h3attn_bwd(e["dout"], e["q"], e["k"], e["v"], lse, e["seg"], e["wq"], e["wk"], eps=EPS)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and dk.numel() == 0 and dv.numel() == 0


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_parity_batch2_full(dmode):
    """Config 5 (2 x 4253 tokens, 40 heads) at full size: dq, dk, dv on every head and both norm-weight
    gradients (sums over every token and head) against the oracle."""
    _check("batch2", workloads.make_inputs(workloads.WORKLOADS["batch2"], with_grad=True), dmode=dmode,
           ref=_oracle_workload_bwd("batch2"))


@functools.lru_cache(maxsize=1)
def _long_segment_inputs():
    x = workloads.random_inputs([8349], 2, seed=7100, qk_scale=3.0, with_grad=True)
    say("[bwd parity] oracle gradients of one 8349-token segment (H=2)")
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"], x["wq"], x["wk"], EPS, SCALE)
    return x, ref


def test_bwd_32768_token_segment_alone_equals_batched():
    """A 32768-token segment (512 query and key tiles per item) alone and between two others, packed
    at an offset: dq, dk, dv of its rows are the same bits, and a repeat of the batch gives the
    same bits (no oracle at this length)."""
    lens = [300, 32768, 200]
    x = workloads.random_inputs(lens, 1, seed=7200, with_grad=True)
    g = to_dev(x)
    say("[bwd bitwise] 32768-token segment alone vs between two others, and a repeat")
    b = run_bwd(g, dmode="o32")
    b2 = run_bwd(g, dmode="o32")
    for u, w in zip(b, b2):
        assert bitwise_equal(u, w)
    s0, s1 = lens[0], lens[0] + lens[1]
    alone = {n: (g[n][s0:s1].contiguous() if n in ("q", "k", "v", "seg", "dout") else g[n]) for n in g}
    a = run_bwd(alone, dmode="o32")
    for nm, u, w in (("dq", a[0], b[0]), ("dk", a[1], b[1]), ("dv", a[2], b[2])):
        assert np.all(np.isfinite(f64(u))), nm
        assert bitwise_equal(u, w[s0:s1]), nm


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_parity_long_segment(dmode):
    """One segment of the headline forward's length (8349 tokens, q/k drawn as there), 2 heads: every
    work item of both attention kernels walks 131 tiles, and P ~ 1e-4 stays in fp16's normal range.
    All outputs and both weight gradients against the oracle."""
    x, ref = _long_segment_inputs()
    _check("long-segment", x, dmode=dmode, ref=ref)


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_repeat_bitwise(dmode):
    g = to_dev(workloads.make_inputs(workloads.WORKLOADS["short3"], with_grad=True))
    say(f"[bwd bitwise] short3 repeat x5 ({dmode})")
    ref = [digest(t) for t in run_bwd(g, dmode=dmode)]
    for _ in range(4):
        assert [digest(t) for t in run_bwd(g, dmode=dmode)] == ref


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_repeat_bitwise_batch2(dmode):
    """Full config-5 size, all five outputs: many tiles per item, so a wave that read a 64-row tile
    before another wave's copy of it had landed would show up as differing bits."""
    g = to_dev(workloads.make_inputs(workloads.WORKLOADS["batch2"], with_grad=True))
    say(f"[bwd bitwise] batch2 repeat x3 ({dmode})")
    ref = [digest(t) for t in run_bwd(g, dmode=dmode)]
    for _ in range(2):
        assert [digest(t) for t in run_bwd(g, dmode=dmode)] == ref


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_batch2_alone_equals_batched(dmode):
    """Each packed row's dq, dk, dv are the same bits alone as inside the batch (rollout vs train)."""
    wl = workloads.WORKLOADS["batch2"]
    g = to_dev(workloads.make_inputs(wl, with_grad=True))
    say(f"[bwd bitwise] batch2 alone vs batched ({dmode})")
    bq, bk, bv, _, _ = run_bwd(g, dmode=dmode)
    for (t0, t1) in workloads.row_slices(wl):
        alone = {n: (g[n][t0:t1].contiguous() if n in ("q", "k", "v", "seg", "dout") else g[n]) for n in g}
        q, k, v, _, _ = run_bwd(alone, dmode=dmode)
        assert bitwise_equal(q, bq[t0:t1]) and bitwise_equal(k, bk[t0:t1]) and bitwise_equal(v, bv[t0:t1])


@pytest.mark.parametrize("dmode", DMODES)
@pytest.mark.parametrize("pad", [1, 64, 127])
def test_bwd_leading_segment_offset_invariance(pad, dmode):
    x = workloads.random_inputs([300, 129, 64], 3, seed=17, with_grad=True)
    g = to_dev(x)
    say(f"[bwd bitwise] offset shift by a {pad}-token leading segment")
    base = run_bwd(g, dmode=dmode)[:3]
    d = workloads.random_inputs([pad], 3, seed=99, with_grad=True)
    sh = {n: torch.cat([d[n].to(g[n].device), g[n]]) for n in ("q", "k", "v", "dout")}
    sh["seg"] = torch.cat([torch.full((pad,), -1, dtype=torch.int32), x["seg"]]).to(g["seg"].device)
    sh["wq"], sh["wk"] = g["wq"], g["wk"]
    shifted = run_bwd(sh, dmode=dmode)[:3]
    for a, b in zip(shifted, base):
        assert bitwise_equal(a[pad:], b)


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_nan_neighbour_does_not_leak(dmode):
    x = workloads.random_inputs([40, 70, 33], 2, seed=5, with_grad=True)
    g = to_dev(x)
    base = run_bwd(g, dmode=dmode)[:3]
    y = {n: g[n].clone() for n in g}
    for n in ("q", "k", "v", "dout"):
        y[n][40:110] = float("nan")
    got = run_bwd(y, dmode=dmode)[:3]
    for a, b in zip(got, base):
        assert bitwise_equal(a[:40], b[:40]) and bitwise_equal(a[110:], b[110:])


@pytest.mark.parametrize("dmode", DMODES)
@pytest.mark.parametrize("dscale", [1e-6, 1e-8, 1e-30, 1e6])
def test_bwd_parity_small_and_large_dout(dscale, dmode):
    """dO far from N(0, 1): bf16 draws times 1e-6, 1e-8, 1e-30 (below fp16's whole range) and 1e6
    (beyond it).  The staging scales each (segment, head) of dO by a power of two before the fp16
    products and the epilogues remove it, so the gradients keep the accuracy of the N(0, 1) case.
    The max-abs bound is relative to the gradient's own largest magnitude here."""
    x = workloads.random_inputs([300, 129, 1, 64], 3, seed=71, with_grad=True)
    x["dout"] = (x["dout"].float() * dscale).to(torch.bfloat16)
    _check(f"dout x{dscale:g}", x, dmode=dmode, abs_rel=True)


@pytest.mark.parametrize("dmode", DMODES)
def test_bwd_dout_power_of_two_scales_every_gradient_exactly(dmode):
    """Every gradient is linear in dO, and the staging's power of two cancels exactly: dO 2^k gives
    dq, dk, dv, dwq, dwk times 2^k bit for bit (while the results stay normal numbers)."""
    x = workloads.random_inputs([200, 77, 5], 2, seed=72, with_grad=True)
    g = to_dev(x)
    say(f"[bwd bitwise] dO times powers of two ({dmode})")
    base = run_bwd(g, dmode=dmode)
    for k in (-100, -24, 20):
        gk = dict(g, dout=(g["dout"].float() * 2.0 ** k).to(torch.bfloat16))
        got = run_bwd(gk, dmode=dmode)
        for nm, a, b in zip(("dq", "dk", "dv", "dwq", "dwk"), got, base):
            expect = (b.float() * 2.0 ** k).to(b.dtype)
            assert bitwise_equal(a, expect), f"{nm} at 2^{k}"


def test_bwd_large_dout_is_scaled_and_v_out_of_range_sets_status():
    """A dO of 1e6 (beyond fp16) is scaled into range and gives correct gradients with status OK; a v
    beyond the fp16 range still cannot enter the products and sets ERR_RANGE (NaN outputs)."""
    x = workloads.random_inputs([20], 2, seed=6, with_grad=True)
    x["dout"][3, 1, 7] = 1e6
    g = to_dev(x)
    _, lse = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], g["wq"], g["wk"], eps=EPS, want_lse=True)
    T, H = x["q"].shape[:2]
    ws = h3.bwd_workspace(T, H, g["q"].device)
    dq, dk, dv, dwq, dwk = h3.h3attn_bwd(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], g["wq"], g["wk"], eps=EPS,
                                         workspace_buf=ws)
    torch.cuda.synchronize()
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_OK
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"], x["wq"], x["wk"], EPS, SCALE)
    for nm, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        rel, mx = metrics(a, r)
        assert rel <= REL_L2_BOUND and mx <= MAX_ABS_BOUND * float(np.abs(r).max()), nm
    g["v"][5, 0, 2] = 7.0e4
    dq, dk, dv, dwq, dwk = h3.h3attn_bwd(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], g["wq"], g["wk"], eps=EPS,
                                         workspace_buf=ws)
    torch.cuda.synchronize()
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_ERR_RANGE
    for t in (dq, dk, dv, dwq, dwk):
        assert torch.isnan(t.float()).all()


def test_fwd_ex_o32_is_the_output_before_its_rounding():
    """o32 rounds (RNE) to exactly the bf16 output, in packed and in position order, and changes no
    bit of out or lse."""
    lens = [300, 129, 64, 1]
    x = workloads.random_inputs(lens, 3, seed=61)
    g = to_dev(x)
    say("[fwd_ex] o32 vs out")
    out, lse = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], g["wq"], g["wk"], eps=EPS, want_lse=True)
    out2, lse2, o32 = h3.h3attn_fwd_ex(g["q"], g["k"], g["v"], g["seg"], None, g["wq"], g["wk"], eps=EPS,
                                       want_lse=True, want_o32=True)
    pos = workloads.position_ids(lens).cuda()
    out3, lse3, o32b = h3.h3attn_fwd_ex(g["q"], g["k"], g["v"], g["seg"], pos, g["wq"], g["wk"], eps=EPS,
                                        want_lse=True, want_o32=True)
    torch.cuda.synchronize()
    assert bitwise_equal(out, out2) and bitwise_equal(lse, lse2) and bitwise_equal(out, out3)
    assert bitwise_equal(o32.to(torch.bfloat16), out)
    assert torch.equal(o32, o32b)
    ref, _ = oracle.fwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], EPS, SCALE)
    rel, mx = metrics(o32, ref)
    say(f"[fwd_ex] o32 vs oracle: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2_BOUND and mx <= MAX_ABS_BOUND


def test_fwd_ex_o32_nan_filled_on_data_error():
    """A value beyond fp16 in segment 0: its rows of o32 and out are NaN, segment 1's are computed."""
    x = workloads.random_inputs([40, 40], 2, seed=53)
    x["v"][10, 1, 5] = 1.0e5
    g = to_dev(x)
    ws = h3.workspace(80, 2, "cuda:0")
    out, lse, o32 = h3.h3attn_fwd_ex(g["q"], g["k"], g["v"], g["seg"], None, g["wq"], g["wk"], eps=EPS,
                                     want_lse=True, want_o32=True, workspace_buf=ws)
    torch.cuda.synchronize()
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_ERR_RANGE
    assert torch.isnan(o32[:40]).all() and torch.isnan(out[:40].float()).all()
    assert torch.isfinite(o32[40:]).all() and bitwise_equal(o32[40:].to(torch.bfloat16), out[40:])


def test_bwd_out_of_range_fails_its_own_segment_only():
    """A v beyond fp16 in the middle segment: the backward's rows of that segment are NaN, the other
    segments' dq, dk, dv keep the bits of a clean run (and of each segment alone); dwq / dwk, sums
    over the whole batch, are NaN."""
    x = workloads.random_inputs([50, 60, 70], 2, seed=79, with_grad=True)
    g = to_dev(x)
    clean = {dm: run_bwd(g, dmode=dm) for dm in DMODES}
    g["v"][70, 1, 3] = 9.0e4
    say("[bwd status] |v| > 65504 in segment 1")
    for dmode in DMODES:
        got = run_bwd(g, dmode=dmode)
        for t in got[:3]:
            assert torch.isnan(t[50:110].float()).all()
        for t in got[3:]:
            assert torch.isnan(t).all()
        for t0, t1 in ((0, 50), (110, 180)):
            alone = {n: (g[n][t0:t1].contiguous() if n in ("q", "k", "v", "seg", "dout") else g[n]) for n in g}
            a = run_bwd(alone, dmode=dmode)
            for t, c, cl in zip(got[:3], a[:3], clean[dmode][:3]):
                assert bitwise_equal(t[t0:t1], cl[t0:t1])
                assert bitwise_equal(t[t0:t1], c)


def test_bwd_flagged_segments_in_a_multi_round_walk():
    """48 segments x 8 heads: over a thousand backward items for the dq and dk/dv workgroups, taken
    from their counters.  Four segments scattered over the work order hold a v beyond fp16: their
    rows of dq, dk and dv are NaN, every other row keeps the bits of a clean run."""
    rng = np.random.default_rng(93)
    lens = [int(n) for n in rng.integers(150, 700, size=48)]
    g = to_dev(workloads.random_inputs(lens, 8, seed=94, with_grad=True))
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    clean = run_bwd(g, dmode="o32")
    bad = [3, 17, 30, 46]
    for sgi in bad:
        g["v"][int(starts[sgi]) + 5, 3, 7] = 9.0e4
    say(f"[bwd status] {sum(lens)} tokens x 8 heads, |v| > 65504 in segments {bad}")
    got = run_bwd(g, dmode="o32")
    flagged = np.zeros(sum(lens), dtype=bool)
    for sgi in bad:
        flagged[starts[sgi]:starts[sgi] + lens[sgi]] = True
    fl = torch.from_numpy(flagged).to(got[0].device)
    for t, c in zip(got[:3], clean[:3]):
        assert torch.isnan(t[fl].float()).all()
        assert bitwise_equal(t[~fl], c[~fl])


def test_bwd_long_batch_past_the_decode_prefetch_alone_equals_batched():
    """The backward's segment decode on 20100 tokens (its chunked path) against each segment alone
    (the prefetched path): dq, dk, dv are the same bits."""
    lens = [9000, 7000, 4100]
    g = to_dev(workloads.random_inputs(lens, 2, seed=73, with_grad=True))
    say(f"[bwd bitwise] {sum(lens)}-token batch vs its segments alone")
    bq, bk, bv, _, _ = run_bwd(g, dmode="o32")
    t0 = 0
    for n in lens:
        alone = {k: (g[k][t0:t0 + n].contiguous() if k in ("q", "k", "v", "seg", "dout") else g[k]) for k in g}
        q, k, v, _, _ = run_bwd(alone, dmode="o32")
        assert bitwise_equal(q, bq[t0:t0 + n]) and bitwise_equal(k, bk[t0:t0 + n]) and bitwise_equal(v, bv[t0:t0 + n])
        t0 += n

