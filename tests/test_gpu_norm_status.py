"""The standalone q/k norm against the oracle, the fused prologue against the standalone norm
(bitwise), and the device status word for data errors."""
import numpy as np
import pytest
import torch

import deterministic_invariant_attention_amd as h3
import oracle
import workloads
from gpu_util import bitwise_equal, f64, run_fwd, say, to_dev

pytestmark = pytest.mark.gpu


def _ulp_distance(a_bits, b_bits):
    """Distance in bf16 steps between two arrays of bf16 patterns (same-sign values)."""
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    ka = np.where(a & 0x8000, -(a & 0x7FFF), a & 0x7FFF)
    kb = np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(ka - kb)


@pytest.mark.parametrize("name", ["short3", "long_w25"])
def test_qknorm_matches_oracle_bitwise(name):
    """Both sides round the FP64 norm once to bf16: the codes are identical.  (The FP64 sums of
    squares are exact for bf16 inputs of any ordinary range, so the summation order cannot move a
    value across a rounding midpoint.)"""
    wl = workloads.WORKLOADS[name]
    x = workloads.make_inputs(wl)
    say(f"[qknorm] {name}")
    for n, w in (("q", "wq"), ("k", "wk")):
        y = h3.h3attn_qknorm(x[n].cuda(), x[w].cuda(), eps=wl.eps)
        torch.cuda.synchronize()
        got = y.cpu().view(torch.int16).numpy().view(np.uint16)
        ref = oracle.qknorm(x[n], x[w], wl.eps)
        dist = _ulp_distance(got, ref)
        frac = float(np.mean(dist > 0))
        say(f"[qknorm] {name}.{n}: max ulp {dist.max()}, flipped fraction {frac:.2e}")
        assert dist.max() == 0


def test_qknorm_extreme_ranges_match_oracle_bitwise():
    """Weights spread over the whole bf16 range, so the normed values reach the bf16 subnormals and
    overflow past the largest bf16 to infinity; plus a zero row and a row holding an infinity (its
    norm is NaN).  Every code equals the oracle's (NaN where the oracle has NaN: the payload and
    sign of a NaN are not part of the contract)."""
    g = torch.Generator().manual_seed(59)
    T, H = 48, 3
    x = torch.randn(T, H, 128, generator=g).to(torch.bfloat16)
    x[5, 1] = 0.0
    x[9, 2, 17] = float("inf")
    e = torch.randint(-133, 128, (128,), generator=g).to(torch.float64)
    sgn = torch.where(torch.rand(128, generator=g) < 0.5, -1.0, 1.0).to(torch.float64)
    w = (sgn * (1.0 + torch.rand(128, generator=g, dtype=torch.float64)) * torch.exp2(e)).to(torch.bfloat16)
    w[0] = 0.0
    say("[qknorm] extreme ranges")
    y = h3.h3attn_qknorm(x.cuda(), w.cuda())
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.qknorm(x, w, 1e-6)
    ref_nan = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    assert np.array_equal(ref_nan, got_nan)
    assert ref_nan.any() and ((ref & 0x7FFF) == 0x7F80).any() and (((ref & 0x7F80) == 0) & ((ref & 0x7F) != 0)).any()
    assert np.array_equal(got[~ref_nan], ref[~ref_nan])


def test_qknorm_in_place_equals_out_of_place():
    x = workloads.random_inputs([333], 7, seed=41)
    a = x["q"].cuda()
    y = h3.h3attn_qknorm(a, x["wq"].cuda())
    b = a.clone()
    h3.h3attn_qknorm(b, x["wq"].cuda(), out=b)
    torch.cuda.synchronize()
    assert bitwise_equal(y, b)


def test_fused_prologue_equals_standalone_norm():
    """fwd with weights == fwd on h3attn_qknorm outputs without weights, bit for bit."""
    x = workloads.random_inputs([255, 513, 70], 6, seed=43)
    g = to_dev(x)
    say("[qknorm] fused prologue vs standalone")
    fused, flse = run_fwd(g, want_lse=True)
    qn = h3.h3attn_qknorm(g["q"], g["wq"])
    kn = h3.h3attn_qknorm(g["k"], g["wk"])
    pre, plse = run_fwd(dict(g, q=qn, k=kn), want_lse=True, weights=False)
    assert bitwise_equal(fused, pre) and bitwise_equal(flse, plse)


def test_decreasing_segment_ids_set_status_and_nan_fill():
    x = workloads.random_inputs([40, 40], 2, seed=47)
    g = to_dev(x)
    g["seg"] = torch.tensor([0] * 30 + [1] * 20 + [0] * 30, dtype=torch.int32, device="cuda:0")
    say("[status] decreasing segment ids")
    ws = h3.workspace(80, 2, "cuda:0")
    out, lse = run_fwd(g, want_lse=True, ws=ws)
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_ERR_SEGMENTS
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()
    # the next valid call on the same workspace resets the status and computes normally
    g["seg"] = x["seg"].cuda()
    out2, _ = run_fwd(g, ws=ws)
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_OK
    assert torch.isfinite(out2.float()).all()


def test_v_out_of_fp16_range_fails_its_own_segment_only():
    """A finite |v| beyond fp16 cannot enter the P.V product: the status word reports ERR_RANGE and
    the rows of that value's segment are NaN (fail closed), while every other segment keeps the
    bits it has alone, so alone == batched holds for such inputs too."""
    x = workloads.random_inputs([40, 40], 2, seed=53)
    g0 = to_dev(x)
    clean, clse = run_fwd(g0, want_lse=True)
    x["v"][10, 1, 5] = 1.0e5
    g = to_dev(x)
    say("[status] |v| > 65504 in segment 0")
    ws = h3.workspace(80, 2, "cuda:0")
    out, lse = run_fwd(g, want_lse=True, ws=ws)
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_ERR_RANGE
    assert torch.isnan(out[:40].float()).all() and torch.isnan(lse[:40]).all()
    assert bitwise_equal(out[40:], clean[40:]) and bitwise_equal(lse[40:], clse[40:])
    alone = {n: (g[n][40:].contiguous() if n in ("q", "k", "v", "seg") else g[n]) for n in g}
    oa, la = run_fwd(alone, want_lse=True)
    assert bitwise_equal(oa, out[40:]) and bitwise_equal(la, lse[40:])
    # infinities are not a range error: they propagate as IEEE values (only in their own segment)
    x["v"][10, 1, 5] = float("inf")
    g = to_dev(x)
    out, _ = run_fwd(g, ws=ws)
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_OK
    assert torch.isfinite(out[40:].float()).all()


def test_flagged_segments_in_a_multi_round_walk():
    """48 segments x 8 heads: about 800 work units for 256 workgroups, so the workgroups take their
    later units from the per-XCD counters.  Four segments scattered over the item list hold a v
    beyond fp16: their rows are NaN, and every other row keeps the bits of a clean run."""
    rng = np.random.default_rng(91)
    lens = [int(n) for n in rng.integers(150, 700, size=48)]
    x = workloads.random_inputs(lens, 8, seed=92)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    g0 = to_dev(x)
    clean, clse = run_fwd(g0, want_lse=True)
    bad = [3, 17, 30, 46]
    for sgi in bad:
        x["v"][int(starts[sgi]) + 5, 3, 7] = 1.0e5
    g = to_dev(x)
    say(f"[status] {sum(lens)} tokens x 8 heads, |v| > 65504 in segments {bad}")
    ws = h3.workspace(sum(lens), 8, "cuda:0")
    out, lse = run_fwd(g, want_lse=True, ws=ws)
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_ERR_RANGE
    flagged = np.zeros(sum(lens), dtype=bool)
    for sgi in bad:
        flagged[starts[sgi]:starts[sgi] + lens[sgi]] = True
    fl = torch.from_numpy(flagged).to(out.device)
    assert torch.isnan(out[fl].float()).all() and torch.isnan(lse[fl]).all()
    assert bitwise_equal(out[~fl], clean[~fl]) and bitwise_equal(lse[~fl], clse[~fl])


def test_wrong_arguments_raise():
    x = to_dev(workloads.random_inputs([8], 2, seed=1))
    with pytest.raises(h3.H3AttnError):
        h3.h3attn_fwd(x["q"], x["k"], x["v"], x["seg"], x["wq"], None)
    with pytest.raises(h3.H3AttnError):
        h3.h3attn_fwd(x["q"], x["k"], x["v"], x["seg"], scale=-1.0)
