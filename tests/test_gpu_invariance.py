"""Bitwise properties of the HIP path: repeatability, single-vs-batched (rollout vs train:
"33B forward/backward" page, dual trajectory), invariance to a segment's offset and neighbours,
head permutation, exact power-of-two scaling of V, and closed forms."""
import numpy as np
import pytest
import torch

import deterministic_invariant_attention_amd as h3
import oracle
import workloads
from gpu_util import EPS, MAX_ABS_BOUND, REL_L2_BOUND, bitwise_equal, digest, f64, metrics, run_fwd, say, to_dev

pytestmark = pytest.mark.gpu


def test_repeat_bitwise_short3_x10():
    g = to_dev(workloads.make_inputs(workloads.WORKLOADS["short3"]))
    say("[bitwise] short3 repeat x10")
    ref, lse = run_fwd(g, want_lse=True)
    d0, l0 = digest(ref), digest(lse)
    for _ in range(9):
        o, l = run_fwd(g, want_lse=True)
        assert digest(o) == d0 and digest(l) == l0


def test_repeat_bitwise_long_x10():
    """The headline workload ten times: output and LSE bit for bit the same every time."""
    g = to_dev(workloads.make_inputs(workloads.WORKLOADS["long"]))
    say("[bitwise] long repeat x10")
    ref, rlse = run_fwd(g, want_lse=True)
    for i in range(9):
        o, l = run_fwd(g, want_lse=True)
        assert bitwise_equal(o, ref) and bitwise_equal(l, rlse), f"repeat {i + 1}"


def test_batch2_alone_equals_batched():
    """Row 0 (one 4253-token segment) and row 1 (2000+2000+253) alone vs in the batch, both orders."""
    wl = workloads.WORKLOADS["batch2"]
    x = workloads.make_inputs(wl)
    g = to_dev(x)
    say("[bitwise] batch2 alone vs batched")
    batched, blse = run_fwd(g, want_lse=True)
    (a0, a1), (b0, b1) = workloads.row_slices(wl)
    for (t0, t1) in ((a0, a1), (b0, b1)):
        alone = {n: (g[n][t0:t1].contiguous() if n in ("q", "k", "v", "seg") else g[n]) for n in g}
        o, l = run_fwd(alone, want_lse=True)
        assert bitwise_equal(o, batched[t0:t1]), f"row [{t0},{t1}) alone differs from batched"
        assert bitwise_equal(l, blse[t0:t1])
    # reversed row order (row 1 first): ids must stay non-decreasing, so re-number
    rev = {n: (torch.cat([g[n][b0:b1], g[n][a0:a1]]) if n in ("q", "k", "v") else g[n]) for n in g}
    rev["seg"] = torch.cat([g["seg"][b0:b1] - 1, torch.full((a1 - a0,), 100, dtype=torch.int32, device=g["seg"].device)])
    o, _ = run_fwd(rev)
    n1 = b1 - b0
    assert bitwise_equal(o[:n1], batched[b0:b1]) and bitwise_equal(o[n1:], batched[a0:a1])


@pytest.mark.parametrize("pad", [1, 63, 64, 65, 127])
def test_leading_segment_offset_invariance(pad):
    """A dummy leading segment shifts every other segment's offset; outputs must not change."""
    x = workloads.random_inputs([300, 129, 64], 3, seed=17)
    g = to_dev(x)
    say(f"[bitwise] offset shift by a {pad}-token leading segment")
    base, blse = run_fwd(g, want_lse=True)
    d = workloads.random_inputs([pad], 3, seed=99)
    sh = {n: torch.cat([d[n].to(g[n].device), g[n]]) for n in ("q", "k", "v")}
    sh["seg"] = torch.cat([torch.full((pad,), -1, dtype=torch.int32), x["seg"]]).to(g["seg"].device)
    sh["wq"], sh["wk"] = g["wq"], g["wk"]
    o, l = run_fwd(sh, want_lse=True)
    assert bitwise_equal(o[pad:], base) and bitwise_equal(l[pad:], blse)


def test_nan_neighbours_do_not_leak():
    x = workloads.random_inputs([70, 131, 45], 2, seed=23)
    g = to_dev(x)
    say("[bitwise] NaN-filled neighbour segments")
    base, _ = run_fwd(g)
    p = {n: g[n].clone() for n in ("q", "k", "v")}
    for n in p:
        p[n][:70] = float("nan")
        p[n][201:] = float("inf")
    p.update(seg=g["seg"], wq=g["wq"], wk=g["wk"])
    o, _ = run_fwd(p)
    assert bitwise_equal(o[70:201], base[70:201])


def test_head_permutation_permutes_output():
    x = workloads.random_inputs([180, 40], 5, seed=29)
    g = to_dev(x)
    say("[bitwise] head permutation")
    base, _ = run_fwd(g)
    perm = torch.tensor([3, 0, 4, 1, 2], device=g["q"].device)
    p = {n: g[n][:, perm].contiguous() for n in ("q", "k", "v")}
    p.update(seg=g["seg"], wq=g["wq"], wk=g["wk"])
    o, _ = run_fwd(p)
    assert bitwise_equal(o, base[:, perm].contiguous())


def test_v_power_of_two_scaling_is_exact():
    x = workloads.random_inputs([150, 66], 3, seed=31)
    v = x["v"].float()
    v[v.abs() < 2.0 ** -10] = 0.0    # keep V out of fp16's subnormal range before and after scaling
    x["v"] = v.to(torch.bfloat16)
    g = to_dev(x)
    say("[bitwise] V * 4 -> O * 4")
    base, _ = run_fwd(g)
    g4 = dict(g)
    g4["v"] = g["v"] * 4
    o4, _ = run_fwd(g4)
    assert bitwise_equal(o4, base * 4)


def test_closed_forms():
    say("[closed form] single key, identical keys, V = 1")
    x = workloads.random_inputs([1, 5, 1, 77, 1], 3, seed=37)
    g = to_dev(x)
    o, _ = run_fwd(g)
    for t in (0, 6, 84):  # single-token segments return their own v (exactly where fp16 holds it)
        got, v = f64(o[t]), f64(g["v"][t])
        exact = (np.abs(v) >= 2.0 ** -17) | (v == 0)
        assert np.array_equal(got[exact], v[exact]) and np.all(np.abs(got - v) <= 2.0 ** -25)
    # identical keys within a segment: uniform softmax, the mean of V (only fp32 summation error)
    k = g["k"].clone()
    k[7:84] = k[7]
    o2, _ = run_fwd(dict(g, k=k))
    mean_v = f64(g["v"][7:84]).mean(0)
    assert np.max(np.abs(f64(o2[7:84]) - mean_v[None])) <= 2 ** -8 * np.max(np.abs(mean_v)) + 1e-6
    # V = 1 everywhere: every output within one bf16 ulp of 1
    ones = torch.ones_like(g["v"])
    o3, _ = run_fwd(dict(g, v=ones))
    assert np.max(np.abs(f64(o3) - 1.0)) <= 2 ** -7


def test_empty_input_is_a_noop():
    e = torch.zeros(0, 2, 128, dtype=torch.bfloat16, device="cuda:0")
    w = torch.ones(128, dtype=torch.bfloat16, device="cuda:0")
    out, _ = run_fwd(dict(q=e, k=e, v=e, seg=torch.zeros(0, dtype=torch.int32, device="cuda:0"), wq=w, wk=w))
    assert out.shape == (0, 2, 128)


def test_long_batch_past_the_decode_prefetch_alone_equals_batched():
    """A batch of 20100 tokens: the segment decode takes its chunked path (more than 16384 ids),
    each segment alone the prefetched one; forward outputs and LSE are the same bits either way."""
    lens = [9000, 7000, 4100]
    x = workloads.random_inputs(lens, 2, seed=71)
    g = to_dev(x)
    say(f"[bitwise] {sum(lens)}-token batch vs its segments alone")
    batched, blse = run_fwd(g, want_lse=True)
    t0 = 0
    for n in lens:
        alone = {k: (g[k][t0:t0 + n].contiguous() if k in ("q", "k", "v", "seg") else g[k]) for k in g}
        o, l = run_fwd(alone, want_lse=True)
        assert bitwise_equal(o, batched[t0:t0 + n]) and bitwise_equal(l, blse[t0:t0 + n]), f"segment at {t0}"
        t0 += n


def test_key_tile_edges_alone_equal_batched():
    """Segments one key short of, at, and one key past two, three and four KV tiles of 96 keys:
    each alone gives the bits it gives in the batch."""
    lens = [191, 192, 193, 287, 288, 289, 383, 384, 385]
    x = workloads.random_inputs(lens, 2, seed=73)
    g = to_dev(x)
    say(f"[bitwise] {sum(lens)}-token batch of key-tile edge lengths vs its segments alone")
    batched, blse = run_fwd(g, want_lse=True)
    t0 = 0
    for n in lens:
        alone = {k: (g[k][t0:t0 + n].contiguous() if k in ("q", "k", "v", "seg") else g[k]) for k in g}
        o, l = run_fwd(alone, want_lse=True)
        assert bitwise_equal(o, batched[t0:t0 + n]) and bitwise_equal(l, blse[t0:t0 + n]), f"segment at {t0}"
        t0 += n


@pytest.mark.parametrize("la", [1000, 800])
def test_half_items_alone_equal_whole_items_batched(la):
    """A segment of 4 query tiles x 8 heads alone is too little work to fill a round, so its tiles
    run as 128-query halves (4 waves computing); packed beside a 7168-token segment the 32 x 8
    items fill whole rounds and run whole.  The rows must come out bitwise equal both ways, and
    the alone run must match the oracle.  la = 800 leaves the second half of the last tile with
    no valid row."""
    x = workloads.random_inputs([la, 28 * 256], 8, seed=31)
    g = to_dev(x)
    say(f"[bitwise] {la}-token segment alone (half items) vs packed with 7168 tokens (whole items)")
    batched, blse = run_fwd(g, want_lse=True)
    alone = {n: (g[n][:la].contiguous() if n in ("q", "k", "v", "seg") else g[n]) for n in g}
    o, l = run_fwd(alone, want_lse=True)
    assert bitwise_equal(o, batched[:la]) and bitwise_equal(l, blse[:la])
    xa = {n: (x[n][:la] if n in ("q", "k", "v", "seg") else x[n]) for n in x}
    ref, _ = oracle.fwd(xa["q"], xa["k"], xa["v"], xa["seg"].numpy(), xa["wq"], xa["wk"], EPS, 128 ** -0.5)
    rel, mx = metrics(o, ref)
    say(f"[parity] {la} alone: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2_BOUND and mx <= MAX_ABS_BOUND


@pytest.mark.parametrize("name", ["batch2", "short3"])
def test_staged_attend_repeated_after_one_plan(name):
    """One plan and one staging, then three attention launches on the same workspace (a caller that
    reuses a plan across blocks): each must equal the one-call forward bit for bit.  On batch2 the
    workgroups take their later units from per-XCD counters that each launch returns to zero at its
    end; short3 fits one round and uses none."""
    wl = workloads.WORKLOADS[name]
    g = to_dev(workloads.make_inputs(wl))
    say(f"[bitwise] {name}: plan once, attend three times")
    ref, rlse = run_fwd(g, want_lse=True)
    T, H = g["q"].shape[0], g["q"].shape[1]
    ws = h3.workspace(T, H, g["q"].device)
    h3.h3attn_plan(g["seg"], H, ws)
    h3.h3attn_prep_qkv(g["q"], g["k"], g["v"], g["wq"], g["wk"], ws, eps=EPS)
    for i in range(3):
        out = torch.full_like(g["q"], float("nan"))
        lse = torch.full((T, H), float("nan"), dtype=torch.float32, device=g["q"].device)
        h3.h3attn_attend(g["q"], g["wq"], ws, out, lse=lse, eps=EPS, scale=128 ** -0.5)
        torch.cuda.synchronize()
        assert bitwise_equal(out, ref) and bitwise_equal(lse, rlse), f"launch {i}"
