"""Seeded random packs of segments through the whole path: parity with the FP64 oracle and one
segment alone equal to its rows in the pack, bit for bit.

Each seed draws a pack of 1 to 12 segments with log-uniform lengths from 1 to 1500 tokens, a head
count, the softmax sharpness (q/k draw scale, norm-weight scale) and whether norm weights are
given.  Such mixes make every work-scheduling path run: items of very different cost in one
launch, XCDs with and without a sparse last round (and so with and without 128-query halves), and
launches that fit in one round.  The rows of the chosen segment are computed in a different
schedule alone than in the pack, which the bitwise comparison checks."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import EPS, MAX_ABS_BOUND, REL_L2_BOUND, bitwise_equal, f64, metrics, run_fwd, say, to_dev
from test_gpu_bwd import _check as bwd_check
from test_gpu_bwd import run_bwd

pytestmark = pytest.mark.gpu


def _draw(seed, max_len=1500, max_segs=12, heads=(1, 2, 3, 5, 8)):
    rng = np.random.default_rng(seed)
    nseg = int(rng.integers(1, max_segs + 1))
    lens = [int(round(np.exp(rng.uniform(0.0, np.log(max_len))))) for _ in range(nseg)]
    H = int(rng.choice(heads))
    qk = float(rng.choice([1.0, 3.0]))
    ws = float(rng.choice([1.0, 1.0, 4.0]))
    normed = bool(rng.random() < 0.85)
    pick = int(rng.integers(0, nseg))
    return lens, H, qk, ws, normed, pick


@pytest.mark.parametrize("seed", range(10))
def test_random_pack_forward(seed):
    lens, H, qk, ws, normed, pick = _draw(1000 + seed)
    x = workloads.random_inputs(lens, H, seed=2000 + seed, qk_scale=qk, w_scale=ws, normed=normed)
    say(f"[random fwd] seed {seed}: segments {lens} H={H} qk x{qk} w x{ws} normed={normed}")
    g = to_dev(x)
    out, lse = run_fwd(g, want_lse=True, weights=normed)
    ref, _ = oracle.fwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"] if normed else None,
                        x["wk"] if normed else None, EPS, 128 ** -0.5)
    rel, mx = metrics(out, ref)
    say(f"[random fwd] seed {seed}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert np.all(np.isfinite(f64(out)))
    assert rel <= REL_L2_BOUND and mx <= MAX_ABS_BOUND
    # the picked segment alone (its own ids) against its rows in the pack
    s0 = sum(lens[:pick])
    s1 = s0 + lens[pick]
    alone = {n: (g[n][s0:s1].contiguous() if n in ("q", "k", "v", "seg") else g[n]) for n in g}
    o1, l1 = run_fwd(alone, want_lse=True, weights=normed)
    assert bitwise_equal(o1, out[s0:s1]) and bitwise_equal(l1, lse[s0:s1])


@pytest.mark.parametrize("seed", range(4))
def test_random_pack_backward(seed):
    lens, H, qk, ws, normed, pick = _draw(3000 + seed, max_len=700, max_segs=8, heads=(1, 2, 3))
    x = workloads.random_inputs(lens, H, seed=4000 + seed, qk_scale=qk, w_scale=ws, normed=normed,
                                with_grad=True)
    dmode = "o32" if seed % 2 else "recompute"
    dq, dk, dv = bwd_check(f"random seed {seed} {lens}", x, weights=normed, dmode=dmode)
    g = to_dev(x)
    s0 = sum(lens[:pick])
    s1 = s0 + lens[pick]
    alone = {n: (g[n][s0:s1].contiguous() if n in ("q", "k", "v", "seg", "dout") else g[n]) for n in g}
    a = run_bwd(alone, weights=normed, dmode=dmode)
    for nm, u, w in (("dq", a[0], dq), ("dk", a[1], dk), ("dv", a[2], dv)):
        assert bitwise_equal(u, w[s0:s1]), nm


@pytest.mark.parametrize("seed", range(4))
def test_random_large_pack_forward(seed):
    """Segments of up to 4000 tokens (log-uniform) until the pack passes 6000 tokens, at most 30 of
    them, 16 to 40 heads: hundreds of work units per XCD, so the workgroups take their later units from the per-XCD counters, and items
    of very different cost meet.  Sampled rows (every head) against the oracle; two segments alone
    against their rows in the pack, bit for bit."""
    rng = np.random.default_rng(5000 + seed)
    lens = []
    while sum(lens) < 6000:
        lens.append(int(round(np.exp(rng.uniform(0.0, np.log(4000))))))
    lens = lens[:30]
    H = int(rng.choice([16, 24, 40]))
    qk = float(rng.choice([1.0, 3.0]))
    x = workloads.random_inputs(lens, H, seed=6000 + seed, qk_scale=qk)
    T = sum(lens)
    say(f"[random fwd large] seed {seed}: {len(lens)} segments, T={T} H={H} qk x{qk}")
    g = to_dev(x)
    out, lse = run_fwd(g, want_lse=True)
    rows = np.unique(np.concatenate([rng.integers(0, T, 40), np.cumsum([0] + lens[:-1]),
                                     np.cumsum(lens) - 1]))
    ref, _ = oracle.fwd_rows(x["q"], x["k"], x["v"], x["seg"].numpy(), rows, x["wq"], x["wk"], EPS)
    rel, mx = metrics(f64(out)[rows], ref)
    say(f"[random fwd large] seed {seed}: {len(rows)} rows, rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert np.all(np.isfinite(f64(out)))
    assert rel <= REL_L2_BOUND and mx <= MAX_ABS_BOUND
    for pick in rng.choice(len(lens), size=2, replace=False):
        s0 = sum(lens[:pick])
        s1 = s0 + lens[pick]
        alone = {n: (g[n][s0:s1].contiguous() if n in ("q", "k", "v", "seg") else g[n]) for n in g}
        o1, l1 = run_fwd(alone, want_lse=True)
        assert bitwise_equal(o1, out[s0:s1]) and bitwise_equal(l1, lse[s0:s1]), f"segment {pick}"
