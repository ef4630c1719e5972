"""MM-RoPE on the GPU path (h3attn_fwd_ex / h3attn_bwd_ex with rope tables): the node the block runs
between q_norm/k_norm and the attention ("ws1_one_h3_block + full-model qualification" page,
Bindings table: rope_q, rope_k; Tests: MM-RoPE rotates 96 of 128 channels), table-driven.

Parity against the oracle's forward and gradients with the same tables (relative L2 <= 2e-3, max
abs <= 2e-2, gradients' max abs scaled by their magnitude), the identity table reproducing the path
without rope bit for bit, alone == batched, and the position order with permuted tables."""
import numpy as np
import pytest
import torch

import deterministic_invariant_attention_amd as h3
import oracle
import workloads
from gpu_util import (EPS, LSE_REL_BOUND, MAX_ABS_BOUND, REL_L2_BOUND, bitwise_equal, f64, lse_error, metrics, say,
                      to_dev)

pytestmark = pytest.mark.gpu
SCALE = 128 ** -0.5


def fwd(g, rope=None, pos=None, o32=False):
    rc, rs = (None, None) if rope is None else rope
    return h3.h3attn_fwd_ex(g["q"], g["k"], g["v"], g["seg"], pos, g["wq"], g["wk"], eps=EPS, scale=SCALE,
                            want_lse=True, want_o32=o32, rope_cos=rc, rope_sin=rs)


def bwd(g, lse, rope=None, pos=None, o32=None):
    rc, rs = (None, None) if rope is None else rope
    return h3.h3attn_bwd_ex(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], pos, o32, g["wq"], g["wk"], eps=EPS,
                            scale=SCALE, rope_cos=rc, rope_sin=rs)


def run(g, rope, dmode, pos=None):
    out, lse, o32 = fwd(g, rope, pos, o32=dmode == "o32")
    grads = bwd(g, lse, rope, pos, o32 if dmode == "o32" else None)
    torch.cuda.synchronize()
    return out, lse, grads


def test_identity_table_is_the_path_without_rope():
    lens = [300, 129, 64, 1]
    x = workloads.random_inputs(lens, 3, seed=81, with_grad=True)
    g = to_dev(x)
    ident = tuple(t.cuda() for t in workloads.rope_tables(lens, "identity"))
    say("[rope] identity table vs no rope")
    for dmode in ("recompute", "o32"):
        a = run(g, None, dmode)
        b = run(g, ident, dmode)
        assert bitwise_equal(a[0], b[0]) and bitwise_equal(a[1], b[1])
        for u, w in zip(a[2], b[2]):
            assert bitwise_equal(u, w)


@pytest.mark.parametrize("kind", ["grid", "random"])
def test_rope_parity_forward_and_backward(kind):
    lens = [300, 97, 1, 200, 64]
    x = workloads.random_inputs(lens, 4, seed=82, with_grad=True, w_scale=2.0)
    rc, rs = workloads.rope_tables(lens, kind, seed=83)
    g = to_dev(x)
    rope = (rc.cuda(), rs.cuda())
    ref, ref_lse = oracle.fwd_ex(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], EPS, SCALE, cos=rc,
                                 sin=rs)
    plain, _ = oracle.fwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], EPS, SCALE)
    assert np.linalg.norm(ref - plain) / np.linalg.norm(plain) > 1e-2  # the tables do rotate
    gref = oracle.bwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["dout"], x["wq"], x["wk"], EPS, SCALE, cos=rc,
                      sin=rs)
    for dmode in ("recompute", "o32"):
        out, lse, grads = run(g, rope, dmode)
        rel, mx = metrics(out, ref)
        le = lse_error(lse, ref_lse)
        say(f"[rope] {kind} {dmode}: out rel_l2={rel:.3e} max_abs={mx:.3e} lse_rel_err={le:.2e}")
        assert rel <= REL_L2_BOUND and mx <= MAX_ABS_BOUND and le <= LSE_REL_BOUND
        for nm, a, r in zip(("dq", "dk", "dv", "dwq", "dwk"), grads, gref):
            a64 = f64(a)
            rel = float(np.linalg.norm(a64 - r) / np.linalg.norm(r))
            mx = float(np.max(np.abs(a64 - r)))
            say(f"[rope] {kind} {dmode}: {nm} rel_l2={rel:.3e} max_abs={mx:.3e}")
            assert rel <= REL_L2_BOUND, nm
            if a.dim() == 3:
                assert mx <= MAX_ABS_BOUND * max(1.0, float(np.abs(r).max())), nm


def test_rope_batch2_alone_equals_batched():
    wl = workloads.WORKLOADS["batch2"]
    x = workloads.make_inputs(wl, with_grad=True)
    rc, rs = workloads.rope_tables(wl.seg_lens, "grid")
    g = to_dev(x)
    say("[rope] batch2 alone vs batched, grid tables")
    out, lse, grads = run(g, (rc.cuda(), rs.cuda()), "o32")
    for t0, t1 in workloads.row_slices(wl):
        alone = {n: (g[n][t0:t1].contiguous() if n in ("q", "k", "v", "seg", "dout") else g[n]) for n in g}
        o, l, gr = run(alone, (rc[t0:t1].contiguous().cuda(), rs[t0:t1].contiguous().cuda()), "o32")
        assert bitwise_equal(o, out[t0:t1]) and bitwise_equal(l, lse[t0:t1])
        for u, w in zip(gr[:3], grads[:3]):
            assert bitwise_equal(u, w[t0:t1])


def test_rope_with_position_order_permutes_bitwise():
    """Shuffling a segment's tokens together with their positions and their table rows permutes the
    outputs and gradients and changes no bit of them (nor of dwq, dwk)."""
    lens = [257, 130, 64]
    x = workloads.random_inputs(lens, 2, seed=84, with_grad=True)
    rc, rs = workloads.rope_tables(lens, "grid")
    pos = workloads.position_ids(lens)
    g = to_dev(x)
    say("[rope] position order, shuffled tokens and tables")
    base = run(g, (rc.cuda(), rs.cuda()), "recompute", pos=pos.cuda())
    p = workloads.shuffle_within_segments(lens, 85)
    y = {n: (x[n][p].contiguous() if n in ("q", "k", "v", "dout") else x[n]) for n in x}
    gy = to_dev(y)
    got = run(gy, (rc[p].contiguous().cuda(), rs[p].contiguous().cuda()), "recompute", pos=pos[p].contiguous().cuda())
    pd = p.cuda()
    assert bitwise_equal(got[0], base[0][pd]) and bitwise_equal(got[1], base[1][pd])
    for a, b in zip(got[2][:3], base[2][:3]):
        assert bitwise_equal(a, b[pd])
    for a, b in zip(got[2][3:], base[2][3:]):
        assert bitwise_equal(a, b)
