"""Position-ordered traversal (h3attn_fwd_pos, h3attn_bwd_pos) on the GPU.

The "ws1_one_h3_block + full-model qualification" page (Results, control H-C3) reports that
permuting the packed rows together with their positions changes output bits, because attention adds
keys in packed order.  With position ids the library adds them in position order, so:
  * shuffling the tokens of each segment together with their position ids shuffles the output rows
    (and LSE rows, and the gradient rows of q, k, v) and changes no bit of them; dwq and dwk do not
    change at all;
  * natural positions (0..L-1 in packing order) give bitwise the plain entry points' results;
  * the result still meets the oracle's bound (the oracle's FP64 sums do not depend on the order);
  * ids that are not a permutation of 0..L-1 in some segment set H3ATTN_ERR_POSITIONS and NaN-fill
    that segment's rows (the other segments keep their bits)
    every output; the next valid call on the workspace computes normally.
"""
import numpy as np
import pytest
import torch

import deterministic_invariant_attention_amd as h3
import oracle
import workloads
from gpu_util import EPS, MAX_ABS_BOUND, REL_L2_BOUND, bitwise_equal, f64, metrics, say, to_dev

pytestmark = pytest.mark.gpu
SCALE = 128 ** -0.5
ROW_INPUTS = ("q", "k", "v", "dout")


def shuffled(x, seg_lens, seed):
    """The batch with each segment's tokens shuffled (with their position ids); returns (x', pos', p)."""
    p = workloads.shuffle_within_segments(seg_lens, seed)
    pos = workloads.position_ids(seg_lens)
    y = {n: (t[p].contiguous() if n in ROW_INPUTS else t) for n, t in x.items()}
    return y, pos[p].contiguous(), p


def fwd_pos(g, pos, weights=True, ws=None):
    wq, wk = (g["wq"], g["wk"]) if weights else (None, None)
    out, lse = h3.h3attn_fwd_pos(g["q"], g["k"], g["v"], g["seg"], pos, wq, wk, eps=EPS, scale=SCALE, want_lse=True,
                                 workspace_buf=ws)
    torch.cuda.synchronize()
    return out, lse


def fwd_plain(g, weights=True):
    wq, wk = (g["wq"], g["wk"]) if weights else (None, None)
    out, lse = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], wq, wk, eps=EPS, scale=SCALE, want_lse=True)
    torch.cuda.synchronize()
    return out, lse


def bwd_pos(g, pos, lse, weights=True, ws=None):
    wq, wk = (g["wq"], g["wk"]) if weights else (None, None)
    res = h3.h3attn_bwd_pos(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], pos, wq, wk, eps=EPS, scale=SCALE,
                            workspace_buf=ws)
    torch.cuda.synchronize()
    return res


def rows_differing(a, b):
    return int((a.view(torch.int16) != b.view(torch.int16)).flatten(1).any(1).sum())


RAGGED = [300, 129, 64, 77, 1, 200]   # several tiles, ragged tails, a one-token segment


@pytest.mark.parametrize("weights", [True, False])
def test_natural_positions_equal_packed_order(weights):
    x = workloads.random_inputs(RAGGED, 3, seed=71, with_grad=True, normed=weights)
    g = to_dev(x)
    pos = workloads.position_ids(RAGGED).cuda()
    say(f"[position] natural positions == packed order, weights={weights}")
    out, lse = fwd_plain(g, weights)
    out_p, lse_p = fwd_pos(g, pos, weights)
    assert bitwise_equal(out, out_p) and bitwise_equal(lse, lse_p)
    wq, wk = (g["wq"], g["wk"]) if weights else (None, None)
    ref = h3.h3attn_bwd(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], wq, wk, eps=EPS, scale=SCALE)
    got = bwd_pos(g, pos, lse, weights)
    for a, b in zip(ref, got):
        assert (a is None and b is None) or bitwise_equal(a, b)


@pytest.mark.parametrize("weights", [True, False])
def test_fwd_shuffle_within_segments_is_bitwise_invariant(weights):
    x = workloads.random_inputs(RAGGED, 3, seed=73, normed=weights)
    g = to_dev(x)
    pos = workloads.position_ids(RAGGED).cuda()
    base, blse = fwd_pos(g, pos, weights)
    for seed in (1, 2, 3):
        y, pos_y, p = shuffled(x, RAGGED, seed)
        say(f"[position] fwd shuffle seed={seed} weights={weights}")
        out, lse = fwd_pos(to_dev(y), pos_y.cuda(), weights)
        pd = p.cuda()
        assert bitwise_equal(out, base[pd]) and bitwise_equal(lse, blse[pd])


def test_fwd_shuffled_parity_with_oracle():
    x = workloads.random_inputs(RAGGED, 3, seed=79)
    y, pos_y, _ = shuffled(x, RAGGED, 5)
    say("[position] fwd shuffled vs oracle")
    out, lse = fwd_pos(to_dev(y), pos_y.cuda())
    ref, ref_lse = oracle.fwd(y["q"], y["k"], y["v"], y["seg"].numpy(), y["wq"], y["wk"], EPS, SCALE)
    rel, mx = metrics(out, ref)
    lse_err = float(np.max(np.abs(f64(lse) - ref_lse)))
    say(f"[position] rel_l2={rel:.3e} max_abs={mx:.3e} lse_err={lse_err:.2e}")
    assert rel <= REL_L2_BOUND and mx <= MAX_ABS_BOUND and lse_err <= 1e-4


@pytest.mark.parametrize("name", ["batch2", "long"])
def test_fwd_shuffle_full_size(name):
    """The full workloads: shuffled rows give the same bits with positions; the packed-order entry
    point is shown to differ on the same shuffle (the effect the control measures)."""
    wl = workloads.WORKLOADS[name]
    x = workloads.make_inputs(wl)
    g = to_dev(x)
    pos = workloads.position_ids(wl.seg_lens).cuda()
    base, blse = fwd_pos(g, pos)
    y, pos_y, p = shuffled(x, wl.seg_lens, 11)
    gy = to_dev(y)
    pd = p.cuda()
    say(f"[position] {name} full size, shuffled")
    out, lse = fwd_pos(gy, pos_y.cuda())
    assert bitwise_equal(out, base[pd]) and bitwise_equal(lse, blse[pd])
    plain, _ = fwd_plain(gy)
    ref_plain, _ = fwd_plain(g)
    say(f"[position] {name}: packed-order attention changes {rows_differing(plain, ref_plain[pd])} of "
        f"{wl.tokens} output rows under the shuffle; position order changes 0")


@pytest.mark.parametrize("weights", [True, False])
def test_bwd_shuffle_within_segments_is_bitwise_invariant(weights):
    x = workloads.random_inputs(RAGGED, 3, seed=83, with_grad=True, normed=weights)
    g = to_dev(x)
    pos = workloads.position_ids(RAGGED).cuda()
    _, lse = fwd_pos(g, pos, weights)
    base = bwd_pos(g, pos, lse, weights)
    for seed in (1, 2):
        y, pos_y, p = shuffled(x, RAGGED, seed)
        gy = to_dev(y)
        say(f"[position] bwd shuffle seed={seed} weights={weights}")
        _, lse_y = fwd_pos(gy, pos_y.cuda(), weights)
        got = bwd_pos(gy, pos_y.cuda(), lse_y, weights)
        pd = p.cuda()
        for a, b in zip(got[:3], base[:3]):
            assert bitwise_equal(a, b[pd])
        if weights:
            assert torch.equal(got[3], base[3]) and torch.equal(got[4], base[4])


def test_bwd_shuffled_parity_with_oracle():
    x = workloads.random_inputs(RAGGED, 3, seed=89, with_grad=True)
    y, pos_y, _ = shuffled(x, RAGGED, 7)
    gy = to_dev(y)
    say("[position] bwd shuffled vs oracle")
    _, lse = fwd_pos(gy, pos_y.cuda())
    got = bwd_pos(gy, pos_y.cuda(), lse)
    ref = oracle.bwd(y["q"], y["k"], y["v"], y["seg"].numpy(), y["dout"], y["wq"], y["wk"], EPS, SCALE)
    for nm, a, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        rel, mx = metrics(a, r)
        say(f"[position] {nm}: rel_l2={rel:.3e} max_abs={mx:.3e}")
        assert rel <= REL_L2_BOUND and mx <= MAX_ABS_BOUND * max(1.0, float(np.abs(r).max())), nm
    for nm, a, r in zip(("dwq", "dwk"), got[3:], ref[3:]):
        rel = float(np.linalg.norm(a.cpu().double().numpy() - r) / np.linalg.norm(r))
        say(f"[position] {nm}: rel_l2={rel:.3e}")
        assert rel <= REL_L2_BOUND, nm


def test_bwd_shuffle_full_size_batch2():
    wl = workloads.WORKLOADS["batch2"]
    x = workloads.make_inputs(wl, with_grad=True)
    g = to_dev(x)
    pos = workloads.position_ids(wl.seg_lens).cuda()
    _, lse = fwd_pos(g, pos)
    base = bwd_pos(g, pos, lse)
    y, pos_y, p = shuffled(x, wl.seg_lens, 13)
    gy = to_dev(y)
    say("[position] bwd batch2 full size, shuffled")
    _, lse_y = fwd_pos(gy, pos_y.cuda())
    got = bwd_pos(gy, pos_y.cuda(), lse_y)
    pd = p.cuda()
    for a, b in zip(got[:3], base[:3]):
        assert bitwise_equal(a, b[pd])
    assert torch.equal(got[3], base[3]) and torch.equal(got[4], base[4])


def bad_positions(kind, seg_lens):
    pos = workloads.position_ids(seg_lens).clone()
    if kind == "duplicate":
        pos[45] = pos[44]        # segment 1 (tokens 40..79): two tokens at one position, one position empty
    elif kind == "too_large":
        pos[50] = seg_lens[1]    # == L
    elif kind == "negative":
        pos[3] = -1
    elif kind == "huge":
        pos[79] = 2 ** 31 - 1
    elif kind == "shifted":
        pos[40:80] += 1          # segment 1 numbered 1..40 instead of 0..39
    return pos


@pytest.mark.parametrize("kind", ["duplicate", "too_large", "negative", "huge", "shifted"])
def test_invalid_positions_fail_their_own_segment_only(kind):
    """Ids that are not a permutation of 0..L-1 in one segment: ERR_POSITIONS, that segment's rows
    NaN (forward and backward), the other segment's rows the bits of valid ids; the weight
    gradients, sums over the whole batch, are NaN."""
    seg_lens = [40, 40]
    x = workloads.random_inputs(seg_lens, 2, seed=97, with_grad=True)
    g = to_dev(x)
    pos = bad_positions(kind, seg_lens).cuda()
    bad = slice(0, 40) if kind == "negative" else slice(40, 80)
    good_rows = slice(40, 80) if kind == "negative" else slice(0, 40)
    say(f"[position] invalid ids: {kind}")
    good = workloads.position_ids(seg_lens).cuda()
    ws = h3.workspace(80, 2, "cuda:0")
    ref, rlse = fwd_pos(g, good, ws=ws)
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_OK
    out, lse = fwd_pos(g, pos, ws=ws)
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_ERR_POSITIONS
    assert torch.isnan(out[bad].float()).all() and torch.isnan(lse[bad]).all()
    assert bitwise_equal(out[good_rows], ref[good_rows]) and bitwise_equal(lse[good_rows], rlse[good_rows])
    bws = h3.bwd_workspace(80, 2, "cuda:0")
    gref = bwd_pos(g, good, rlse, ws=bws)
    assert h3.h3attn_status_read(bws) == h3.H3ATTN_OK
    for t in gref:
        assert torch.isfinite(t.float()).all()
    res = bwd_pos(g, pos, rlse, ws=bws)
    assert h3.h3attn_status_read(bws) == h3.H3ATTN_ERR_POSITIONS
    for t, r in zip(res[:3], gref[:3]):
        assert torch.isnan(t[bad].float()).all()
        assert bitwise_equal(t[good_rows], r[good_rows])
    for t in res[3:]:
        assert torch.isnan(t).all()


def test_decreasing_segments_take_precedence_over_positions():
    x = workloads.random_inputs([40, 40], 2, seed=101)
    g = to_dev(x)
    g["seg"] = torch.tensor([0] * 30 + [1] * 20 + [0] * 30, dtype=torch.int32, device="cuda:0")
    pos = bad_positions("negative", [40, 40]).cuda()
    ws = h3.workspace(80, 2, "cuda:0")
    say("[position] decreasing segment ids and invalid positions")
    out, _ = fwd_pos(g, pos, ws=ws)
    assert h3.h3attn_status_read(ws) == h3.H3ATTN_ERR_SEGMENTS
    assert torch.isnan(out.float()).all()


def test_empty_input_is_a_noop():
    e = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda:0")
    seg = torch.empty(0, dtype=torch.int32, device="cuda:0")
    w = torch.ones(128, dtype=torch.bfloat16, device="cuda:0")
    out, lse = h3.h3attn_fwd_pos(e, e, e, seg, seg, w, w, want_lse=True)
    res = h3.h3attn_bwd_pos(e, e, e, e, torch.empty((0, 2), device="cuda:0"), seg, seg, w, w)
    torch.cuda.synchronize()
    assert out.numel() == 0 and lse.numel() == 0 and res[0].numel() == 0


def test_bwd_shuffle_with_o32_is_bitwise_invariant():
    """The same with D = dO . O from the forward's fp32 output (h3attn_fwd_ex / h3attn_bwd_ex)."""
    x = workloads.random_inputs(RAGGED, 3, seed=87, with_grad=True)
    g = to_dev(x)
    pos = workloads.position_ids(RAGGED).cuda()

    def run(gg, pp):
        _, lse, o32 = h3.h3attn_fwd_ex(gg["q"], gg["k"], gg["v"], gg["seg"], pp, gg["wq"], gg["wk"], eps=EPS,
                                       scale=SCALE, want_lse=True, want_o32=True)
        res = h3.h3attn_bwd_ex(gg["dout"], gg["q"], gg["k"], gg["v"], lse, gg["seg"], pp, o32, gg["wq"], gg["wk"],
                               eps=EPS, scale=SCALE)
        torch.cuda.synchronize()
        return res

    base = run(g, pos)
    y, pos_y, p = shuffled(x, RAGGED, 3)
    say("[position] bwd_ex with o32, shuffled")
    got = run(to_dev(y), pos_y.cuda())
    pd = p.cuda()
    for a, b in zip(got[:3], base[:3]):
        assert bitwise_equal(a, b[pd])
    assert torch.equal(got[3], base[3]) and torch.equal(got[4], base[4])
