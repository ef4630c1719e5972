"""Streams: the binding on a side stream (its allocations ride on the launch stream), a raw
hipStream_t handle, the status check option, and bitwise repeatability while another stream keeps
the compute units busy (the rollout-vs-train property must not depend on occupancy: "33B
forward/backward and rollout-vs-train control" page, dual-trajectory results)."""
import pytest
import torch

import deterministic_invariant_attention_amd as h3
import workloads
from gpu_util import EPS, bitwise_equal, say, to_dev

pytestmark = pytest.mark.gpu


def fwd_bwd(g, stream=None):
    out, lse, o32 = h3.h3attn_fwd_ex(g["q"], g["k"], g["v"], g["seg"], None, g["wq"], g["wk"], eps=EPS,
                                     want_lse=True, want_o32=True, stream=stream)
    grads = h3.h3attn_bwd_ex(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], None, o32, g["wq"], g["wk"], eps=EPS,
                             stream=stream)
    return [out, lse, *grads]


def test_side_stream_and_raw_handle_give_the_same_bits():
    g = to_dev(workloads.make_inputs(workloads.WORKLOADS["short3"], with_grad=True))
    say("[streams] short3 fwd+bwd: current stream, side stream, raw handle")
    ref = fwd_bwd(g)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    got = fwd_bwd(g, stream=side)
    # allocations on the current stream right away: the binding's buffers belong to the side stream,
    # so the allocator cannot hand them out while its kernels may still run
    junk = [torch.full((1 << 22,), 7.0, device="cuda") for _ in range(8)]
    raw = fwd_bwd(g, stream=side.cuda_stream)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    for a, b, c in zip(ref, got, raw):
        assert bitwise_equal(a, b) and bitwise_equal(a, c)


def test_check_status_raises_on_a_data_error():
    x = workloads.random_inputs([40, 40], 2, seed=3, with_grad=True)
    x["v"][50, 1, 9] = 1.0e5  # beyond the fp16 range of the P.V operand
    g = to_dev(x)
    with pytest.raises(h3.H3AttnError) as e:
        h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], g["wq"], g["wk"], eps=EPS, check_status=True)
    assert e.value.code == h3.H3ATTN_ERR_RANGE
    ok = to_dev(workloads.random_inputs([40, 40], 2, seed=3))
    h3.h3attn_fwd(ok["q"], ok["k"], ok["v"], ok["seg"], ok["wq"], ok["wk"], eps=EPS, check_status=True)


def test_repeat_bitwise_under_concurrent_load():
    """batch2 forward and backward (both ways of forming D) while a second stream of the same
    priority runs long fp32 matrix products: the persistent grids then start on whatever compute
    units are free, in whatever order.  Every output must keep the bits of a quiet run."""
    wl = workloads.WORKLOADS["batch2"]
    g = to_dev(workloads.make_inputs(wl, with_grad=True))
    say("[streams] batch2 fwd+bwd quiet reference")
    quiet = [t.clone() for t in fwd_bwd(g)]
    _, lse = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], g["wq"], g["wk"], eps=EPS, want_lse=True)
    quiet_rec = [t.clone() for t in h3.h3attn_bwd(g["dout"], g["q"], g["k"], g["v"], lse, g["seg"], g["wq"], g["wk"],
                                                  eps=EPS)]
    torch.cuda.synchronize()
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.randn(4096, 4096, device="cuda")
    load = torch.cuda.Stream()  # default priority
    for rep in range(3):
        say(f"[streams] batch2 under load, repetition {rep}")
        load.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(load):
            c = a
            for _ in range(12):
                c = torch.mm(c, b) * 1e-3
        got = fwd_bwd(g)
        _, lse2 = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], g["wq"], g["wk"], eps=EPS, want_lse=True)
        rec = h3.h3attn_bwd(g["dout"], g["q"], g["k"], g["v"], lse2, g["seg"], g["wq"], g["wk"], eps=EPS)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(got, quiet)):
            assert bitwise_equal(x, y), f"output {i} (o32 path) differs under load, repetition {rep}"
        for i, (x, y) in enumerate(zip(rec, quiet_rec)):
            assert bitwise_equal(x, y), f"gradient {i} (recomputed D) differs under load, repetition {rep}"
