"""The allocation-free forward (h3attn_fwd_noalloc) through the C ABI: on the library's static
scratch it gives the bits of h3attn_fwd, call after call, with a smaller input after a larger one
(the scratch keeps the previous call's contents), reports data errors in its status output, and
refuses sizes beyond the scratch before doing anything."""
import pytest
import torch

import deterministic_invariant_attention_amd as h3
import workloads
from gpu_util import EPS, bitwise_equal, say, to_dev

pytestmark = pytest.mark.gpu


def both(g):
    ref, rlse = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], g["wq"], g["wk"], eps=EPS, want_lse=True)
    out = torch.empty_like(g["q"])
    lse = torch.empty_like(rlse)
    status = torch.full((1,), -1, dtype=torch.int32, device=g["q"].device)
    h3.h3attn_fwd_noalloc(g["q"], g["k"], g["v"], g["seg"], g["wq"], g["wk"], out, lse=lse, status=status, eps=EPS)
    torch.cuda.synchronize()
    return ref, rlse, out, lse, int(status.item())


def test_noalloc_matches_fwd_larger_then_smaller():
    for name in ("batch2", "short3", "tiny"):
        g = to_dev(workloads.make_inputs(workloads.WORKLOADS[name]))
        say(f"[noalloc] {name}: T={g['q'].shape[0]} H={g['q'].shape[1]}")
        ref, rlse, out, lse, st = both(g)
        assert st == h3.H3ATTN_OK
        assert bitwise_equal(out, ref) and bitwise_equal(lse, rlse)


def test_noalloc_status_and_recovery():
    x = workloads.random_inputs([40, 40], 2, seed=53)
    x["v"][10, 1, 5] = 1.0e5  # beyond fp16: segment 0 fails closed
    g = to_dev(x)
    say("[noalloc] data error, then a clean call on the same scratch")
    ref, rlse, out, lse, st = both(g)
    assert st == h3.H3ATTN_ERR_RANGE
    assert torch.isnan(out[:40].float()).all() and bitwise_equal(out, ref) and bitwise_equal(lse, rlse)
    g = to_dev(workloads.random_inputs([33, 7], 2, seed=54))
    ref, rlse, out, lse, st = both(g)
    assert st == h3.H3ATTN_OK and bitwise_equal(out, ref) and bitwise_equal(lse, rlse)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    T, H = 16384, 40
    q = torch.zeros((T, H, 128), dtype=torch.bfloat16, device="cuda:0")
    seg = torch.zeros(T, dtype=torch.int32, device="cuda:0")
    w = torch.ones(128, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(h3.H3AttnError) as e:
        h3.h3attn_fwd_noalloc(q, q, q, seg, w, w, torch.empty_like(q))
    assert e.value.code == h3.H3ATTN_ERR_SCRATCH
