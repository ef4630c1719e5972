"""The Python binding checks every tensor argument before the library sees a pointer (CPU only).

A tensor of the wrong shape, dtype or device would hand the kernels an undersized buffer or a host
address; strict mode ("33B forward/backward" page, Scope: unsupported shapes, dtypes and devices
raise) makes each such call raise.  Every case here must raise before any compute entry point of
the library is reached: the library object is replaced by one that fails the test on such a call.
"""
import pytest
import torch

import deterministic_invariant_attention_amd as h3

T, H, D = 12, 2, 128
HOST_QUERIES = ("h3attn_workspace_bytes", "h3attn_bwd_workspace_bytes", "h3attn_strerror", "h3attn_version")


class _GuardLib:
    """Passes the host-only size and message queries through; any other entry point fails."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in HOST_QUERIES:
            return getattr(self._real, name)
        raise AssertionError(f"the library's {name} was reached with invalid arguments")


@pytest.fixture(autouse=True)
def guard(monkeypatch):
    real = h3.load()
    monkeypatch.setattr(h3, "_lib", _GuardLib(real))
    yield


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def args(**kw):
    a = dict(q=bf(T, H, D), k=bf(T, H, D), v=bf(T, H, D), seg_ids=torch.zeros(T, dtype=torch.int32),
             wq=bf(D), wk=bf(D))
    a.update(kw)
    return a


def code(fn, *a, **kw):
    with pytest.raises(h3.H3AttnError) as e:
        fn(*a, **kw)
    return e.value.code


@pytest.mark.parametrize("bad", [
    dict(k=bf(T - 1, H, D)), dict(v=bf(T, H + 1, D)), dict(seg_ids=torch.zeros(T + 1, dtype=torch.int32)),
    dict(wq=bf(64)), dict(wk=bf(D, 1)), dict(out=bf(T, H, 64)), dict(lse=torch.zeros(T, dtype=torch.float32)),
    dict(q=bf(T, H, 64), k=bf(T, H, 64), v=bf(T, H, 64)),
])
def test_fwd_shape_mismatch_raises(bad):
    assert code(h3.h3attn_fwd, **args(**bad)) == h3.H3ATTN_ERR_SHAPE


def test_fwd_variants_check_their_extra_tensors():
    assert code(h3.h3attn_fwd_pos, **args(), pos_ids=torch.zeros(T - 2, dtype=torch.int32)) == h3.H3ATTN_ERR_SHAPE
    assert code(h3.h3attn_fwd_ex, **args(), o32=torch.zeros(T, H, D - 1)) == h3.H3ATTN_ERR_SHAPE
    small = torch.zeros(64, dtype=torch.uint8)
    assert code(h3.h3attn_fwd, **args(), workspace_buf=small) == h3.H3ATTN_ERR_WORKSPACE


def test_fwd_dtype_and_layout_raise():
    with pytest.raises(TypeError):
        h3.h3attn_fwd(**args(k=torch.zeros(T, H, D, dtype=torch.float16)))
    with pytest.raises(TypeError):
        h3.h3attn_fwd(**args(seg_ids=torch.zeros(T, dtype=torch.int64)))
    with pytest.raises(TypeError):
        h3.h3attn_fwd(**args(v=bf(T, D, H).transpose(1, 2)))
    with pytest.raises(TypeError):
        h3.h3attn_fwd_ex(**args(), o32=torch.zeros(T, H, D, dtype=torch.float64))


def test_host_tensors_raise_device_error():
    """Valid shapes on the CPU (or on no device at all) are refused: no host address reaches a kernel."""
    assert code(h3.h3attn_fwd, **args()) == h3.H3ATTN_ERR_DEVICE
    meta = {n: (t.to("meta") if n == "q" else t) for n, t in args().items()}
    assert code(h3.h3attn_fwd, **meta) == h3.H3ATTN_ERR_DEVICE
    assert code(h3.h3attn_qknorm, bf(T, H, D), bf(D)) == h3.H3ATTN_ERR_DEVICE
    assert code(h3.h3attn_plan, torch.zeros(T, dtype=torch.int32), H,
                torch.zeros(h3.h3attn_workspace_bytes(T, H), dtype=torch.uint8)) == h3.H3ATTN_ERR_DEVICE


def test_qknorm_and_staged_calls_check_shapes():
    assert code(h3.h3attn_qknorm, bf(T, H, D), bf(D + 1)) == h3.H3ATTN_ERR_SHAPE
    assert code(h3.h3attn_qknorm, bf(T, H, D), bf(D), out=bf(T, H - 1, D)) == h3.H3ATTN_ERR_SHAPE
    ws = torch.zeros(h3.h3attn_workspace_bytes(T, H), dtype=torch.uint8)
    assert code(h3.h3attn_prep_qkv, bf(T, H, D), bf(T, H, D), bf(T - 1, H, D), None, None, ws) == h3.H3ATTN_ERR_SHAPE
    assert code(h3.h3attn_attend, bf(T, H, D), None, ws, bf(T, H, D), lse=torch.zeros(T, H + 1)) == h3.H3ATTN_ERR_SHAPE
    assert code(h3.h3attn_attend, bf(T, H, D), None, ws[:100], bf(T, H, D)) == h3.H3ATTN_ERR_WORKSPACE
    assert code(h3.h3attn_plan, torch.zeros(T, dtype=torch.int32), H, ws[:100]) == h3.H3ATTN_ERR_WORKSPACE


def bargs(**kw):
    a = dict(dout=bf(T, H, D), q=bf(T, H, D), k=bf(T, H, D), v=bf(T, H, D), lse=torch.zeros(T, H),
             seg_ids=torch.zeros(T, dtype=torch.int32), wq=bf(D), wk=bf(D))
    a.update(kw)
    return a


@pytest.mark.parametrize("bad", [
    dict(dout=bf(T, H, D - 8)), dict(lse=torch.zeros(T, H, 1)), dict(seg_ids=torch.zeros(T - 1, dtype=torch.int32)),
    dict(dq=bf(T + 1, H, D)), dict(dk=bf(T, H, 1)), dict(dv=bf(1, H, D)), dict(dwq=torch.zeros(D - 1)),
    dict(dwk=torch.zeros(2, D)), dict(k=bf(T, 1, D)),
])
def test_bwd_shape_mismatch_raises(bad):
    assert code(h3.h3attn_bwd, **bargs(**bad)) == h3.H3ATTN_ERR_SHAPE


def test_bwd_variants_and_devices():
    assert code(h3.h3attn_bwd_pos, **bargs(), pos_ids=torch.zeros(T + 3, dtype=torch.int32)) == h3.H3ATTN_ERR_SHAPE
    assert code(h3.h3attn_bwd_ex, **bargs(), o32=torch.zeros(T, H)) == h3.H3ATTN_ERR_SHAPE
    assert code(h3.h3attn_bwd, **bargs(lse=None)) == h3.H3ATTN_ERR_NULL
    assert code(h3.h3attn_bwd, **bargs(), workspace_buf=torch.zeros(8, dtype=torch.uint8)) == h3.H3ATTN_ERR_WORKSPACE
    assert code(h3.h3attn_bwd, **bargs()) == h3.H3ATTN_ERR_DEVICE
    with pytest.raises(TypeError):
        h3.h3attn_bwd(**bargs(lse=torch.zeros(T, H, dtype=torch.float64)))
