"""The C ABI library on a machine without a GPU: it loads, exports every declared symbol, and
rejects bad arguments synchronously before touching the device (strict mode: "unsupported shapes,
dtypes and devices raise instead of falling back", "33B forward/backward" page, Scope)."""
import ctypes
import os
import re

import pytest

import deterministic_invariant_attention_amd as h3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h3attn_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = h3.load()
    names = declared_functions()
    assert len(names) == 16
    for n in names:
        assert hasattr(lib, n), f"{n} missing from libh3attn.so"
    assert sorted(h3.EXPORTS) == names


def test_version_and_strerror():
    assert h3.h3attn_version() == 3
    for code in range(12):
        assert h3.h3attn_strerror(code)
    assert h3.h3attn_strerror(999) == "unknown status"


def test_workspace_bytes():
    assert h3.h3attn_workspace_bytes(0, 1) > 0
    n = h3.h3attn_workspace_bytes(8349, 40)
    assert n >= 2 * 8349 * 40 * 256
    assert n % 256 == 0
    assert h3.h3attn_workspace_bytes(-1, 4) == 0
    assert h3.h3attn_workspace_bytes(10, 0) == 0


# fake, suitably aligned addresses: every call below fails its checks before any pointer is used
A = 0x7F0000000000
P = ctypes.c_void_p


def fwd(lib, q=A, k=A + 0x1000000, v=A + 0x2000000, seg=A + 0x3000000, wq=A + 0x4000000, wk=A + 0x4001000, T=16,
        H=2, D=128, eps=1e-6, scale=0.088, out=A + 0x5000000, lse=None, ws=A + 0x6000000, wsb=None):
    if wsb is None:
        wsb = h3.h3attn_workspace_bytes(T, H) if T >= 0 and H >= 1 else 0
    return lib.h3attn_fwd(q, k, v, seg, wq, wk, T, H, D, eps, scale, out, lse, ws, wsb, None)


def test_fwd_argument_errors():
    lib = h3.load()
    assert fwd(lib, T=0) == h3.H3ATTN_OK                       # empty input is a no-op
    assert fwd(lib, T=-1) == h3.H3ATTN_ERR_SHAPE
    assert fwd(lib, H=0) == h3.H3ATTN_ERR_SHAPE
    assert fwd(lib, D=64) == h3.H3ATTN_ERR_SHAPE
    assert fwd(lib, scale=0.0) == h3.H3ATTN_ERR_SHAPE
    assert fwd(lib, scale=float("nan")) == h3.H3ATTN_ERR_SHAPE
    assert fwd(lib, eps=0.0) == h3.H3ATTN_ERR_SHAPE
    assert fwd(lib, T=2 ** 31) == h3.H3ATTN_ERR_SHAPE
    assert fwd(lib, q=None) == h3.H3ATTN_ERR_NULL
    assert fwd(lib, out=None) == h3.H3ATTN_ERR_NULL
    assert fwd(lib, seg=None) == h3.H3ATTN_ERR_NULL
    assert fwd(lib, wq=None) == h3.H3ATTN_ERR_NULL             # exactly one weight missing
    assert fwd(lib, wk=None) == h3.H3ATTN_ERR_NULL
    assert fwd(lib, q=A + 8) == h3.H3ATTN_ERR_ALIGN
    assert fwd(lib, out=A + 0x5000002) == h3.H3ATTN_ERR_ALIGN
    assert fwd(lib, ws=A + 0x6000010) == h3.H3ATTN_ERR_ALIGN
    assert fwd(lib, seg=A + 0x3000002) == h3.H3ATTN_ERR_ALIGN
    assert fwd(lib, out=A) == h3.H3ATTN_ERR_ALIAS              # out == q
    assert fwd(lib, out=A + 0x6000000 + 4096) == h3.H3ATTN_ERR_ALIAS   # out inside the workspace
    assert fwd(lib, wsb=1024) == h3.H3ATTN_ERR_WORKSPACE


def test_no_device_is_refused_not_faked():
    """With valid arguments and no GPU the library reports ERR_DEVICE (never a CPU fallback)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device path")
    lib = h3.load()
    assert fwd(lib) == h3.H3ATTN_ERR_DEVICE
    assert fwd(lib, wq=None, wk=None) == h3.H3ATTN_ERR_DEVICE
    n = 16 * 2 * 128 * 2
    assert lib.h3attn_qknorm(A, A + 0x100000, A + 0x200000, 16, 2, 128, 1e-6, None) == h3.H3ATTN_ERR_DEVICE
    assert lib.h3attn_qknorm(A, A + 0x100000, A + n // 2, 16, 2, 128, 1e-6, None) == h3.H3ATTN_ERR_ALIAS
    assert lib.h3attn_qknorm(A, A + 0x100000, A, 16, 2, 128, 1e-6, None) == h3.H3ATTN_ERR_DEVICE  # in place is fine


def test_staged_calls_check_arguments():
    lib = h3.load()
    wsb = h3.h3attn_workspace_bytes(16, 2)
    assert lib.h3attn_plan(None, 16, 2, A, wsb, None) == h3.H3ATTN_ERR_NULL
    assert lib.h3attn_plan(A, 16, 2, A + 0x1000000, 8, None) == h3.H3ATTN_ERR_WORKSPACE
    assert lib.h3attn_prep_qkv(A, A, None, None, None, 16, 2, 128, 1e-6, A + 0x1000000, wsb, None) == h3.H3ATTN_ERR_NULL
    assert lib.h3attn_prep_qkv(A, A, A, A + 0x100000, None, 16, 2, 128, 1e-6, A + 0x1000000, wsb,
                               None) == h3.H3ATTN_ERR_NULL   # exactly one weight
    assert lib.h3attn_prep_qkv(A, A, A, None, None, 16, 2, 128, 1e-6, A + 0x1000000, 64, None) == h3.H3ATTN_ERR_WORKSPACE
    assert lib.h3attn_prep_qkv(A + 0x1000000 + 512, A, A, None, None, 16, 2, 128, 1e-6, A + 0x1000000, wsb,
                               None) == h3.H3ATTN_ERR_ALIAS  # q inside the workspace
    assert lib.h3attn_attend(A, None, 16, 2, 128, 1e-6, -1.0, A + 0x100000, None, A + 0x1000000, wsb,
                             None) == h3.H3ATTN_ERR_SHAPE
    st = ctypes.c_int32(0)
    assert lib.h3attn_status_read(None, ctypes.byref(st), None) == h3.H3ATTN_ERR_NULL
    assert lib.h3attn_status_read(A + 4, ctypes.byref(st), None) == h3.H3ATTN_ERR_ALIGN


def bwd(lib, dout=A + 0x7000000, q=A, k=A + 0x1000000, v=A + 0x2000000, lse=A + 0x8000000, seg=A + 0x3000000,
        wq=A + 0x4000000, wk=A + 0x4001000, T=16, H=2, D=128, eps=1e-6, scale=0.088, dq=A + 0x9000000,
        dk=A + 0xA000000, dv=A + 0xB000000, dwq=A + 0xC000000, dwk=A + 0xC001000, ws=A + 0x10000000, wsb=None):
    if wsb is None:
        wsb = h3.h3attn_bwd_workspace_bytes(T, H) if T >= 0 and H >= 1 else 0
    return lib.h3attn_bwd(dout, q, k, v, lse, seg, wq, wk, T, H, D, eps, scale, dq, dk, dv, dwq, dwk, ws, wsb, None)


def fwd_pos(lib, pos=A + 0xD000000, q=A, k=A + 0x1000000, v=A + 0x2000000, seg=A + 0x3000000, wq=A + 0x4000000,
            wk=A + 0x4001000, T=16, H=2, D=128, eps=1e-6, scale=0.088, out=A + 0x5000000, lse=None, ws=A + 0x6000000,
            wsb=None):
    if wsb is None:
        wsb = h3.h3attn_workspace_bytes(T, H) if T >= 0 and H >= 1 else 0
    return lib.h3attn_fwd_pos(q, k, v, seg, pos, wq, wk, T, H, D, eps, scale, out, lse, ws, wsb, None)


def test_fwd_pos_argument_errors():
    lib = h3.load()
    assert fwd_pos(lib, T=0) == h3.H3ATTN_OK
    assert fwd_pos(lib, pos=None) == h3.H3ATTN_ERR_NULL
    assert fwd_pos(lib, pos=A + 0xD000002) == h3.H3ATTN_ERR_ALIGN
    assert fwd_pos(lib, out=A + 0xD000000 - 64) == h3.H3ATTN_ERR_ALIAS     # out runs into pos_ids
    assert fwd_pos(lib, lse=A + 0xD000000 + 16) == h3.H3ATTN_ERR_ALIAS     # lse overlaps pos_ids
    assert fwd_pos(lib, pos=A + 0x6000000 + 256) == h3.H3ATTN_ERR_ALIAS    # pos_ids inside the workspace
    assert fwd_pos(lib, D=64) == h3.H3ATTN_ERR_SHAPE
    assert fwd_pos(lib, wq=None) == h3.H3ATTN_ERR_NULL
    # the position order needs the two int32 [T] maps beyond the plain forward's workspace
    full = h3.h3attn_workspace_bytes(16, 2)
    assert fwd_pos(lib, wsb=full - 512) == h3.H3ATTN_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        assert fwd(lib, wsb=full - 512) == h3.H3ATTN_ERR_DEVICE   # enough for the plain forward
        assert fwd_pos(lib) == h3.H3ATTN_ERR_DEVICE
        assert fwd_pos(lib, wq=None, wk=None) == h3.H3ATTN_ERR_DEVICE


def test_bwd_workspace_bytes():
    n = h3.h3attn_bwd_workspace_bytes(8506, 40)
    assert n >= 7 * 8506 * 40 * 256 + 2 * 8506 * 40 * 4 and n % 256 == 0
    assert h3.h3attn_bwd_workspace_bytes(-1, 4) == 0 and h3.h3attn_bwd_workspace_bytes(10, 0) == 0


def test_bwd_argument_errors():
    lib = h3.load()
    assert bwd(lib, T=0) == h3.H3ATTN_OK
    assert bwd(lib, T=-1) == h3.H3ATTN_ERR_SHAPE
    assert bwd(lib, D=64) == h3.H3ATTN_ERR_SHAPE
    assert bwd(lib, scale=0.0) == h3.H3ATTN_ERR_SHAPE
    assert bwd(lib, eps=float("inf")) == h3.H3ATTN_ERR_SHAPE
    assert bwd(lib, lse=None) == h3.H3ATTN_ERR_NULL
    assert bwd(lib, dout=None) == h3.H3ATTN_ERR_NULL
    assert bwd(lib, dwq=None) == h3.H3ATTN_ERR_NULL              # weights given, gradient missing
    assert bwd(lib, wk=None) == h3.H3ATTN_ERR_NULL               # exactly one weight missing
    assert bwd(lib, dq=A + 0x9000008) == h3.H3ATTN_ERR_ALIGN
    assert bwd(lib, lse=A + 0x8000002) == h3.H3ATTN_ERR_ALIGN
    assert bwd(lib, dk=A) == h3.H3ATTN_ERR_ALIAS                  # dk == q
    assert bwd(lib, dv=A + 0x9000000) == h3.H3ATTN_ERR_ALIAS      # dv == dq
    assert bwd(lib, dwq=A + 0x10000000 + 512) == h3.H3ATTN_ERR_ALIAS  # inside the workspace
    assert bwd(lib, wsb=4096) == h3.H3ATTN_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        assert bwd(lib) == h3.H3ATTN_ERR_DEVICE
        assert bwd(lib, wq=None, wk=None, dwq=None, dwk=None) == h3.H3ATTN_ERR_DEVICE


def bwd_pos(lib, pos=A + 0xD000000, T=16, H=2, wsb=None, **kw):
    args = dict(dout=A + 0x7000000, q=A, k=A + 0x1000000, v=A + 0x2000000, lse=A + 0x8000000, seg=A + 0x3000000,
                wq=A + 0x4000000, wk=A + 0x4001000, D=128, eps=1e-6, scale=0.088, dq=A + 0x9000000, dk=A + 0xA000000,
                dv=A + 0xB000000, dwq=A + 0xC000000, dwk=A + 0xC001000, ws=A + 0x10000000)
    args.update(kw)
    if wsb is None:
        wsb = h3.h3attn_bwd_workspace_bytes(T, H) if T >= 0 and H >= 1 else 0
    a = args
    return lib.h3attn_bwd_pos(a["dout"], a["q"], a["k"], a["v"], a["lse"], a["seg"], pos, a["wq"], a["wk"], T, H,
                              a["D"], a["eps"], a["scale"], a["dq"], a["dk"], a["dv"], a["dwq"], a["dwk"], a["ws"], wsb,
                              None)


def test_bwd_pos_argument_errors():
    lib = h3.load()
    assert bwd_pos(lib, T=0) == h3.H3ATTN_OK
    assert bwd_pos(lib, pos=None) == h3.H3ATTN_ERR_NULL
    assert bwd_pos(lib, pos=A + 0xD000001) == h3.H3ATTN_ERR_ALIGN
    assert bwd_pos(lib, dq=A + 0xD000000) == h3.H3ATTN_ERR_ALIAS           # an output on pos_ids
    assert bwd_pos(lib, pos=A + 0x10000000 + 1024) == h3.H3ATTN_ERR_ALIAS  # pos_ids inside the workspace
    full = h3.h3attn_bwd_workspace_bytes(16, 2)
    assert bwd_pos(lib, wsb=full - 512) == h3.H3ATTN_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        assert bwd(lib, wsb=full - 512) == h3.H3ATTN_ERR_DEVICE   # enough for the plain backward
        assert bwd_pos(lib) == h3.H3ATTN_ERR_DEVICE


def test_ex_argument_errors():
    """h3attn_fwd_ex / h3attn_bwd_ex: the optional fp32 output is checked like any other buffer."""
    lib = h3.load()
    wsb = h3.h3attn_workspace_bytes(16, 2)
    O32 = A + 0xE000000
    n = 16 * 2 * 128 * 2

    def fx(pos=None, o32=O32, out=A + 0x5000000, lse=None, T=16, rc=None, rs=None, wq=A + 0x4000000, wk=A + 0x4001000):
        return lib.h3attn_fwd_ex(A, A + 0x1000000, A + 0x2000000, A + 0x3000000, pos, wq, wk, rc, rs,
                                 T, 2, 128, 1e-6, 0.088, out, lse, o32, A + 0x6000000, wsb, None)

    assert fx(T=0) == h3.H3ATTN_OK
    assert fx(o32=O32 + 4) == h3.H3ATTN_ERR_ALIGN
    assert fx(o32=A + 0x5000000 - 64) == h3.H3ATTN_ERR_ALIAS          # runs into out
    assert fx(o32=A + 0x1000000 + n - 16) == h3.H3ATTN_ERR_ALIAS      # overlaps k
    assert fx(o32=A + 0x6000000 + 256) == h3.H3ATTN_ERR_ALIAS         # inside the workspace
    assert fx(lse=O32 + 1024) == h3.H3ATTN_ERR_ALIAS                  # lse inside o32
    assert fx(pos=A + 0xD000002) == h3.H3ATTN_ERR_ALIGN
    bwsb = h3.h3attn_bwd_workspace_bytes(16, 2)

    def bx(o32=O32, pos=None, dq=A + 0x9000000, rc=None, rs=None):
        return lib.h3attn_bwd_ex(A + 0x7000000, A, A + 0x1000000, A + 0x2000000, A + 0x8000000, o32, A + 0x3000000,
                                 pos, A + 0x4000000, A + 0x4001000, rc, rs, 16, 2, 128, 1e-6, 0.088, dq, A + 0xA000000,
                                 A + 0xB000000, A + 0xC000000, A + 0xC001000, A + 0x10000000, bwsb, None)

    assert bx(o32=O32 + 8) == h3.H3ATTN_ERR_ALIGN
    assert bx(dq=O32) == h3.H3ATTN_ERR_ALIAS                          # an output on o32
    assert bx(o32=A + 0x10000000 + 512) == h3.H3ATTN_ERR_ALIAS        # o32 inside the workspace
    R = A + 0xF000000  # rope tables: float32 [16, 48] each
    assert fx(rc=R) == h3.H3ATTN_ERR_NULL                             # one table only
    assert fx(rc=R, rs=R + 4096, wq=None, wk=None) == h3.H3ATTN_ERR_NULL  # rope needs the norm weights
    assert fx(rc=R + 4, rs=R + 4096) == h3.H3ATTN_ERR_ALIGN
    assert fx(rc=R, rs=R + 4096, o32=R + 1024) == h3.H3ATTN_ERR_ALIAS  # an output on a table
    assert bx(rc=R + 8, rs=R + 4096) == h3.H3ATTN_ERR_ALIGN
    assert bx(rc=R, rs=R + 4096, dq=R + 2048) == h3.H3ATTN_ERR_ALIAS
    import torch
    if not torch.cuda.is_available():
        assert fx() == h3.H3ATTN_ERR_DEVICE and fx(o32=None) == h3.H3ATTN_ERR_DEVICE
        assert fx(pos=A + 0xD000000) == h3.H3ATTN_ERR_DEVICE
        assert fx(rc=A + 0xF000000, rs=A + 0xF001000) == h3.H3ATTN_ERR_DEVICE
        assert bx(rc=A + 0xF000000, rs=A + 0xF001000) == h3.H3ATTN_ERR_DEVICE
        assert bx() == h3.H3ATTN_ERR_DEVICE and bx(o32=None) == h3.H3ATTN_ERR_DEVICE


def test_fwd_noalloc_argument_errors():
    """The allocation-free forward: sizes beyond its static scratch, NULLs and misaligned status are
    refused before anything touches a device; without a GPU, valid arguments give ERR_DEVICE."""
    import torch
    lib = h3.load()

    def na(T=16, H=2, q=A, out=A + 0x5000000, status=None, D=128):
        return lib.h3attn_fwd_noalloc(q, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, A + 0x4001000,
                                      T, H, D, 1e-6, 0.088, out, None, status, None)

    assert na(T=0) == h3.H3ATTN_OK
    assert na(T=16384, H=40) == h3.H3ATTN_ERR_SCRATCH       # 480 MiB of workspace > 256 MiB
    assert h3.h3attn_workspace_bytes(8349, 40) <= 256 << 20   # the 8349 x 40 workload fits
    assert na(D=64) == h3.H3ATTN_ERR_SHAPE
    assert na(q=None) == h3.H3ATTN_ERR_NULL and na(out=None) == h3.H3ATTN_ERR_NULL
    assert na(status=A + 0x7000002) == h3.H3ATTN_ERR_ALIGN
    assert na(status=A + 0x5000000 + 64) == h3.H3ATTN_ERR_ALIAS   # status inside out
    if not torch.cuda.is_available():
        assert na() == h3.H3ATTN_ERR_DEVICE and na(status=A + 0x7000000) == h3.H3ATTN_ERR_DEVICE
