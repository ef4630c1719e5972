"""Deterministic, batch-invariant H3 full attention for MI355X (gfx950).

A thin ctypes binding of ``libh3attn.so`` (C ABI in ``include/h3attn.h``).  The functions keep the
C names and only marshal arguments: torch provides device memory and the stream, every step of the
computation runs in the library's HIP kernels.  There is no other code path: if the library is not
built, or the tensors are not on a gfx950 device, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libh3attn.so")
HEAD_DIM = 128

H3ATTN_OK = 0
H3ATTN_ERR_NULL = 1
H3ATTN_ERR_SHAPE = 2
H3ATTN_ERR_ALIGN = 3
H3ATTN_ERR_ALIAS = 4
H3ATTN_ERR_WORKSPACE = 5
H3ATTN_ERR_DEVICE = 6
H3ATTN_ERR_LAUNCH = 7
H3ATTN_ERR_SEGMENTS = 8
H3ATTN_ERR_RANGE = 9
H3ATTN_ERR_POSITIONS = 10

# every symbol the header declares
EXPORTS = ("h3attn_version", "h3attn_strerror", "h3attn_workspace_bytes", "h3attn_qknorm", "h3attn_fwd",
           "h3attn_fwd_pos", "h3attn_fwd_ex", "h3attn_plan", "h3attn_prep_qkv", "h3attn_attend", "h3attn_status_read",
           "h3attn_bwd_workspace_bytes", "h3attn_bwd", "h3attn_bwd_pos", "h3attn_bwd_ex")


class H3AttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {h3attn_strerror(code)} (status {code})")


_lib = None


def load():
    """Load libh3attn.so (built in-tree by __graft_entry__.build()); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.h3attn_version.restype = ctypes.c_int
    lib.h3attn_strerror.argtypes = [ctypes.c_int]
    lib.h3attn_strerror.restype = ctypes.c_char_p
    lib.h3attn_workspace_bytes.argtypes = [I64, I32]
    lib.h3attn_workspace_bytes.restype = SZ
    lib.h3attn_qknorm.argtypes = [P, P, P, I64, I32, I32, F, P]
    lib.h3attn_fwd.argtypes = [P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, SZ, P]
    lib.h3attn_fwd_pos.argtypes = [P, P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, SZ, P]
    lib.h3attn_fwd_ex.argtypes = [P, P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, P, SZ, P]
    lib.h3attn_plan.argtypes = [P, I64, I32, P, SZ, P]
    lib.h3attn_prep_qkv.argtypes = [P, P, P, P, P, I64, I32, I32, F, P, SZ, P]
    lib.h3attn_attend.argtypes = [P, P, I64, I32, I32, F, F, P, P, P, SZ, P]
    lib.h3attn_status_read.argtypes = [P, ctypes.POINTER(ctypes.c_int32), P]
    lib.h3attn_bwd_workspace_bytes.argtypes = [I64, I32]
    lib.h3attn_bwd_workspace_bytes.restype = SZ
    lib.h3attn_bwd.argtypes = [P, P, P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, P, P, P, SZ, P]
    lib.h3attn_bwd_pos.argtypes = [P, P, P, P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, P, P, P, SZ, P]
    lib.h3attn_bwd_ex.argtypes = [P, P, P, P, P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, P, P, P, SZ, P]
    for name in ("h3attn_qknorm", "h3attn_fwd", "h3attn_fwd_pos", "h3attn_fwd_ex", "h3attn_plan", "h3attn_prep_qkv",
                 "h3attn_attend", "h3attn_status_read", "h3attn_bwd", "h3attn_bwd_pos", "h3attn_bwd_ex"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int, where: str):
    if rc != H3ATTN_OK:
        raise H3AttnError(rc, where)


def _shape(q):
    if q.dim() != 3:
        raise H3AttnError(H3ATTN_ERR_SHAPE, "expected [tokens, heads, head_dim]")
    return q.shape[0], q.shape[1], q.shape[2]


def _bf16(t, name):
    if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous bfloat16 tensor")
    return t


def h3attn_version() -> int:
    return load().h3attn_version()


def h3attn_strerror(code: int) -> str:
    return load().h3attn_strerror(int(code)).decode()


def h3attn_workspace_bytes(tokens: int, heads: int) -> int:
    return load().h3attn_workspace_bytes(int(tokens), int(heads))


def workspace(tokens: int, heads: int, device) -> torch.Tensor:
    """A device buffer of h3attn_workspace_bytes(tokens, heads) bytes (torch's allocator is 256-B aligned)."""
    n = h3attn_workspace_bytes(tokens, heads)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def h3attn_qknorm(x, w, eps: float = 1e-6, out=None, stream=None):
    """RMSNorm of every 128-wide (token, head) row of x [T, H, 128] with weight w [128]; returns y."""
    _bf16(x, "x"), _bf16(w, "w")
    T, H, D = _shape(x)
    y = torch.empty_like(x) if out is None else _bf16(out, "out")
    rc = load().h3attn_qknorm(_ptr(x), _ptr(w), _ptr(y), T, H, D, float(eps), _stream(stream, x.device))
    _check(rc, "h3attn_qknorm")
    return y


def _int32(t, name):
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    return t


def h3attn_fwd(q, k, v, seg_ids, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None, out=None,
               lse=None, workspace_buf=None, stream=None, want_lse: bool = False):
    """Forward of the attention node with its fused q/k norm.  Returns (out, lse) (lse None unless asked)."""
    return _fwd(q, k, v, seg_ids, None, wq, wk, eps, scale, out, lse, workspace_buf, stream, want_lse)


def h3attn_fwd_pos(q, k, v, seg_ids, pos_ids, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None,
                   out=None, lse=None, workspace_buf=None, stream=None, want_lse: bool = False):
    """h3attn_fwd with each segment's keys walked in the order of pos_ids (int32 [T], a permutation of
    0..L-1 within each segment).  Returns (out, lse)."""
    return _fwd(q, k, v, seg_ids, _int32(pos_ids, "pos_ids"), wq, wk, eps, scale, out, lse, workspace_buf, stream,
                want_lse)


def h3attn_fwd_ex(q, k, v, seg_ids, pos_ids=None, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None,
                  out=None, lse=None, o32=None, workspace_buf=None, stream=None, want_lse: bool = False,
                  want_o32: bool = False):
    """The forward with every option: position order when pos_ids is given, and the fp32 output
    before its bf16 rounding (o32, for h3attn_bwd_ex) when asked.  Returns (out, lse, o32)."""
    T = q.shape[0]
    if o32 is None and want_o32:
        o32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if o32 is not None and (o32.dtype != torch.float32 or not o32.is_contiguous()):
        raise TypeError("o32 must be a contiguous float32 tensor")
    out, lse = _fwd(q, k, v, seg_ids, None if pos_ids is None else _int32(pos_ids, "pos_ids"), wq, wk, eps, scale,
                    out, lse, workspace_buf, stream, want_lse, o32=o32, ex=True)
    return out, lse, o32


def _fwd(q, k, v, seg_ids, pos_ids, wq, wk, eps, scale, out, lse, workspace_buf, stream, want_lse, o32=None,
         ex=False):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (wq, "wq"), (wk, "wk")):
        _bf16(t, n)
    _int32(seg_ids, "seg_ids")
    T, H, D = _shape(q)
    scale = D ** -0.5 if scale is None else scale
    out = torch.empty_like(q) if out is None else _bf16(out, "out")
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    ws = workspace(T, H, q.device) if workspace_buf is None else workspace_buf
    st = _stream(stream, q.device)
    if ex:
        rc = load().h3attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(seg_ids), _ptr(pos_ids), _ptr(wq), _ptr(wk), T, H,
                                  D, float(eps), float(scale), _ptr(out), _ptr(lse), _ptr(o32), _ptr(ws), ws.numel(),
                                  st)
        _check(rc, "h3attn_fwd_ex")
    elif pos_ids is None:
        rc = load().h3attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(seg_ids), _ptr(wq), _ptr(wk), T, H, D, float(eps),
                               float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), st)
        _check(rc, "h3attn_fwd")
    else:
        rc = load().h3attn_fwd_pos(_ptr(q), _ptr(k), _ptr(v), _ptr(seg_ids), _ptr(pos_ids), _ptr(wq), _ptr(wk), T, H,
                                   D, float(eps), float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), st)
        _check(rc, "h3attn_fwd_pos")
    return out, lse


def h3attn_plan(seg_ids, heads: int, workspace_buf, stream=None):
    T = seg_ids.shape[0]
    rc = load().h3attn_plan(_ptr(seg_ids), T, int(heads), _ptr(workspace_buf), workspace_buf.numel(),
                            _stream(stream, seg_ids.device))
    _check(rc, "h3attn_plan")


def h3attn_prep_qkv(q, k, v, wq, wk, workspace_buf, eps: float = 1e-6, stream=None):
    T, H, D = _shape(k)
    rc = load().h3attn_prep_qkv(_ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), T, H, D, float(eps),
                                _ptr(workspace_buf), workspace_buf.numel(), _stream(stream, k.device))
    _check(rc, "h3attn_prep_qkv")


def h3attn_attend(q, wq, workspace_buf, out, lse=None, eps: float = 1e-6, scale: float | None = None, stream=None):
    T, H, D = _shape(q)
    scale = D ** -0.5 if scale is None else scale
    rc = load().h3attn_attend(_ptr(q), _ptr(wq), T, H, D, float(eps), float(scale), _ptr(out), _ptr(lse),
                              _ptr(workspace_buf), workspace_buf.numel(), _stream(stream, q.device))
    _check(rc, "h3attn_attend")
    return out


def h3attn_status_read(workspace_buf, stream=None) -> int:
    st = ctypes.c_int32(-1)
    rc = load().h3attn_status_read(_ptr(workspace_buf), ctypes.byref(st), _stream(stream, workspace_buf.device))
    _check(rc, "h3attn_status_read")
    return st.value


def h3attn_bwd_workspace_bytes(tokens: int, heads: int) -> int:
    return load().h3attn_bwd_workspace_bytes(int(tokens), int(heads))


def bwd_workspace(tokens: int, heads: int, device) -> torch.Tensor:
    """A device buffer of h3attn_bwd_workspace_bytes(tokens, heads) bytes."""
    n = h3attn_bwd_workspace_bytes(tokens, heads)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def h3attn_bwd(dout, q, k, v, lse, seg_ids, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None,
               dq=None, dk=None, dv=None, dwq=None, dwk=None, workspace_buf=None, stream=None):
    """Backward of the node: returns (dq, dk, dv, dwq, dwk) (dwq/dwk None without norm weights).
    lse is the forward's fp32 [T, H] log-sum-exp (h3attn_fwd(..., want_lse=True))."""
    return _bwd(dout, q, k, v, lse, seg_ids, None, wq, wk, eps, scale, dq, dk, dv, dwq, dwk, workspace_buf, stream)


def h3attn_bwd_pos(dout, q, k, v, lse, seg_ids, pos_ids, wq=None, wk=None, eps: float = 1e-6,
                   scale: float | None = None, dq=None, dk=None, dv=None, dwq=None, dwk=None, workspace_buf=None,
                   stream=None):
    """h3attn_bwd with every sum taken in the order of pos_ids (as for h3attn_fwd_pos)."""
    return _bwd(dout, q, k, v, lse, seg_ids, _int32(pos_ids, "pos_ids"), wq, wk, eps, scale, dq, dk, dv, dwq, dwk,
                workspace_buf, stream)


def h3attn_bwd_ex(dout, q, k, v, lse, seg_ids, pos_ids=None, o32=None, wq=None, wk=None, eps: float = 1e-6,
                  scale: float | None = None, dq=None, dk=None, dv=None, dwq=None, dwk=None, workspace_buf=None,
                  stream=None):
    """The backward with every option: position order when pos_ids is given; D = dO . O from the
    forward's o32 (h3attn_fwd_ex) when given, else recomputed.  Returns (dq, dk, dv, dwq, dwk)."""
    if o32 is not None and (o32.dtype != torch.float32 or not o32.is_contiguous()):
        raise TypeError("o32 must be a contiguous float32 tensor")
    return _bwd(dout, q, k, v, lse, seg_ids, None if pos_ids is None else _int32(pos_ids, "pos_ids"), wq, wk, eps,
                scale, dq, dk, dv, dwq, dwk, workspace_buf, stream, o32=o32, ex=True)


def _bwd(dout, q, k, v, lse, seg_ids, pos_ids, wq, wk, eps, scale, dq, dk, dv, dwq, dwk, workspace_buf, stream,
         o32=None, ex=False):
    for t, n in ((dout, "dout"), (q, "q"), (k, "k"), (v, "v"), (wq, "wq"), (wk, "wk")):
        _bf16(t, n)
    _int32(seg_ids, "seg_ids")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    T, H, D = _shape(q)
    scale = D ** -0.5 if scale is None else scale
    dq = torch.empty_like(q) if dq is None else _bf16(dq, "dq")
    dk = torch.empty_like(q) if dk is None else _bf16(dk, "dk")
    dv = torch.empty_like(q) if dv is None else _bf16(dv, "dv")
    if wq is not None:
        dwq = torch.empty(D, dtype=torch.float32, device=q.device) if dwq is None else dwq
        dwk = torch.empty(D, dtype=torch.float32, device=q.device) if dwk is None else dwk
    ws = bwd_workspace(T, H, q.device) if workspace_buf is None else workspace_buf
    st = _stream(stream, q.device)
    if ex:
        rc = load().h3attn_bwd_ex(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(o32), _ptr(seg_ids),
                                  _ptr(pos_ids), _ptr(wq), _ptr(wk), T, H, D, float(eps), float(scale), _ptr(dq),
                                  _ptr(dk), _ptr(dv), _ptr(dwq), _ptr(dwk), _ptr(ws), ws.numel(), st)
        _check(rc, "h3attn_bwd_ex")
    elif pos_ids is None:
        rc = load().h3attn_bwd(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(seg_ids), _ptr(wq), _ptr(wk),
                               T, H, D, float(eps), float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dwq), _ptr(dwk),
                               _ptr(ws), ws.numel(), st)
        _check(rc, "h3attn_bwd")
    else:
        rc = load().h3attn_bwd_pos(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(seg_ids), _ptr(pos_ids),
                                   _ptr(wq), _ptr(wk), T, H, D, float(eps), float(scale), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _ptr(dwq), _ptr(dwk), _ptr(ws), ws.numel(), st)
        _check(rc, "h3attn_bwd_pos")
    return dq, dk, dv, dwq, dwk
