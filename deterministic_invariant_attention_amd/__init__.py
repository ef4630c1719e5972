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
ROPE_PAIRS = 48  # MM-RoPE: the rotated pairs of channels (96 of 128)

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
H3ATTN_ERR_SCRATCH = 11

# every symbol the header declares
EXPORTS = ("h3attn_version", "h3attn_strerror", "h3attn_workspace_bytes", "h3attn_qknorm", "h3attn_fwd",
           "h3attn_fwd_pos", "h3attn_fwd_ex", "h3attn_plan", "h3attn_prep_qkv", "h3attn_attend", "h3attn_status_read",
           "h3attn_bwd_workspace_bytes", "h3attn_bwd", "h3attn_bwd_pos", "h3attn_bwd_ex", "h3attn_fwd_noalloc")


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
    lib.h3attn_fwd_ex.argtypes = [P, P, P, P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, P, SZ, P]
    lib.h3attn_fwd_noalloc.argtypes = [P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, P]
    lib.h3attn_plan.argtypes = [P, I64, I32, P, SZ, P]
    lib.h3attn_prep_qkv.argtypes = [P, P, P, P, P, I64, I32, I32, F, P, SZ, P]
    lib.h3attn_attend.argtypes = [P, P, I64, I32, I32, F, F, P, P, P, SZ, P]
    lib.h3attn_status_read.argtypes = [P, ctypes.POINTER(ctypes.c_int32), P]
    lib.h3attn_bwd_workspace_bytes.argtypes = [I64, I32]
    lib.h3attn_bwd_workspace_bytes.restype = SZ
    lib.h3attn_bwd.argtypes = [P, P, P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, P, P, P, SZ, P]
    lib.h3attn_bwd_pos.argtypes = [P, P, P, P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, P, P, P, SZ, P]
    lib.h3attn_bwd_ex.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I64, I32, I32, F, F, P, P, P, P, P, P, SZ, P]
    for name in ("h3attn_qknorm", "h3attn_fwd", "h3attn_fwd_pos", "h3attn_fwd_ex", "h3attn_plan", "h3attn_prep_qkv",
                 "h3attn_attend", "h3attn_status_read", "h3attn_bwd", "h3attn_bwd_pos", "h3attn_bwd_ex",
                 "h3attn_fwd_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _as_stream(stream, device):
    """The torch stream object for a stream argument: None = torch's current stream on the device; a
    torch.cuda.Stream as given; a raw hipStream_t handle (int) wrapped as an external stream."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _stream(stream, device):
    """The hipStream_t handle for a stream argument (see _as_stream)."""
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int, where: str):
    if rc != H3ATTN_OK:
        raise H3AttnError(rc, where)


def _shape(q):
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise H3AttnError(H3ATTN_ERR_SHAPE, "expected [tokens, heads, head_dim]")
    return q.shape[0], q.shape[1], q.shape[2]


def _bf16(t, name):
    if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous bfloat16 tensor")
    return t


class _Args:
    """Checks every tensor argument of one call against the shapes the C ABI assumes, before the
    library sees a pointer: a tensor of the wrong shape or on another device would hand the kernels
    an undersized buffer or a host address.  Strict mode ("33B forward/backward" page, Scope):
    wrong shapes, dtypes and devices raise; nothing falls back."""

    def __init__(self, where, q):
        self.where = where
        T, H, D = _shape(q)
        self.T, self.H, self.D = T, H, D
        self.tensors = []
        self.want(q, "q", torch.bfloat16, (T, H, D))

    def want(self, t, name, dtype, shape):
        if t is None:
            return None
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.where}: {name} must be a torch tensor")
        if t.dtype != dtype or not t.is_contiguous():
            raise TypeError(f"{self.where}: {name} must be a contiguous {dtype} tensor")
        if tuple(t.shape) != tuple(shape):
            raise H3AttnError(H3ATTN_ERR_SHAPE, f"{self.where}: {name} has shape {tuple(t.shape)}, expected "
                                                f"{tuple(shape)}")
        self.tensors.append((name, t))
        return t

    def device(self):
        """Every tensor on q's device, and that device a GPU (else ERR_DEVICE); returns it."""
        dev = self.tensors[0][1].device
        if dev.type != "cuda":
            raise H3AttnError(H3ATTN_ERR_DEVICE, f"{self.where}: q is on {dev}, not a GPU")
        for name, t in self.tensors:
            if t.device != dev:
                raise H3AttnError(H3ATTN_ERR_DEVICE, f"{self.where}: {name} is on {t.device}, q on {dev}")
        return dev


def _tok(a, t, name):
    """An int32 [T] per-token tensor (segment or position ids)."""
    return a.want(t, name, torch.int32, (a.T,))


def _ws(a, t, need, name="workspace_buf"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.dim() != 1 or not t.is_contiguous() or t.element_size() != 1:
        raise TypeError(f"{a.where}: {name} must be a contiguous 1-D byte tensor")
    if t.numel() < need:
        raise H3AttnError(H3ATTN_ERR_WORKSPACE, f"{a.where}: {name} holds {t.numel()} bytes, needs {need}")
    a.tensors.append((name, t))
    return t


def _status_or_raise(ws, stream, where):
    """Read the device status word (synchronises the stream) and raise on a recorded data error."""
    st = h3attn_status_read(ws, stream)
    if st != H3ATTN_OK:
        raise H3AttnError(st, where + " (device status)")


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
    a = _Args("h3attn_qknorm", x)
    a.want(w, "w", torch.bfloat16, (a.D,))
    a.want(out, "out", torch.bfloat16, (a.T, a.H, a.D))
    dev = a.device()
    st = _as_stream(stream, dev)
    with torch.cuda.device(dev), torch.cuda.stream(st):
        y = torch.empty_like(x) if out is None else out
        rc = load().h3attn_qknorm(_ptr(x), _ptr(w), _ptr(y), a.T, a.H, a.D, float(eps), st.cuda_stream)
    _check(rc, "h3attn_qknorm")
    return y


def _int32(t, name):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    return t


def h3attn_fwd(q, k, v, seg_ids, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None, out=None,
               lse=None, workspace_buf=None, stream=None, want_lse: bool = False, check_status: bool = False):
    """Forward of the attention node with its fused q/k norm.  Returns (out, lse) (lse None unless asked).
    check_status: read the device status word after the call (synchronises the stream) and raise on
    a recorded data error (decreasing segment ids, a value beyond the fp16 range)."""
    return _fwd(q, k, v, seg_ids, None, wq, wk, eps, scale, out, lse, workspace_buf, stream, want_lse,
                check_status=check_status)


def h3attn_fwd_pos(q, k, v, seg_ids, pos_ids, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None,
                   out=None, lse=None, workspace_buf=None, stream=None, want_lse: bool = False,
                   check_status: bool = False):
    """h3attn_fwd with each segment's keys walked in the order of pos_ids (int32 [T], a permutation of
    0..L-1 within each segment).  Returns (out, lse)."""
    return _fwd(q, k, v, seg_ids, _int32(pos_ids, "pos_ids"), wq, wk, eps, scale, out, lse, workspace_buf, stream,
                want_lse, check_status=check_status)


def h3attn_fwd_ex(q, k, v, seg_ids, pos_ids=None, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None,
                  out=None, lse=None, o32=None, workspace_buf=None, stream=None, want_lse: bool = False,
                  want_o32: bool = False, check_status: bool = False, rope_cos=None, rope_sin=None):
    """The forward with every option: position order when pos_ids is given, the fp32 output before
    its bf16 rounding (o32, for h3attn_bwd_ex) when asked, and the MM-RoPE node on the normed q and k
    when rope tables are given (rope_cos, rope_sin: float32 [T, 48]; with wq/wk only).
    Returns (out, lse, o32)."""
    return _fwd(q, k, v, seg_ids, None if pos_ids is None else _int32(pos_ids, "pos_ids"), wq, wk, eps, scale,
                out, lse, workspace_buf, stream, want_lse, o32=o32, want_o32=want_o32, ex=True,
                check_status=check_status, rope=(rope_cos, rope_sin))


def _rope(a, rope):
    """The two rope tables (both or neither), float32 [T, 48]."""
    rc, rs = rope
    if (rc is None) != (rs is None):
        raise H3AttnError(H3ATTN_ERR_NULL, f"{a.where}: give both rope tables or neither")
    a.want(rc, "rope_cos", torch.float32, (a.T, ROPE_PAIRS))
    a.want(rs, "rope_sin", torch.float32, (a.T, ROPE_PAIRS))
    return rc, rs


def _fwd(q, k, v, seg_ids, pos_ids, wq, wk, eps, scale, out, lse, workspace_buf, stream, want_lse, o32=None,
         want_o32=False, ex=False, check_status=False, rope=(None, None)):
    a = _Args("h3attn_fwd", q)
    T, H, D = a.T, a.H, a.D
    for t, n in ((k, "k"), (v, "v")):
        if t is None:
            raise H3AttnError(H3ATTN_ERR_NULL, f"h3attn_fwd: {n} is required")
        a.want(t, n, torch.bfloat16, (T, H, D))
    _tok(a, _int32(seg_ids, "seg_ids"), "seg_ids")
    _tok(a, pos_ids, "pos_ids")
    a.want(wq, "wq", torch.bfloat16, (D,))
    a.want(wk, "wk", torch.bfloat16, (D,))
    a.want(out, "out", torch.bfloat16, (T, H, D))
    a.want(lse, "lse", torch.float32, (T, H))
    a.want(o32, "o32", torch.float32, (T, H, D))
    rc_, rs_ = _rope(a, rope)
    _ws(a, workspace_buf, h3attn_workspace_bytes(T, H))
    dev = a.device()
    scale = D ** -0.5 if scale is None else scale
    st = _as_stream(stream, dev)
    # outputs and the workspace are allocated on the launch stream, so the caching allocator never
    # hands their memory to other work while the kernels still use it
    with torch.cuda.device(dev), torch.cuda.stream(st):
        out = torch.empty_like(q) if out is None else out
        if lse is None and want_lse:
            lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        if o32 is None and want_o32:
            o32 = torch.empty((T, H, D), dtype=torch.float32, device=dev)
        ws = workspace(T, H, dev) if workspace_buf is None else workspace_buf
        h = st.cuda_stream
        if ex:
            rc = load().h3attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(seg_ids), _ptr(pos_ids), _ptr(wq), _ptr(wk),
                                      _ptr(rc_), _ptr(rs_), T, H, D, float(eps), float(scale), _ptr(out), _ptr(lse),
                                      _ptr(o32), _ptr(ws), ws.numel(), h)
            _check(rc, "h3attn_fwd_ex")
        elif pos_ids is None:
            rc = load().h3attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(seg_ids), _ptr(wq), _ptr(wk), T, H, D, float(eps),
                                   float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), h)
            _check(rc, "h3attn_fwd")
        else:
            rc = load().h3attn_fwd_pos(_ptr(q), _ptr(k), _ptr(v), _ptr(seg_ids), _ptr(pos_ids), _ptr(wq), _ptr(wk),
                                       T, H, D, float(eps), float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                       h)
            _check(rc, "h3attn_fwd_pos")
        if check_status and T > 0:
            _status_or_raise(ws, st, "h3attn_fwd")
    return (out, lse, o32) if ex else (out, lse)


def h3attn_fwd_noalloc(q, k, v, seg_ids, wq, wk, out, lse=None, status=None, eps: float = 1e-6,
                       scale: float | None = None, stream=None):
    """h3attn_fwd on the library's static scratch: allocates nothing (out, and lse / status when
    wanted, are the caller's).  status: optional int32 [1] device tensor receiving the call's
    data-error code.  Sizes whose workspace would exceed 256 MiB raise H3ATTN_ERR_SCRATCH."""
    a = _Args("h3attn_fwd_noalloc", q)
    T, H, D = a.T, a.H, a.D
    for t, n in ((k, "k"), (v, "v"), (out, "out")):
        if t is None:
            raise H3AttnError(H3ATTN_ERR_NULL, f"h3attn_fwd_noalloc: {n} is required")
        a.want(t, n, torch.bfloat16, (T, H, D))
    _tok(a, _int32(seg_ids, "seg_ids"), "seg_ids")
    a.want(wq, "wq", torch.bfloat16, (D,))
    a.want(wk, "wk", torch.bfloat16, (D,))
    a.want(lse, "lse", torch.float32, (T, H))
    a.want(status, "status", torch.int32, (1,))
    dev = a.device()
    scale = D ** -0.5 if scale is None else scale
    with torch.cuda.device(dev):
        rc = load().h3attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(seg_ids), _ptr(wq), _ptr(wk), T, H, D,
                                       float(eps), float(scale), _ptr(out), _ptr(lse), _ptr(status),
                                       _stream(stream, dev))
    _check(rc, "h3attn_fwd_noalloc")
    return out


def h3attn_plan(seg_ids, heads: int, workspace_buf, stream=None):
    _int32(seg_ids, "seg_ids")
    if seg_ids.dim() != 1:
        raise H3AttnError(H3ATTN_ERR_SHAPE, "h3attn_plan: seg_ids must be int32 [T]")
    T, H = seg_ids.shape[0], int(heads)
    if not isinstance(workspace_buf, torch.Tensor) or workspace_buf.numel() < h3attn_workspace_bytes(T, H):
        raise H3AttnError(H3ATTN_ERR_WORKSPACE, "h3attn_plan: workspace_buf is too small")
    dev = seg_ids.device
    if dev.type != "cuda" or workspace_buf.device != dev:
        raise H3AttnError(H3ATTN_ERR_DEVICE, "h3attn_plan: seg_ids and the workspace must be on one GPU")
    with torch.cuda.device(dev):
        rc = load().h3attn_plan(_ptr(seg_ids), T, H, _ptr(workspace_buf), workspace_buf.numel(), _stream(stream, dev))
    _check(rc, "h3attn_plan")


def h3attn_prep_qkv(q, k, v, wq, wk, workspace_buf, eps: float = 1e-6, stream=None):
    a = _Args("h3attn_prep_qkv", q)
    a.want(k, "k", torch.bfloat16, (a.T, a.H, a.D))
    a.want(v, "v", torch.bfloat16, (a.T, a.H, a.D))
    a.want(wq, "wq", torch.bfloat16, (a.D,))
    a.want(wk, "wk", torch.bfloat16, (a.D,))
    _ws(a, workspace_buf, h3attn_workspace_bytes(a.T, a.H))
    dev = a.device()
    with torch.cuda.device(dev):
        rc = load().h3attn_prep_qkv(_ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), a.T, a.H, a.D, float(eps),
                                    _ptr(workspace_buf), workspace_buf.numel(), _stream(stream, dev))
    _check(rc, "h3attn_prep_qkv")


def h3attn_attend(q, wq, workspace_buf, out, lse=None, eps: float = 1e-6, scale: float | None = None, stream=None):
    a = _Args("h3attn_attend", q)
    a.want(wq, "wq", torch.bfloat16, (a.D,))
    a.want(out, "out", torch.bfloat16, (a.T, a.H, a.D))
    a.want(lse, "lse", torch.float32, (a.T, a.H))
    _ws(a, workspace_buf, h3attn_workspace_bytes(a.T, a.H))
    dev = a.device()
    scale = a.D ** -0.5 if scale is None else scale
    with torch.cuda.device(dev):
        rc = load().h3attn_attend(_ptr(q), _ptr(wq), a.T, a.H, a.D, float(eps), float(scale), _ptr(out), _ptr(lse),
                                  _ptr(workspace_buf), workspace_buf.numel(), _stream(stream, dev))
    _check(rc, "h3attn_attend")
    return out


def h3attn_status_read(workspace_buf, stream=None) -> int:
    if not isinstance(workspace_buf, torch.Tensor) or workspace_buf.device.type != "cuda":
        raise H3AttnError(H3ATTN_ERR_DEVICE, "h3attn_status_read: the workspace is not on a GPU")
    st = ctypes.c_int32(-1)
    with torch.cuda.device(workspace_buf.device):
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
               dq=None, dk=None, dv=None, dwq=None, dwk=None, workspace_buf=None, stream=None,
               check_status: bool = False):
    """Backward of the node: returns (dq, dk, dv, dwq, dwk) (dwq/dwk None without norm weights).
    lse is the forward's fp32 [T, H] log-sum-exp (h3attn_fwd(..., want_lse=True))."""
    return _bwd(dout, q, k, v, lse, seg_ids, None, wq, wk, eps, scale, dq, dk, dv, dwq, dwk, workspace_buf, stream,
                check_status=check_status)


def h3attn_bwd_pos(dout, q, k, v, lse, seg_ids, pos_ids, wq=None, wk=None, eps: float = 1e-6,
                   scale: float | None = None, dq=None, dk=None, dv=None, dwq=None, dwk=None, workspace_buf=None,
                   stream=None, check_status: bool = False):
    """h3attn_bwd with every sum taken in the order of pos_ids (as for h3attn_fwd_pos)."""
    return _bwd(dout, q, k, v, lse, seg_ids, _int32(pos_ids, "pos_ids"), wq, wk, eps, scale, dq, dk, dv, dwq, dwk,
                workspace_buf, stream, check_status=check_status)


def h3attn_bwd_ex(dout, q, k, v, lse, seg_ids, pos_ids=None, o32=None, wq=None, wk=None, eps: float = 1e-6,
                  scale: float | None = None, dq=None, dk=None, dv=None, dwq=None, dwk=None, workspace_buf=None,
                  stream=None, check_status: bool = False, rope_cos=None, rope_sin=None):
    """The backward with every option: position order when pos_ids is given; D = dO . O from the
    forward's o32 (h3attn_fwd_ex) when given, else recomputed; the rope tables given to the forward.
    Returns (dq, dk, dv, dwq, dwk)."""
    return _bwd(dout, q, k, v, lse, seg_ids, None if pos_ids is None else _int32(pos_ids, "pos_ids"), wq, wk, eps,
                scale, dq, dk, dv, dwq, dwk, workspace_buf, stream, o32=o32, ex=True, check_status=check_status,
                rope=(rope_cos, rope_sin))


def _bwd(dout, q, k, v, lse, seg_ids, pos_ids, wq, wk, eps, scale, dq, dk, dv, dwq, dwk, workspace_buf, stream,
         o32=None, ex=False, check_status=False, rope=(None, None)):
    a = _Args("h3attn_bwd", q)
    T, H, D = a.T, a.H, a.D
    for t, n in ((dout, "dout"), (k, "k"), (v, "v")):
        if t is None:
            raise H3AttnError(H3ATTN_ERR_NULL, f"h3attn_bwd: {n} is required")
        a.want(t, n, torch.bfloat16, (T, H, D))
    if lse is None:
        raise H3AttnError(H3ATTN_ERR_NULL, "h3attn_bwd: lse is required")
    a.want(lse, "lse", torch.float32, (T, H))
    _tok(a, _int32(seg_ids, "seg_ids"), "seg_ids")
    _tok(a, pos_ids, "pos_ids")
    a.want(o32, "o32", torch.float32, (T, H, D))
    a.want(wq, "wq", torch.bfloat16, (D,))
    a.want(wk, "wk", torch.bfloat16, (D,))
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        a.want(t, n, torch.bfloat16, (T, H, D))
    a.want(dwq, "dwq", torch.float32, (D,))
    a.want(dwk, "dwk", torch.float32, (D,))
    rc_, rs_ = _rope(a, rope)
    _ws(a, workspace_buf, h3attn_bwd_workspace_bytes(T, H))
    dev = a.device()
    scale = D ** -0.5 if scale is None else scale
    st = _as_stream(stream, dev)
    with torch.cuda.device(dev), torch.cuda.stream(st):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
        if wq is not None:
            dwq = torch.empty(D, dtype=torch.float32, device=dev) if dwq is None else dwq
            dwk = torch.empty(D, dtype=torch.float32, device=dev) if dwk is None else dwk
        ws = bwd_workspace(T, H, dev) if workspace_buf is None else workspace_buf
        h = st.cuda_stream
        if ex:
            rc = load().h3attn_bwd_ex(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(o32), _ptr(seg_ids),
                                      _ptr(pos_ids), _ptr(wq), _ptr(wk), _ptr(rc_), _ptr(rs_), T, H, D, float(eps),
                                      float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dwq), _ptr(dwk), _ptr(ws),
                                      ws.numel(), h)
            _check(rc, "h3attn_bwd_ex")
        elif pos_ids is None:
            rc = load().h3attn_bwd(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(seg_ids), _ptr(wq),
                                   _ptr(wk), T, H, D, float(eps), float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _ptr(dwq), _ptr(dwk), _ptr(ws), ws.numel(), h)
            _check(rc, "h3attn_bwd")
        else:
            rc = load().h3attn_bwd_pos(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(seg_ids),
                                       _ptr(pos_ids), _ptr(wq), _ptr(wk), T, H, D, float(eps), float(scale),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dwq), _ptr(dwk), _ptr(ws), ws.numel(), h)
            _check(rc, "h3attn_bwd_pos")
        if check_status and T > 0:
            _status_or_raise(ws, st, "h3attn_bwd")
    return dq, dk, dv, dwq, dwk
