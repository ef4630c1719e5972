"""FP64 CPU oracle of the H3 attention node (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may import
this package.  The product path never does: it shares no code with the HIP library, and the HIP
library does not know it exists.

The arithmetic lives in ``h3_oracle.c`` (plain C, FP64, OpenMP over independent query rows); this
module only marshals numpy arrays.  bf16 tensors travel as their uint16 bit patterns.

Functions follow the RL-Kernel MiniMax-H3 pull-request pages:
  * ``qknorm`` / ``rmsnorm_f64``: the q_norm/k_norm node ("ws1_one_h3_block", Bindings table:
    RMSNorm over 128-wide heads, equal to nn.RMSNorm; Results: one 128-element weight for all heads).
  * ``fwd`` / ``fwd_rows``: attention(causal=False) over packed sequences (same page, Bindings and
    Summary), evaluated exactly in FP64 ("33B forward/backward", Scope: FP32 accumulation, one
    final rounding -- the oracle is the value such a kernel approximates).
  * ``bwd``: the gradients of that composite (norm, bf16 rounding taken as the identity, attention)
    with respect to q, k, v and both norm weights, in FP64 -- the node inside the training step's
    backward ("33B forward/backward" page).
  * ``rope_f64`` and the ``cos``/``sin`` arguments of ``fwd_ex`` / ``bwd``: the MM-RoPE node between
    the norm and the attention ("ws1_one_h3_block", Bindings: rope_q/rope_k; Tests: 96 of 128
    channels rotated), driven by per-token tables of the 48 pairs' cosines and sines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "h3_oracle.c")
_LIB_PATH = os.path.join(_DIR, "libh3oracle.so")

HEAD_DIM = 128
OK, ERR_ARGS, ERR_SEGMENTS, ERR_NOMEM = 0, 1, 2, 3


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (portable x86-64-v3, no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = D
    lib.oracle_f64_to_bf16.argtypes = [D]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_f64_to_bf16_array.argtypes = [P, P, I64]
    lib.oracle_segments.argtypes = [P, I64, P, P, P]
    lib.oracle_rmsnorm_f64.argtypes = [P, P, P, I64, I32, D]
    lib.oracle_qknorm.argtypes = [P, P, P, I64, I32, D]
    lib.oracle_fwd.argtypes = [P, P, P, P, P, P, I64, I32, D, D, P, P]
    lib.oracle_fwd_rows.argtypes = [P, P, P, P, P, P, I64, I32, D, D, P, I64, P, P]
    lib.oracle_bwd.argtypes = [P, P, P, P, P, P, P, I64, I32, D, D, ctypes.c_int, P, P, P, P, P]
    lib.oracle_fwd_opt.argtypes = [P, P, P, P, P, P, I64, I32, D, D, ctypes.c_int, P]
    lib.oracle_fwd_ex.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, I64, I32, D, D, P, I64, P, P]
    lib.oracle_bwd_ex.argtypes = [P, P, P, P, P, P, P, P, P, I64, I32, D, D, ctypes.c_int, P, P, P, P, P]
    lib.oracle_rope_f64.argtypes = [P, P, P, P, I64, I32]
    for f in (lib.oracle_segments, lib.oracle_rmsnorm_f64, lib.oracle_qknorm, lib.oracle_fwd, lib.oracle_fwd_rows,
              lib.oracle_bwd, lib.oracle_fwd_opt, lib.oracle_fwd_ex, lib.oracle_bwd_ex, lib.oracle_rope_f64):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _bits(a, shape=None):
    """Accept a uint16 bit-pattern array (or a torch bf16 tensor) and return contiguous uint16."""
    if a is None:
        return None
    if hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch
        a = a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    a = np.ascontiguousarray(a, dtype=np.uint16)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _check(rc):
    if rc != OK:
        raise OracleError({ERR_ARGS: "bad arguments", ERR_SEGMENTS: "segment ids decrease",
                           ERR_NOMEM: "out of memory"}.get(rc, f"status {rc}"))


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact FP64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """FP64 values -> bf16 bit patterns, one round-to-nearest-even step (the oracle's rounding)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_f64_to_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def segments(seg_ids):
    """(starts, lens) of the maximal runs of equal ids; raises if ids decrease."""
    s = np.ascontiguousarray(seg_ids, dtype=np.int32)
    T = s.shape[0]
    starts = np.zeros(max(T, 1), np.int64)
    lens = np.zeros(max(T, 1), np.int64)
    n = np.zeros(1, np.int64)
    _check(_load().oracle_segments(_ptr(s), T, _ptr(starts), _ptr(lens), _ptr(n)))
    return starts[: n[0]].copy(), lens[: n[0]].copy()


def rmsnorm_f64(x, w, eps: float) -> np.ndarray:
    """Unrounded FP64 RMSNorm of every 128-wide row of x [T, H, 128]."""
    x = _bits(x)
    T, H, D = x.shape
    assert D == HEAD_DIM
    w = _bits(w, (HEAD_DIM,))
    y = np.empty((T, H, D), np.float64)
    _check(_load().oracle_rmsnorm_f64(_ptr(x), _ptr(w), _ptr(y), T, H, float(eps)))
    return y


def qknorm(x, w, eps: float) -> np.ndarray:
    """The q_norm/k_norm node: FP64 RMSNorm rounded once to bf16 (uint16 bit patterns)."""
    x = _bits(x)
    T, H, D = x.shape
    assert D == HEAD_DIM
    w = _bits(w, (HEAD_DIM,))
    y = np.empty((T, H, D), np.uint16)
    _check(_load().oracle_qknorm(_ptr(x), _ptr(w), _ptr(y), T, H, float(eps)))
    return y


def fwd(q, k, v, seg_ids, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None):
    """Exact FP64 attention of the whole node.  Returns (out [T,H,128] FP64, lse [T,H] FP64)."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    T, H, D = q.shape
    assert D == HEAD_DIM and k.shape == q.shape and v.shape == q.shape
    wq, wk = _bits(wq, (HEAD_DIM,)), _bits(wk, (HEAD_DIM,))
    s = np.ascontiguousarray(seg_ids, dtype=np.int32)
    assert s.shape == (T,)
    scale = float(HEAD_DIM ** -0.5 if scale is None else scale)
    out = np.empty((T, H, D), np.float64)
    lse = np.empty((T, H), np.float64)
    _check(_load().oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(wq), _ptr(wk), T, H, float(eps), scale,
                              _ptr(out), _ptr(lse)))
    return out, lse


def fwd_rows(q, k, v, seg_ids, rows, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None):
    """Exact FP64 attention for the listed query tokens only: (out [n,H,128], lse [n,H])."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    T, H, D = q.shape
    assert D == HEAD_DIM and k.shape == q.shape and v.shape == q.shape
    wq, wk = _bits(wq, (HEAD_DIM,)), _bits(wk, (HEAD_DIM,))
    s = np.ascontiguousarray(seg_ids, dtype=np.int32)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    scale = float(HEAD_DIM ** -0.5 if scale is None else scale)
    out = np.empty((r.shape[0], H, D), np.float64)
    lse = np.empty((r.shape[0], H), np.float64)
    _check(_load().oracle_fwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(wq), _ptr(wk), T, H, float(eps), scale,
                                   _ptr(r), r.shape[0], _ptr(out), _ptr(lse)))
    return out, lse


ROPE_PAIRS = 48


def _table(t, T):
    """A rope table: float32 [T, 48] (the cosines or sines of every token's 48 rotated pairs)."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        t = t.detach().cpu().numpy()
    t = np.ascontiguousarray(t, dtype=np.float32)
    if t.shape != (T, ROPE_PAIRS):
        raise ValueError(f"rope table must be [{T}, {ROPE_PAIRS}], got {t.shape}")
    return t


def rope_f64(x, cos, sin) -> np.ndarray:
    """Unrounded FP64 rotation of every 128-wide row of x [T, H, 128] (bf16) by its token's table:
    pairs (2i, 2i+1), i < 48, rotated by (cos[t, i], sin[t, i]); channels 96..127 unchanged."""
    x = _bits(x)
    T, H, D = x.shape
    c, sn = _table(cos, T), _table(sin, T)
    y = np.empty((T, H, D), np.float64)
    _check(_load().oracle_rope_f64(_ptr(x), _ptr(c), _ptr(sn), _ptr(y), T, H))
    return y


def fwd_ex(q, k, v, seg_ids, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None, cos=None, sin=None,
           round_operands: bool = True, rows=None):
    """The forward with every option: rope tables (cos, sin float32 [T, 48], with weights only), the
    operands' bf16 roundings (round_operands=False: exact FP64 norm and rope outputs) and selected
    query rows.  Returns (out FP64, lse FP64) for every token or for the listed rows."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    T, H, D = q.shape
    assert D == HEAD_DIM and k.shape == q.shape and v.shape == q.shape
    wq, wk = _bits(wq, (HEAD_DIM,)), _bits(wk, (HEAD_DIM,))
    c, sn = _table(cos, T), _table(sin, T)
    s = np.ascontiguousarray(seg_ids, dtype=np.int32)
    assert s.shape == (T,)
    scale = float(HEAD_DIM ** -0.5 if scale is None else scale)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = T if r is None else r.shape[0]
    out = np.empty((n, H, D), np.float64)
    lse = np.empty((n, H), np.float64)
    _check(_load().oracle_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(wq), _ptr(wk), _ptr(c), _ptr(sn),
                                 int(bool(round_operands)), T, H, float(eps), scale, _ptr(r), 0 if r is None else n,
                                 _ptr(out), _ptr(lse)))
    return out, lse


def bwd(q, k, v, seg_ids, dout, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None,
        round_operands: bool = True, cos=None, sin=None):
    """FP64 gradients of the node for upstream gradient dout [T,H,128] (bf16 bits).

    Returns (dq, dk, dv) FP64 [T,H,128] and (dwq, dwk) FP64 [128] (None without weights).  With
    round_operands=False the normed operands are not rounded to bf16 (exact gradient of a smooth
    function, for finite-difference checks).  cos, sin: rope tables as for fwd_ex."""
    q, k, v, dout = _bits(q), _bits(k), _bits(v), _bits(dout)
    T, H, D = q.shape
    assert D == HEAD_DIM and k.shape == q.shape and v.shape == q.shape and dout.shape == q.shape
    wq, wk = _bits(wq, (HEAD_DIM,)), _bits(wk, (HEAD_DIM,))
    s = np.ascontiguousarray(seg_ids, dtype=np.int32)
    assert s.shape == (T,)
    scale = float(HEAD_DIM ** -0.5 if scale is None else scale)
    dq = np.empty((T, H, D), np.float64)
    dk = np.empty((T, H, D), np.float64)
    dv = np.empty((T, H, D), np.float64)
    dwq = np.zeros(HEAD_DIM, np.float64) if wq is not None else None
    dwk = np.zeros(HEAD_DIM, np.float64) if wq is not None else None
    c, sn = _table(cos, T), _table(sin, T)
    _check(_load().oracle_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(wq), _ptr(wk), _ptr(c), _ptr(sn), _ptr(dout),
                                 T, H, float(eps), scale, int(bool(round_operands)), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(dwq), _ptr(dwk)))
    return dq, dk, dv, dwq, dwk


def fwd_opt(q, k, v, seg_ids, wq=None, wk=None, eps: float = 1e-6, scale: float | None = None,
            round_operands: bool = True) -> np.ndarray:
    """FP64 forward output with the operand rounding optional (see ``bwd``)."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    T, H, D = q.shape
    wq, wk = _bits(wq, (HEAD_DIM,)), _bits(wk, (HEAD_DIM,))
    s = np.ascontiguousarray(seg_ids, dtype=np.int32)
    scale = float(HEAD_DIM ** -0.5 if scale is None else scale)
    out = np.empty((T, H, D), np.float64)
    _check(_load().oracle_fwd_opt(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(wq), _ptr(wk), T, H, float(eps), scale,
                                  int(bool(round_operands)), _ptr(out)))
    return out
