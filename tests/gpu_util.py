"""Helpers of the GPU tests: move seeded inputs to the device, run the C ABI, compare with the oracle."""
import hashlib
import sys

import numpy as np
import torch

import deterministic_invariant_attention_amd as h3

REL_L2_BOUND = 2e-3   # relative L2 of the bf16 output against the FP64 oracle, whole tensor
MAX_ABS_BOUND = 2e-2  # largest absolute difference
LSE_REL_BOUND = 1e-5  # LSE from FP32 logits: |error| <= 1e-5 * max(1, |LSE|)
EPS = 9.999999974752427e-07   # 1e-6 as the float32 value the C ABI receives


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(x):
    return {n: (t.to(dev()) if isinstance(t, torch.Tensor) else t) for n, t in x.items()}


def run_fwd(g, eps=EPS, scale=128 ** -0.5, want_lse=False, weights=True, ws=None):
    wq, wk = (g.get("wq"), g.get("wk")) if weights else (None, None)
    out, lse = h3.h3attn_fwd(g["q"], g["k"], g["v"], g["seg"], wq, wk, eps=eps, scale=scale, want_lse=want_lse,
                             workspace_buf=ws)
    torch.cuda.synchronize()
    return out, lse


def f64(t):
    return t.detach().float().cpu().double().numpy()


def metrics(gpu_out, ref):
    o = f64(gpu_out) if isinstance(gpu_out, torch.Tensor) else gpu_out
    diff = o - ref
    rel = float(np.linalg.norm(diff) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    return rel, mx


def bits(t):
    """The tensor's bit patterns (so that NaN == NaN and -0 != +0 in a bitwise comparison)."""
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.detach().contiguous().view(torch.int16)
    if t.dtype == torch.float32:
        return t.detach().contiguous().view(torch.int32)
    return t


def digest(t):
    return hashlib.sha256(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


def bitwise_equal(a, b):
    return torch.equal(bits(a), bits(b))


def lse_error(gpu_lse, ref_lse):
    """Largest LSE error relative to max(1, |LSE|)."""
    g = f64(gpu_lse) if isinstance(gpu_lse, torch.Tensor) else gpu_lse
    return float(np.max(np.abs(g - ref_lse) / np.maximum(1.0, np.abs(ref_lse)))) if g.size else 0.0
