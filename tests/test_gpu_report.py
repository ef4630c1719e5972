"""Ungated parity report: the GPU output against three references, with the worst (segment, head).

  exact     the FP64 oracle of the node (the gate of the parity tests, reported again here);
  rounded   that output rounded once to bf16 (RNE): how many elements differ from it, and the
            error in bf16 spacings at the exact value;
  pure      an FP64 oracle whose normed q and k are not rounded to bf16 (the node without its
            q_norm/k_norm output rounding): the error the operand rounding itself contributes.
The numbers are printed (run with -s) and only required to be finite: the gate is elsewhere.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import EPS, f64, metrics, run_fwd, say, to_dev

pytestmark = pytest.mark.gpu


def _bf16_rne(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def _err_in_ulps(got, ref, floor=1e-3):
    """|got - ref| in units of the bf16 spacing at |ref| (2^(floor(log2|ref|) - 7)), where |ref| >= floor."""
    g, r = f64(got), np.asarray(ref)
    m = np.abs(r) >= floor
    spacing = np.exp2(np.floor(np.log2(np.abs(r[m]))) - 7)
    return np.abs(g[m] - r[m]) / spacing


@pytest.mark.parametrize("name", ["tiny", "short3", "batch2"])
def test_report_against_rounded_and_pure_oracles(name):
    wl = workloads.WORKLOADS[name]
    x = workloads.make_inputs(wl)
    out, _ = run_fwd(to_dev(x), eps=wl.eps, scale=wl.scale)
    got = out.cpu()
    ref, _ = oracle.fwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], wl.eps, wl.scale)
    pure = oracle.fwd_opt(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], wl.eps, wl.scale,
                          round_operands=False)
    rel, mx = metrics(got, ref)
    rel_p, mx_p = metrics(got, pure)
    rel_rp, _ = metrics(ref, pure)  # the operand rounding's own share
    frac = float((got.view(torch.int16) != _bf16_rne(ref).view(torch.int16)).double().mean())
    ulps = _err_in_ulps(got, ref)
    # worst (segment, head) by relative L2 against the exact oracle
    starts, lens = oracle.segments(x["seg"].numpy())
    worst = (0.0, None, None)
    g64 = f64(got)
    for s0, L in zip(starts, lens):
        for h in range(wl.heads):
            d = g64[s0:s0 + L, h] - ref[s0:s0 + L, h]
            r = float(np.linalg.norm(d) / max(np.linalg.norm(ref[s0:s0 + L, h]), 1e-300))
            if r > worst[0]:
                worst = (r, int(s0), h)
    say(f"[report] {name}: exact rel_l2={rel:.3e} max_abs={mx:.3e} | rounded: {100 * frac:.2f}% of elements differ; "
        f"error in bf16 spacings at the exact value (|ref| >= 1e-3): p99.9 {np.percentile(ulps, 99.9):.2f}, "
        f"max {ulps.max():.2f} | pure: rel_l2={rel_p:.3e} max_abs={mx_p:.3e} (exact vs pure {rel_rp:.3e}) | "
        f"worst segment start {worst[1]} head {worst[2]}: rel_l2={worst[0]:.3e}")
    assert np.isfinite([rel, mx, rel_p, mx_p, frac]).all()
