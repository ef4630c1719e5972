"""Writes tests/golden/tiny_oracle.json from the FP64 oracle alone (no HIP code is involved).

The pages print no attention values for any input, so this fixture is a regression guard on the
oracle itself: the 12-token, two-segment (5 + 7), 4-head workload with seed 0, its input digests,
every LSE and the first 8 channels of every output row.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    wl = workloads.WORKLOADS["tiny"]
    x = workloads.make_inputs(wl)
    out, lse = oracle.fwd(x["q"], x["k"], x["v"], x["seg"].numpy(), x["wq"], x["wk"], wl.eps, wl.scale)
    doc = {
        "about": "FP64 oracle outputs for the tiny workload (12 tokens, segments 5+7, 4 heads, seed 0); "
                 "written by tests/golden/make_golden.py, which calls only oracle/ and workloads/",
        "workload": wl.name,
        "sha256": {n: workloads.sha256(x[n]) for n in ("q", "k", "v", "seg", "wq", "wk")},
        "lse": [[float(v) for v in row] for row in lse],
        "out_first8": [[[float(v) for v in out[t, h, :8]] for h in range(wl.heads)] for t in range(wl.tokens)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
