"""Writes tests/golden/tiny_oracle_summary.json from the float64 oracle only.

The fixture records a few figures of the C oracle's output on the tiny workload
(B=1, H=2, T=256, d=64, fp32 inputs, zero initial state, seed 0) so that any
later change to the oracle's arithmetic shows up as a test failure.  Run from
the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

x = workloads.make_inputs(workloads.WORKLOADS["tiny"])
o, sT = oracle.run_c(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
out = {
    "workload": "tiny (B=1, H=2, T=256, d=64, fp32, zero state, seed 0)",
    "source": "oracle.run_c (float64 token recurrence)",
    "o_norm": float(np.linalg.norm(o)),
    "state_norm": float(np.linalg.norm(sT)),
    "o_samples": [float(a) for a in o[::37, :, ::13].ravel()],
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_summary.json"), "w") as f:
    json.dump(out, f, indent=1)
print("wrote", len(out["o_samples"]), "samples")
