"""Write the oracle regression fixture for the tiny fp32 workload.

Run from the repository root:  python tests/golden/make_golden.py
Calls only the fp64 oracle (oracle/) on inputs from the seeded generator; the
HIP library is not involved.  The fixture freezes the oracle's results so that
a later change to its arithmetic shows up as a test failure.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from gated_deltanet_linear_rule_amd.inputs import make_inputs  # noqa: E402
from oracle import c_oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle.json")
SAMPLES = [(0, 0, 0), (1, 1, 5), (63, 0, 63), (64, 1, 0), (200, 0, 17), (255, 1, 63)]


def summarize():
    inp = make_inputs("tiny_f32", seed=0)
    out, fin = c_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, None, None)
    return {
        "workload": "tiny_f32: T=256, H=2, d_k=d_v=64, fp32, zero initial state, seed 0",
        "source": "oracle/gdn_oracle.c via tests/golden/make_golden.py",
        "out_sum": float(out.sum()),
        "out_abs_sum": float(np.abs(out).sum()),
        "out_max_abs": float(np.abs(out).max()),
        "final_sum": float(fin.sum()),
        "final_abs_sum": float(np.abs(fin).sum()),
        "out_samples": [[t, h, i, float(out[t, h, i])] for t, h, i in SAMPLES],
        "final_samples": [[h, i, j, float(fin[0, h, i, j])] for h, i, j in
                          [(0, 0, 0), (1, 10, 20), (0, 63, 63)]],
    }


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(summarize(), f, indent=1)
    print("wrote", OUT)
