"""Write tests/golden/oracle_small.json from the fp64 oracle only.

The fixture stores seeded inputs and the oracle's outputs for a small case
(B=1, H=2, T=20, dk=dv=8, fp32 inputs, nonzero start state) so that later runs
can detect any change in the oracle's arithmetic.  Run from the repo root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import kda_inputs as ki  # noqa: E402
import oracle  # noqa: E402


def main():
    d = ki.gen_prefill(1, 2, 20, 8, 8, "f32", seed=7, s0_std=0.1)
    o, ST = oracle.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], nthreads=1)
    out = {
        "what": "fp64 oracle outputs for seeded fp32 inputs; written by make_golden.py",
        "shape": {"B": 1, "H": 2, "T": 20, "dk": 8, "dv": 8},
        "inputs": {k: d[k].double().numpy().tolist() for k in ("q", "k", "v", "log_alpha", "beta", "S0")},
        "o": o.tolist(),
        "S_T": ST.tolist(),
    }
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(out, f, separators=(",", ":"))


if __name__ == "__main__":
    main()
