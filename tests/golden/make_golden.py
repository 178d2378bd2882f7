"""Writes tiny_rows.json: fp64 oracle outputs for a few rows of the tiny
workload (B=1, H=2, T=128, lambda=0.5).  Calls only oracle/ and synth/.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

ROWS = [(0, 0, 0), (0, 1, 1), (0, 31, 0), (0, 32, 1), (0, 63, 0), (0, 64, 1), (0, 127, 0), (0, 127, 1)]


def main():
    wl = synth.WORKLOADS["tiny_b1_h2_t128"]
    x = synth.make_prefill_inputs(wl)
    o, y = oracle.prefill(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], x["gain"],
                          x["eps"], x["scale"], rows=ROWS)
    out = {
        "source": "fp64 oracle (oracle/diffattn_oracle.c) on synth workload tiny_b1_h2_t128",
        "workload": wl.name,
        "rows": [list(r) for r in ROWS],
        "o_pre": [[float(t) for t in r] for r in o],
        "y": [[float(t) for t in r] for r in y],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_rows.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()
