"""Writes the oracle regression fixtures in this folder.

Calls only ``oracle`` and the seeded ``workloads`` generators. The fixtures
freeze a few oracle outputs of the tiny workload (B=1, H=2, N=256, D=64,
scale 1/8) so that an accidental change to the oracle's arithmetic shows up
as a failing test; the oracle itself is pinned by tests/test_oracle_pins.py.

    python tests/golden/make_golden.py
"""
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    c = workloads.CONFIGS["tiny"]
    q, k, v = workloads.workload_qkv("tiny")
    scale = 1.0 / math.sqrt(c["D"])
    o, lse = oracle.attention(q, k, v, scale)
    rows = [0, 1, 63, 64, 128, 200, 255]
    fixture = {
        "what": "oracle O[0,h,row,:4] and LSE[0,h,row] for the tiny workload",
        "scale": scale,
        "rows": rows,
        "o_head0_first4": [[float(x) for x in o[0, 0, r, :4]] for r in rows],
        "o_head1_first4": [[float(x) for x in o[0, 1, r, :4]] for r in rows],
        "lse_head0": [float(lse[0, 0, r]) for r in rows],
        "lse_head1": [float(lse[0, 1, r]) for r in rows],
        "o_sum": float(np.sum(o)),
        "lse_sum": float(np.sum(lse)),
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(fixture, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
