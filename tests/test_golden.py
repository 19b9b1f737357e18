"""Oracle regression against the frozen fixtures in tests/golden/ (no GPU)."""
import json
import math
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_oracle_fixture_unchanged():
    with open(os.path.join(GOLDEN, "tiny_oracle.json")) as f:
        g = json.load(f)
    q, k, v = workloads.workload_qkv("tiny")
    o, lse = oracle.attention(q, k, v, 1.0 / math.sqrt(64))
    rows = g["rows"]
    np.testing.assert_allclose(o[0, 0, rows, :4], g["o_head0_first4"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(o[0, 1, rows, :4], g["o_head1_first4"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, rows], g["lse_head0"], rtol=1e-13)
    np.testing.assert_allclose(lse[0, 1, rows], g["lse_head1"], rtol=1e-13)
    assert abs(float(np.sum(lse)) - g["lse_sum"]) < 1e-9
