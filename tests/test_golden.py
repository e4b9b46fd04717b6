"""Hand-derived closed-form fixtures against the CPU oracle (exact)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")


def golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def expand(case):
    """Return (q, k, v, n, expected_o) as float64 [L, d] arrays."""
    if "q" in case:
        q, k, v = (np.array(case[t], dtype=np.float64) for t in ("q", "k", "v"))
        return q, k, v, case["n"], np.array(case["o"], dtype=np.float64)
    L, d, n = case["lmax"], case["d"], case["n"]
    q = np.full((L, d), float(case["q_fill"]))
    k = np.tile(np.array(case["k_seed_values"], dtype=np.float64), (L, 1)) * (1 + np.arange(L))[:, None]
    v = np.full((L, d), float(case["v_fill"]))
    v[n:] = -3.0  # padded garbage
    o = np.zeros((L, d))
    o[:n] = case["o_valid"]
    return q, k, v, n, o


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_golden_oracle(case):
    q, k, v, n, want = expand(case)
    got = oracle.attention(q[None, None], k[None, None], v[None, None], [n])["o"][0, 0]
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=1e-15)
