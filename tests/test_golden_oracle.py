"""The oracle reproduces the exact examples in tests/golden (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "page_examples.json")
CASES = json.load(open(GOLDEN))["cases"]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
def test_oracle_reproduces_page_example(case):
    q = np.array(case["q"], np.float64)[None, None]
    k = np.array(case["k"], np.float64)[None, None]
    v = np.array(case["v"], np.float64)[None, None]
    if case["kind"] == "delta":
        beta = np.array(case["beta"], np.float64)[None, None]
        o, S = oracle.delta_recurrent(q, k, v, beta)
        np.testing.assert_allclose(S[0, 0], np.array(case["expected_S"]), rtol=0, atol=1e-15)
    else:
        o, S, z = oracle.la_recurrent(q, k, v)
        np.testing.assert_allclose(z[0, 0], np.array(case["expected_z"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], np.array(case["expected_o"]), rtol=0, atol=1e-14)
