"""The smallest workload's inputs and oracle results must not drift.

tests/golden/c1_oracle.json was written by tests/golden/make_golden.py, which
calls only the oracle and the input generator.
"""

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "c1_oracle.json")


def test_c1_golden_unchanged():
    from tests.golden.make_golden import build

    with open(GOLDEN) as f:
        ref = json.load(f)
    got = build()
    assert got["workload"] == ref["workload"]
    assert got["input_sha256"] == ref["input_sha256"]
    for key, val in ref["oracle"].items():
        np.testing.assert_allclose(np.asarray(got["oracle"][key], dtype=float),
                                   np.asarray(val, dtype=float), rtol=0, atol=1e-12)
