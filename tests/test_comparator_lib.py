"""The comparator's softmax library without a GPU: it loads, exports its one
entry point and rejects bad arguments before any GPU call."""

import math

import comparator


def test_comparator_library_rejects_bad_arguments():
    f = comparator._softmax()
    A = 0x10000
    assert f(A, A, 1, 8, 0.0, 1, 1, None) == 1          # scale must be > 0
    assert f(A, A, 1, 8, math.nan, 1, 1, None) == 1
    assert f(A, A, 1, 8, 0.5, 2, 1, None) == 1          # causal in {0, 1}
    assert f(A, A, 1, 8, 0.5, 1, 2, None) == 1          # dtype in {0, 1}
    assert f(A, A, -1, 8, 0.5, 1, 1, None) == 1
    assert f(None, A, 1, 8, 0.5, 1, 1, None) == 1
    assert f(None, None, 0, 8, 0.5, 1, 1, None) == 0    # empty: nothing to do
    assert f(None, None, 3, 0, 0.5, 1, 1, None) == 0
