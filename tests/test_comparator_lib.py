"""The comparator library without a GPU: it loads, exports its entry points
and rejects bad arguments before any GPU call."""

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


def test_atomic_floor_rejects_bad_arguments():
    f = comparator._floor()
    A = 0x10000
    assert f(A, 1, 64, 48, 1, None) == 1            # hd in {16, 32, 64, 128}
    assert f(A, 1, 64, 64, 2, None) == 1            # causal in {0, 1}
    assert f(A, -1, 64, 64, 1, None) == 1
    assert f(None, 1, 64, 64, 1, None) == 1
    assert f(None, 0, 64, 64, 1, None) == 0         # empty: nothing to do
    assert f(None, 2, 0, 64, 1, None) == 0


def test_atomic_floor_expected_counts():
    e = comparator.dq_atomic_floor_expected(300, 16, True)
    assert e.shape == (300, 16)
    assert e[0, 0] == 1 and e[127, 3] == 1 and e[128, 0] == 2 and e[299, 15] == 3
    assert (comparator.dq_atomic_floor_expected(300, 16, False) == 3).all()
