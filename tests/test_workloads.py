"""The input generator: shapes, seeds and bf16 rounding."""

import numpy as np
import pytest

import workloads


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200_000).astype(np.float32) * 3
    # exact ties between two bf16 values, both parities
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1e-40, 3e38])])
    ours = workloads.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_shapes_and_determinism():
    for w in (workloads.C1, workloads.C2):
        a = workloads.make_inputs(w)
        b = workloads.make_inputs(w)
        for n in ("q", "k", "v", "do"):
            assert getattr(a, n).shape == w.shape
            np.testing.assert_array_equal(getattr(a, n), getattr(b, n))


def test_bf16_values_are_bf16():
    w = workloads.C3.with_(B=1, H=2, S=64)
    x = workloads.make_inputs(w)
    for n in ("q", "k", "v", "do"):
        vals = getattr(x, n)
        assert np.all(vals.view(np.uint32) & 0xFFFF == 0)
        np.testing.assert_array_equal(workloads.bf16_bits_to_f32(getattr(x, n + "_bits")), vals)
    # dO carries the smaller standard deviation
    assert 0.08 < x.do.std() < 0.12 and 0.9 < x.q.std() < 1.1


def test_flop_counts():
    c4 = workloads.C4
    assert c4.pairs_per_head == 4096 * 4097 // 2
    assert abs(c4.fwd_flop - 5.499e11) / 5.499e11 < 1e-3
    assert abs(c4.bwd_flop - 1.375e12) / 1.375e12 < 1e-3
