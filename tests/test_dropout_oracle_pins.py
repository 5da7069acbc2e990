"""Pins of the dropout oracle (oracle/dropout.py) to results fixed
independently of its code:
  * the generator's published reference outputs (splitmix64 from state 0),
    and through them the keep decision of chosen (seed, index) pairs: the
    index times the golden increment, the XOR with the seed and the 24-bit
    window >> 40 are each fixed by the same outputs;
  * the keep rate and the uniformity of u over many indices (binomial and
    chi-square bounds);
  * p = 0 reduces exactly to plain attention;
  * a pure-Python scalar brute force of attention with a given mask;
  * float64 central differences of the loss with the mask held fixed;
  * unbiasedness of inverted dropout: the mean over seeds of the dropped
    output approaches the plain output;
  * the D identity rowsum(P o dP) = dO . out.
"""

import math

import numpy as np
import pytest

from oracle import (attention_dropout_backward_head, attention_dropout_forward_head, attention_forward_head,
                    attention_backward_head, keep_mask, splitmix64)
from oracle.dropout import probs_mask

RNG = np.random.default_rng(777)


def test_splitmix64_reference_outputs():
    # the first outputs of splitmix64 seeded with 0, as published with the
    # generator: the state steps by the golden-ratio increment before mixing
    golden = 0x9E3779B97F4A7C15
    states = np.array([0, golden, (2 * golden) % 2**64], dtype=np.uint64)
    got = [int(x) for x in splitmix64(states)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


# splitmix64's first three outputs from state 0 (published with the
# generator).  With seed 0 the key of index i is i * golden, which is the
# generator's state after i steps, so h(0, i) is its output number i + 1.
SPLITMIX_FIRST = (0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F)
GOLDEN = 0x9E3779B97F4A7C15


def _keep_cases():
    """(seed, index, u) triples whose u follows from the published outputs
    alone: u = (output >> 40) / 2^24 of the output the key selects."""
    u = [(h >> 40) / float(1 << 24) for h in SPLITMIX_FIRST]
    cases = [(0, i, u[i]) for i in range(3)]
    # seed XOR index*golden selects the state: seed golden at index 1 gives
    # key 0 (output 1); seed (golden XOR 2 golden) at index 1 gives key
    # 2 golden (output 3), which an addition in place of the XOR would miss
    g2 = (2 * GOLDEN) % 2**64
    cases += [(GOLDEN, 1, u[0]), (GOLDEN ^ g2, 1, u[2]), (g2, 2, u[0])]
    return cases


@pytest.mark.parametrize("seed,index,u", _keep_cases())
def test_keep_decision_at_published_outputs(seed, index, u):
    # u = k / 2^24 is exact in float32; keep iff u >= p
    u32 = np.float32(u)
    assert float(u32) == u
    below = np.nextafter(u32, np.float32(0))
    above = np.nextafter(u32, np.float32(1))
    idx = np.array([index], dtype=np.uint64)
    assert keep_mask(seed, idx, float(below))[0]
    assert keep_mask(seed, idx, float(u32))[0]
    assert not keep_mask(seed, idx, float(above))[0]


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_rate_binomial(p):
    n = 1 << 20
    keep = keep_mask(2024, np.arange(n, dtype=np.uint64), p)
    sigma = math.sqrt(n * p * (1 - p))
    assert abs(keep.sum() - n * (1 - p)) <= 5 * sigma


def test_u_uniform_chi_square():
    n, bins = 1 << 18, 16
    # u below 1/16, 2/16, ... : keep_mask(p = b/16) drops exactly the u < b/16
    counts = []
    prev = 0
    for b in range(1, bins + 1):
        below = n - keep_mask(99, np.arange(n, dtype=np.uint64), b / bins).sum() if b < bins else n
        counts.append(below - prev)
        prev = below
    exp = n / bins
    chi2 = sum((c - exp) ** 2 / exp for c in counts)
    assert chi2 < 50.0, counts        # 15 degrees of freedom: P(chi2 > 50) < 1e-5


def test_seed_and_index_change_the_mask():
    idx = np.arange(4096, dtype=np.uint64)
    a, b = keep_mask(1, idx, 0.5), keep_mask(2, idx, 0.5)
    assert 0.4 < (a != b).mean() < 0.6
    assert np.array_equal(a, keep_mask(1, idx, 0.5))          # reproducible


def test_p_zero_is_plain_attention():
    S, hd = 33, 8
    q, k, v, do = (RNG.standard_normal((S, hd)) for _ in range(4))
    for causal in (True, False):
        o1, l1 = attention_dropout_forward_head(q, k, v, 0.3, causal, 0.0, 5, 0)
        o0, l0 = attention_forward_head(q, k, v, 0.3, causal)
        assert np.array_equal(o1, o0) and np.array_equal(l1, l0)
        g1 = attention_dropout_backward_head(q, k, v, do, 0.3, causal, 0.0, 5, 0)
        g0 = attention_backward_head(q, k, v, do, 0.3, causal)
        for a, b in zip(g1, g0):
            assert np.array_equal(a, b)


def _brute(q, k, v, do, scale, causal, M):
    """Scalar loops from the definition: out = (P o M).V, loss sum(do * out)."""
    q, k, v, do, M = (a.tolist() for a in (q, k, v, do, M))
    S, hd = len(q), len(q[0])
    P = [[0.0] * S for _ in range(S)]
    for i in range(S):
        keys = [j for j in range(S) if (not causal) or j <= i]
        logit = {j: scale * sum(q[i][d] * k[j][d] for d in range(hd)) for j in keys}
        mx = max(logit.values())
        z = sum(math.exp(logit[j] - mx) for j in keys)
        for j in keys:
            P[i][j] = math.exp(logit[j] - mx) / z
    out = [[sum(P[i][j] * M[i][j] * v[j][d] for j in range(S)) for d in range(hd)] for i in range(S)]
    # d loss / d P[i][j] = M[i][j] * sum_d do[i][d] v[j][d]
    dP = [[M[i][j] * sum(do[i][d] * v[j][d] for d in range(hd)) for j in range(S)] for i in range(S)]
    dl = [[0.0] * S for _ in range(S)]
    for i in range(S):
        r = sum(P[i][j] * dP[i][j] for j in range(S))
        for j in range(S):
            dl[i][j] = P[i][j] * (dP[i][j] - r)
    dq = [[scale * sum(dl[i][j] * k[j][d] for j in range(S)) for d in range(hd)] for i in range(S)]
    dk = [[scale * sum(dl[i][j] * q[i][d] for i in range(S)) for d in range(hd)] for j in range(S)]
    dv = [[sum(P[i][j] * M[i][j] * do[i][d] for i in range(S)) for d in range(hd)] for j in range(S)]
    return tuple(np.array(a) for a in (out, dq, dk, dv))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,hd,p,bh", [(5, 3, 0.3, 0), (8, 2, 0.5, 3), (7, 4, 0.1, 1)])
def test_dropout_brute_force(S, hd, p, bh, causal):
    q, k, v, do = (RNG.standard_normal((S, hd)) for _ in range(4))
    seed, scale = 4242, 0.7
    # the mask the oracle applies, from the pinned generator and the index rule
    idx = np.array([[(bh * S + i) * S + j for j in range(S)] for i in range(S)], dtype=np.uint64)
    M = keep_mask(seed, idx, p).astype(np.float64) / (1 - p)
    assert np.array_equal(M, probs_mask(seed, p, bh, S, 0, S))
    out_b, dq_b, dk_b, dv_b = _brute(q, k, v, do, scale, causal, M)
    out, _ = attention_dropout_forward_head(q, k, v, scale, causal, p, seed, bh)
    dq, dk, dv, _ = attention_dropout_backward_head(q, k, v, do, scale, causal, p, seed, bh)
    for a, b in ((out, out_b), (dq, dq_b), (dk, dk_b), (dv, dv_b)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_dropout_central_differences(causal):
    S, hd, p, seed, bh, scale = 6, 3, 0.4, 77, 2, 0.9
    q, k, v, do = (RNG.standard_normal((S, hd)) for _ in range(4))

    def loss(q_, k_, v_):
        o, _ = attention_dropout_forward_head(q_, k_, v_, scale, causal, p, seed, bh)
        return float((o * do).sum())

    dq, dk, dv, _ = attention_dropout_backward_head(q, k, v, do, scale, causal, p, seed, bh)
    eps = 1e-6
    for which, g in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_inverted_dropout_is_unbiased():
    S, hd, p = 16, 4, 0.5
    q, k, v = (RNG.standard_normal((S, hd)) for _ in range(3))
    plain, _ = attention_forward_head(q, k, v, 0.5, True)
    n = 600
    acc = np.zeros_like(plain)
    acc2 = np.zeros_like(plain)
    for seed in range(n):
        o, _ = attention_dropout_forward_head(q, k, v, 0.5, True, p, seed, 0)
        acc += o
        acc2 += o * o
    mean = acc / n
    std_err = np.sqrt(np.maximum(acc2 / n - mean ** 2, 0) / n)
    assert np.all(np.abs(mean - plain) <= 5 * std_err + 1e-12)


def test_dropout_d_identity():
    S, hd = 24, 5
    q, k, v, do = (RNG.standard_normal((S, hd)) for _ in range(4))
    out, _ = attention_dropout_forward_head(q, k, v, 0.6, True, 0.25, 31, 4)
    *_, dref = attention_dropout_backward_head(q, k, v, do, 0.6, True, 0.25, 31, 4)
    np.testing.assert_allclose(dref, (do * out).sum(axis=1), rtol=1e-12, atol=1e-12)
