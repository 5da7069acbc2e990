"""Pins of the CPU oracle to results fixed independently of its code.

Each test checks the oracle against something other than itself:
  * a pure-Python scalar brute force written from the definition element by
    element (no NumPy, no matrix products);
  * float64 central differences of the loss sum(dO * out);
  * torch's own CPU scaled-dot-product attention and autograd in float64;
  * closed forms (Q = 0, a single key, two keys as a logistic function);
  * invariants (rows of P sum to 1, the D identity, shift invariance,
    gradient sums, logsumexp bounds, linearity in V).
A plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong mask direction, log base) fails at least one.
"""

import math

import numpy as np
import pytest

from oracle import (attention_backward, attention_backward_head, attention_forward,
                    attention_forward_head, attention_forward_rows)

RNG = np.random.default_rng(12345)


def _rand(S, hd, std=1.0, rng=RNG):
    return rng.standard_normal((S, hd)) * std


# --------------------------------------------------------------- brute force
def _brute(q, k, v, do, scale, causal):
    """Scalar loops straight from the definition; lists and math only."""
    q, k, v, do = (a.tolist() for a in (q, k, v, do))
    S, hd = len(q), len(q[0])
    P = [[0.0] * S for _ in range(S)]
    out = [[0.0] * hd for _ in range(S)]
    lse = [0.0] * S
    for i in range(S):
        keys = [j for j in range(S) if (not causal) or j <= i]
        logit = {}
        for j in keys:
            acc = 0.0
            for d in range(hd):
                acc += q[i][d] * k[j][d]
            logit[j] = acc * scale
        mx = max(logit.values())
        z = 0.0
        for j in keys:
            z += math.exp(logit[j] - mx)
        lse[i] = mx + math.log(z)
        for j in keys:
            P[i][j] = math.exp(logit[j] - mx) / z
        for d in range(hd):
            acc = 0.0
            for j in keys:
                acc += P[i][j] * v[j][d]
            out[i][d] = acc
    # d loss / d P[i][j] for loss = sum_{i,d} do[i][d] * out[i][d]
    dP = [[sum(do[i][d] * v[j][d] for d in range(hd)) for j in range(S)] for i in range(S)]
    dlogit = [[0.0] * S for _ in range(S)]
    dref = [0.0] * S
    for i in range(S):
        r = 0.0
        for j in range(S):
            r += P[i][j] * dP[i][j]
        dref[i] = r
        for j in range(S):
            # d softmax_j / d logit_t = P_j (delta_jt - P_t)
            dlogit[i][j] = P[i][j] * (dP[i][j] - r)
    dq = [[scale * sum(dlogit[i][j] * k[j][d] for j in range(S)) for d in range(hd)] for i in range(S)]
    dk = [[scale * sum(dlogit[i][j] * q[i][d] for i in range(S)) for d in range(hd)] for j in range(S)]
    dv = [[sum(P[i][j] * do[i][d] for i in range(S)) for d in range(hd)] for j in range(S)]
    return tuple(np.array(a) for a in (out, lse, dq, dk, dv, dref))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,hd", [(1, 1), (2, 3), (5, 4), (8, 2), (7, 3)])
def test_brute_force(S, hd, causal):
    rng = np.random.default_rng(S * 100 + hd + 7 * causal)
    q, k, v, do = (_rand(S, hd, rng=rng) for _ in range(4))
    scale = 0.7
    out, lse = attention_forward_head(q, k, v, scale, causal)
    dq, dk, dv, dref = attention_backward_head(q, k, v, do, scale, causal)
    b_out, b_lse, b_dq, b_dk, b_dv, b_dref = _brute(q, k, v, do, scale, causal)
    for got, ref in ((out, b_out), (lse, b_lse), (dq, b_dq), (dk, b_dk), (dv, b_dv), (dref, b_dref)):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_causal_mask_direction():
    # Changing a key/value that lies after query i must not change row i.
    S, hd = 6, 3
    q, k, v = (_rand(S, hd) for _ in range(3))
    out, lse = attention_forward_head(q, k, v, 0.5, True)
    k2, v2 = k.copy(), v.copy()
    k2[4] += 3.0
    v2[4] -= 2.0
    out2, lse2 = attention_forward_head(q, k2, v2, 0.5, True)
    np.testing.assert_array_equal(out[:4], out2[:4])
    np.testing.assert_array_equal(lse[:4], lse2[:4])
    assert np.abs(out[4:] - out2[4:]).max() > 1e-3


# --------------------------------------------------------- finite differences
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,hd", [(7, 3), (5, 4)])
def test_central_differences(S, hd, causal):
    rng = np.random.default_rng(99 + S)
    q, k, v, do = (_rand(S, hd, rng=rng) for _ in range(4))
    scale = 1.0 / math.sqrt(hd)
    dq, dk, dv, _ = attention_backward_head(q, k, v, do, scale, causal)

    def loss(qq, kk, vv):
        o, _ = attention_forward_head(qq, kk, vv, scale, causal)
        return float((o * do).sum())

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = [q, k, v]
        fd = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=0, atol=1e-7)


# ------------------------------------------------------- torch CPU reference
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,hd,scale", [(37, 16, 0.25), (64, 8, None), (100, 32, 0.1)])
def test_torch_sdpa_float64(S, hd, scale, causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(S + hd)
    q, k, v, do = (_rand(S, hd, rng=rng) for _ in range(4))
    sc = 1.0 / math.sqrt(hd) if scale is None else scale
    qt, kt, vt = (torch.tensor(a[None, None], dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=sc)
    (ot * torch.tensor(do[None, None])).sum().backward()
    logits = (torch.tensor(q) @ torch.tensor(k).T) * sc
    if causal:
        logits = logits.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    lse_t = torch.logsumexp(logits, dim=1).numpy()

    out, lse = attention_forward_head(q, k, v, sc, causal)
    dq, dk, dv, _ = attention_backward_head(q, k, v, do, sc, causal)
    np.testing.assert_allclose(out, ot.detach().numpy()[0, 0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, lse_t, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dq, qt.grad.numpy()[0, 0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy()[0, 0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy()[0, 0], rtol=0, atol=1e-11)


# --------------------------------------------------------------- closed forms
def test_zero_query_closed_form():
    # Q = 0: every unmasked logit is 0, so row i averages V_0..V_i and
    # L_i = ln(i+1); p_ij = 1/(i+1) gives the backward in closed form.
    S, hd, scale = 23, 5, 0.3
    k, v, do = (_rand(S, hd) for _ in range(3))
    q = np.zeros((S, hd))
    out, lse = attention_forward_head(q, k, v, scale, True)
    cnt = np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(out, np.cumsum(v, axis=0) / cnt, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.arange(1, S + 1)), rtol=0, atol=1e-13)

    dq, dk, dv, _ = attention_backward_head(q, k, v, do, scale, True)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)
    dv_ref = np.array([sum(do[i] / (i + 1) for i in range(j, S)) for j in range(S)])
    np.testing.assert_allclose(dv, dv_ref, rtol=0, atol=1e-12)
    dq_ref = np.array([scale / (i + 1) * sum((do[i] @ (v[j] - out[i])) * k[j] for j in range(i + 1))
                       for i in range(S)])
    np.testing.assert_allclose(dq, dq_ref, rtol=0, atol=1e-12)


def test_single_key():
    # S = 1: the only probability is 1.
    q, k, v, do = (_rand(1, 6) for _ in range(4))
    out, lse = attention_forward_head(q, k, v, 0.4, True)
    np.testing.assert_allclose(out, v, atol=1e-15)
    np.testing.assert_allclose(lse, [0.4 * float(q[0] @ k[0])], atol=1e-15)
    dq, dk, dv, _ = attention_backward_head(q, k, v, do, 0.4, True)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, do, atol=1e-15)


def test_first_row():
    # Row 0 of a causal head sees only key 0: out_0 = V_0, L_0 = s_00, dQ_0 = 0.
    S, hd, scale = 9, 4, 0.5
    q, k, v, do = (_rand(S, hd) for _ in range(4))
    out, lse = attention_forward_head(q, k, v, scale, True)
    dq, _, _, _ = attention_backward_head(q, k, v, do, scale, True)
    np.testing.assert_allclose(out[0], v[0], atol=1e-15)
    np.testing.assert_allclose(lse[0], scale * float(q[0] @ k[0]), atol=1e-15)
    np.testing.assert_allclose(dq[0], 0.0, atol=1e-15)


def test_two_keys_logistic():
    # Two keys: P_11 = sigmoid(s_11 - s_10), so with hd = 1 every output is a
    # logistic function of scale * q1 * (k1 - k0).
    scale = 0.9
    q = np.array([[0.3], [1.7]])
    k = np.array([[-0.4], [0.8]])
    v = np.array([[2.0], [-1.5]])
    do = np.array([[0.6], [-1.1]])
    out, lse = attention_forward_head(q, k, v, scale, True)
    x = scale * q[1, 0] * (k[1, 0] - k[0, 0])
    sig = 1.0 / (1.0 + math.exp(-x))
    assert abs(out[1, 0] - (sig * v[1, 0] + (1 - sig) * v[0, 0])) < 1e-15
    s10, s11 = scale * q[1, 0] * k[0, 0], scale * q[1, 0] * k[1, 0]
    assert abs(lse[1] - (s10 + math.log1p(math.exp(s11 - s10)))) < 1e-15
    dq, dk, dv, _ = attention_backward_head(q, k, v, do, scale, True)
    # d out_1 / d x = sig (1 - sig) (v1 - v0)
    dxd = do[1, 0] * sig * (1 - sig) * (v[1, 0] - v[0, 0])
    assert abs(dq[1, 0] - dxd * scale * (k[1, 0] - k[0, 0])) < 1e-14
    assert abs(dk[1, 0] - dxd * scale * q[1, 0]) < 1e-14
    assert abs(dk[0, 0] + dxd * scale * q[1, 0]) < 1e-14
    assert abs(dv[1, 0] - do[1, 0] * sig) < 1e-15
    assert abs(dv[0, 0] - (do[0, 0] + do[1, 0] * (1 - sig))) < 1e-15


# ---------------------------------------------------------------- invariants
def test_rows_stochastic():
    S, hd = 40, 6
    q, k = _rand(S, hd, 2.0), _rand(S, hd, 2.0)
    for causal in (True, False):
        out, _ = attention_forward_head(q, k, np.ones((S, hd)), 0.6, causal)
        np.testing.assert_allclose(out, 1.0, atol=1e-13)


def test_d_identity():
    S, hd = 50, 8
    q, k, v, do = (_rand(S, hd) for _ in range(4))
    out, _ = attention_forward_head(q, k, v, 0.35, True)
    *_, dref = attention_backward_head(q, k, v, do, 0.35, True)
    np.testing.assert_allclose((do * out).sum(axis=1), dref, rtol=0, atol=1e-12)


def test_shift_invariance():
    S, hd, scale = 33, 7, 0.45
    q, k, v = (_rand(S, hd) for _ in range(3))
    c = RNG.standard_normal(hd)
    out, lse = attention_forward_head(q, k, v, scale, True)
    out2, lse2 = attention_forward_head(q, k + c[None, :], v, scale, True)
    np.testing.assert_allclose(out2, out, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + scale * (q @ c), atol=1e-12)


def test_gradient_sums():
    S, hd, scale = 45, 6, 0.5
    q, k, v, do = (_rand(S, hd) for _ in range(4))
    for causal in (True, False):
        dq, dk, dv, _ = attention_backward_head(q, k, v, do, scale, causal)
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
        np.testing.assert_allclose(q.T @ dq, dk.T @ k, atol=1e-12)


def test_lse_bounds():
    S, hd, scale = 60, 8, 0.8
    q, k, v = _rand(S, hd, 1.5), _rand(S, hd, 1.5), _rand(S, hd)
    _, lse = attention_forward_head(q, k, v, scale, True)
    s = (q @ k.T) * scale
    mx = np.array([s[i, : i + 1].max() for i in range(S)])
    assert np.all(lse >= mx - 1e-12)
    assert np.all(lse <= mx + np.log(np.arange(1, S + 1)) + 1e-12)


def test_linear_in_v():
    S, hd = 30, 5
    q, k, v1, v2 = (_rand(S, hd) for _ in range(4))
    o1, _ = attention_forward_head(q, k, v1, 0.5, True)
    o2, _ = attention_forward_head(q, k, v2, 0.5, True)
    o12, _ = attention_forward_head(q, k, v1 + 2.0 * v2, 0.5, True)
    np.testing.assert_allclose(o12, o1 + 2.0 * o2, atol=1e-12)


def test_row_blocks_match_whole():
    S, hd = 70, 4
    q, k, v, do = (_rand(S, hd) for _ in range(4))
    for causal in (True, False):
        a = attention_forward_head(q, k, v, 0.5, causal)
        b = attention_forward_head(q, k, v, 0.5, causal, row_block=16)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-13)
        a = attention_backward_head(q, k, v, do, 0.5, causal)
        b = attention_backward_head(q, k, v, do, 0.5, causal, row_block=9)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


def test_batched_heads_independent():
    B, H, S, hd = 2, 3, 12, 4
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal((B, H, S, hd)) for _ in range(4))
    fw = attention_forward(q, k, v, 0.5, True)
    bw = attention_backward(q, k, v, do, 0.5, True, heads=[4])
    assert sorted(fw) == list(range(B * H))
    o, l = attention_forward_head(q[1, 1], k[1, 1], v[1, 1], 0.5, True)
    np.testing.assert_array_equal(fw[4][0], o)
    np.testing.assert_array_equal(fw[4][1], l)
    ref = attention_backward_head(q[1, 1], k[1, 1], v[1, 1], do[1, 1], 0.5, True)
    for x, y in zip(bw[4], ref):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("causal", [True, False])
def test_selected_rows(causal):
    S, hd = 8, 3
    rng = np.random.default_rng(77)
    q, k, v, do = (_rand(S, hd, rng=rng) for _ in range(4))
    rows = [7, 0, 3, 3, 5]
    out, lse = attention_forward_rows(q, k, v, rows, 0.6, causal)
    b_out, b_lse, *_ = _brute(q, k, v, do, 0.6, causal)
    np.testing.assert_allclose(out, b_out[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, b_lse[rows], rtol=0, atol=1e-12)
