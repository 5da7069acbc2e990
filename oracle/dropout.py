"""Attention-probabilities dropout with a counter-based generator, float64 on
the CPU: the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the GPU
library imports this module, and this module imports nothing of it.

The generator (xtrain dropout design doc, section "RNG: counter-based"): the
keep decision of element i depends on (seed, i) only, so the backward can
regenerate the forward's mask instead of storing it:
    key  = seed XOR (i * 0x9E3779B97F4A7C15)      (arithmetic mod 2^64)
    h    = splitmix64(key)
    u    = (h >> 40) / 2^24                        (a float32 in [0, 1))
    keep = u >= p,  and kept elements are scaled by 1 / (1 - p)
(same section; the doc also fixes that u is formed and compared in float32).
splitmix64 is the published generator of Steele, Lea and Flood: its state
advances by the golden-ratio increment 0x9E3779B97F4A7C15, and the output is
the state passed through two xorshift-multiply rounds (shifts 30 and 27,
multipliers 0xBF58476D1CE4E5B9 and 0x94D049BB133111EB) and a final xorshift
by 31.  Reading: splitmix64(key) is one step of that generator from state key,
i.e. the mix of key + 0x9E3779B97F4A7C15.

Where the mask applies.  The doc declines attention-probabilities dropout for
its fused op (same doc, Goal); the variant built here applies it to the
softmax probabilities P of attention before the product with V, as inverted
dropout: with M_ij = keep_ij / (1 - p),
    out = (P o M) V,        L unchanged (it is the softmax's own logsumexp).
Element (head bh, query i, key j) of the [B*H, S, S] probabilities has index
i_flat = (bh * S + i) * S + j.  Masked-out (causal) entries have P = 0 and
their keep bit is irrelevant.

Backward, by the chain rule through the element-wise mask (a fixed linear
map for a given seed, same doc, "dropout node backward"):
    dV = (P o M)^T dO,   dPd = dO V^T (gradient of the dropped probabilities),
    dP = M o dPd,        dS = P o (dP - rowsum(P o dP)),   dQ, dK as without
dropout (times scale).  rowsum(P o dP) is returned as dref; it equals
dO_i . out_i, so the fused method's D shortcut still holds.
"""

from __future__ import annotations

import numpy as np

from .attention import _check_head, _scores, _softmax_rows

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(key) -> np.ndarray:
    """One splitmix64 step from state ``key`` (uint64 array, wrapping)."""
    z = np.asarray(key, dtype=np.uint64) + GOLDEN
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def keep_mask(seed: int, index, p: float) -> np.ndarray:
    """Keep decisions (bool) of elements with flat indices ``index``."""
    idx = np.asarray(index, dtype=np.uint64)
    key = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) ^ (idx * GOLDEN)
    h = splitmix64(key)
    u = (h >> np.uint64(40)).astype(np.float32) / np.float32(1 << 24)
    return u >= np.float32(p)


def probs_mask(seed: int, p: float, bh: int, S: int, r0: int, r1: int) -> np.ndarray:
    """M = keep / (1 - p) for query rows [r0, r1) of head bh, all S keys."""
    i = np.arange(r0, r1, dtype=np.uint64)[:, None]
    j = np.arange(S, dtype=np.uint64)[None, :]
    idx = (np.uint64(bh) * np.uint64(S) + i) * np.uint64(S) + j
    return keep_mask(seed, idx, p).astype(np.float64) / (1.0 - p)


def attention_dropout_forward_head(q, k, v, scale: float, causal: bool, p: float, seed: int, bh: int,
                                   row_block: int | None = None):
    """One head with dropout on P: (out ``[S, hd]``, lse ``[S]``), float64."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    _check_head(q, k, v)
    S = q.shape[0]
    rb = S if row_block is None else max(1, int(row_block))
    out = np.empty_like(q)
    lse = np.empty(S, dtype=np.float64)
    for r0 in range(0, S, rb):
        r1 = min(S, r0 + rb)
        pr, l_rows = _softmax_rows(_scores(q[r0:r1], k, r0, scale, causal))
        out[r0:r1] = (pr * probs_mask(seed, p, bh, S, r0, r1)) @ v
        lse[r0:r1] = l_rows
    return out, lse


def attention_dropout_backward_head(q, k, v, dout, scale: float, causal: bool, p: float, seed: int,
                                    bh: int, row_block: int | None = None):
    """One head: gradients of sum(dout * out) with dropout on P.

    Returns (dq, dk, dv, dref), dref_i = sum_j P_ij dP_ij, float64.
    """
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    _check_head(q, k, v, dout)
    S = q.shape[0]
    rb = S if row_block is None else max(1, int(row_block))
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dref = np.empty(S, dtype=np.float64)
    for r0 in range(0, S, rb):
        r1 = min(S, r0 + rb)
        pr, _ = _softmax_rows(_scores(q[r0:r1], k, r0, scale, causal))
        m = probs_mask(seed, p, bh, S, r0, r1)
        do_rows = dout[r0:r1]
        # out = (P o M).V  ->  dV = (P o M)^T.dO,  d(P o M) = dO.V^T,  dP = M o d(P o M)
        dv += (pr * m).T @ do_rows
        dp = m * (do_rows @ v.T)
        # softmax backward, then the scale and Q.K^T as without dropout
        rs = (pr * dp).sum(axis=1)
        g = pr * (dp - rs[:, None]) * scale
        dq[r0:r1] = g @ k
        dk += g.T @ q[r0:r1]
        dref[r0:r1] = rs
    return dq, dk, dv, dref
