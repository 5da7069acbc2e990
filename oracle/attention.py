"""Composed softmax attention in float64 on the CPU: the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the GPU
library imports this module, and this module imports nothing of it.

What is computed.  The pages define attention by composition: scores are the
product Q.K^T scaled by ``scale``, a row-wise softmax turns them into
probabilities P, and the output is P.V (Autograd Engine + Op Backward design
doc, section "Attention by composition, no fused kernel"; the T14 flash
attention design doc, section "What flash-attention is", gives the same
formula with scale 1/sqrt(d)).  The causal variant sets the score of key j for
query i to -inf when j > i, so that its probability is exactly 0 (T14 design
doc, same section, paragraph on the inlined causal mask: query position is the
row index within its own sequence).  The fused kernel reaches this same result
(up to rounding order) without materialising the S x S scores; the oracle is
the plain definition and materialises them.

The forward also returns the logsumexp L of each query row's scaled, masked
logits, L_i = max_j s_ij + ln(sum_j exp(s_ij - max_j s_ij)), natural log
(T14 design doc: the recurrence's final step L = m + log(l), and Key Design
Decision 2, "the forward stores only L").

The backward follows the chain rule through the composed nodes, using the
per-op rules of the Autograd Engine design doc (table of backward maths):
  * matmul C = A.B:  dA = dC.B^T,  dB = A^T.dC;
  * scale  y = a x:  dx = a dy;
  * softmax y = softmax(x) row-wise:  dx = y * (dy - rowsum(dy * y))
    (section "Softmax backward derivation").
It deliberately uses rowsum(P * dP) itself rather than the shortcut
D_i = dO_i . O_i of the fused method (T14 design doc, Key Design Decision 3),
and returns that row sum as ``dref`` so the shortcut can be checked against it.

Queries may be processed in blocks of rows to bound memory; each block sees
every key, so a row's softmax is never split.  That only groups the sums of
the matrix products, it changes no term.
"""

from __future__ import annotations

import numpy as np

_NEG_INF = -np.inf


def _scores(q_rows: np.ndarray, k: np.ndarray, r0: int, scale: float, causal: bool) -> np.ndarray:
    """Scaled (and, if causal, masked) logits of query rows r0.. against all keys."""
    s = (q_rows @ k.T) * scale
    if causal:
        rows = np.arange(r0, r0 + q_rows.shape[0])[:, None]
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > rows, _NEG_INF, s)
    return s


def _softmax_rows(s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Row-wise safe softmax; also returns the row logsumexp (natural log)."""
    mx = s.max(axis=1)
    e = np.exp(s - mx[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], mx + np.log(l)


def _check_head(*arrs: np.ndarray) -> None:
    S, hd = arrs[0].shape
    for a in arrs:
        if a.shape != (S, hd):
            raise ValueError(f"expected [S, hd] = {(S, hd)}, got {a.shape}")


def attention_forward_head(q, k, v, scale: float, causal: bool = True,
                           row_block: int | None = None):
    """One head: q, k, v ``[S, hd]`` -> (out ``[S, hd]``, lse ``[S]``), float64."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    _check_head(q, k, v)
    S = q.shape[0]
    rb = S if row_block is None else max(1, int(row_block))
    out = np.empty_like(q)
    lse = np.empty(S, dtype=np.float64)
    for r0 in range(0, S, rb):
        r1 = min(S, r0 + rb)
        p, l_rows = _softmax_rows(_scores(q[r0:r1], k, r0, scale, causal))
        out[r0:r1] = p @ v
        lse[r0:r1] = l_rows
    return out, lse


def attention_backward_head(q, k, v, dout, scale: float, causal: bool = True,
                            row_block: int | None = None):
    """One head: gradients of the loss sum(dout * out) with respect to q, k, v.

    Returns (dq, dk, dv, dref), with dref_i = sum_j P_ij dP_ij, float64.
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
        p, _ = _softmax_rows(_scores(q[r0:r1], k, r0, scale, causal))
        do_rows = dout[r0:r1]
        # out = P.V  ->  dP = dO.V^T,  dV = P^T.dO
        dp = do_rows @ v.T
        dv += p.T @ do_rows
        # softmax backward
        rs = (p * dp).sum(axis=1)
        dsm = p * (dp - rs[:, None])
        # scale backward
        g = dsm * scale
        # scores = Q.K^T  ->  dQ = G.K,  dK = G^T.Q
        dq[r0:r1] = g @ k
        dk += g.T @ q[r0:r1]
        dref[r0:r1] = rs
    return dq, dk, dv, dref


def attention_forward_rows(q, k, v, rows, scale: float, causal: bool = True):
    """One head, selected query rows only: (out ``[len(rows), hd]``, lse).

    Each requested row i is the same definition as in attention_forward_head
    (softmax over keys j <= i when causal); used to check single rows of very
    long sequences.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    _check_head(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    s = (q[rows] @ k.T) * scale
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], _NEG_INF, s)
    p, lse = _softmax_rows(s)
    return p @ v, lse


def _heads(shape, heads):
    B, H, S, hd = shape
    return list(range(B * H)) if heads is None else [int(h) for h in heads]


def attention_forward(q, k, v, scale: float, causal: bool = True, heads=None,
                      row_block: int | None = None):
    """``[B, H, S, hd]`` inputs -> dict head -> (out, lse).

    ``heads`` selects flattened head indices bh = b*H + h (default: all).
    """
    B, H, S, hd = q.shape
    qf, kf, vf = (np.asarray(a).reshape(B * H, S, hd) for a in (q, k, v))
    return {bh: attention_forward_head(qf[bh], kf[bh], vf[bh], scale, causal, row_block)
            for bh in _heads(q.shape, heads)}


def attention_backward(q, k, v, dout, scale: float, causal: bool = True, heads=None,
                       row_block: int | None = None):
    """``[B, H, S, hd]`` inputs -> dict head -> (dq, dk, dv, dref)."""
    B, H, S, hd = q.shape
    qf, kf, vf, df = (np.asarray(a).reshape(B * H, S, hd) for a in (q, k, v, dout))
    return {bh: attention_backward_head(qf[bh], kf[bh], vf[bh], df[bh], scale, causal, row_block)
            for bh in _heads(q.shape, heads)}
