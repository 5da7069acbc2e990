"""Non-finite inputs: a NaN in Q and a +Inf in V of one head propagate into
that head's outputs where the definition puts them, every call returns, and
the other heads are untouched (they match the oracle).

Workload: C3's shape and inputs (bf16, B=4, H=8, S=1024, hd=64), head 5 with
Q[300, 7] = NaN and V[500, 3] = +Inf.  By the definition
(out_i = sum_{j <= i} P_ij V_j, L_i = logsumexp_j s_ij, and the backward's
ds_ij = p_ij (dp_ij - D_i)):
  * query 300 sees only NaN logits: out[300, :], L[300], dQ[300, :] are NaN,
    and so are dK_j, dV_j of every key j <= 300 it sees;
  * queries i >= 500 see key 500: out[i, 3] is not finite, and so is
    dQ[i, :] (dp_i,500 is infinite);
  * L never involves V: L[i] for i != 300 is the oracle's L on the head
    without the planted values;
  * out[i, d] for d != 3 and i != 300 involves neither planted value.
Queries 384..499 do not see key 500, but they sit in the same 128-query
forward workgroup as queries that do: the workgroup streams key blocks up to
its last query's diagonal and multiplies the weights of masked keys (exactly
0) by V, and 0 * Inf is NaN there, as in composed attention's P.V.  So the
test claims nothing about out[384..499, 3]; rows before that tile are
claimed finite and equal to the oracle.
"""

import numpy as np
import pytest

import workloads
from oracle import attention_backward_head, attention_forward_head

torch = pytest.importorskip("torch")
import transformer_attention_xfa_amd as xfa  # noqa: E402

pytestmark = pytest.mark.gpu

BH_BAD, Q_ROW, Q_COL, V_ROW, V_COL = 5, 300, 7, 500, 3
NAN_BF16, INF_BF16 = np.uint16(0x7FC0), np.uint16(0x7F80)


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def test_nan_in_q_and_inf_in_v_of_one_head():
    w = workloads.C3
    x = workloads.make_inputs(w)
    B, H, S, hd = w.shape
    qb = x.q_bits.reshape(w.BH, S, hd).copy()
    vb = x.v_bits.reshape(w.BH, S, hd).copy()
    qb[BH_BAD, Q_ROW, Q_COL] = NAN_BF16
    vb[BH_BAD, V_ROW, V_COL] = INF_BF16

    def dev(bits):
        return torch.from_numpy(bits.reshape(w.shape).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, do = dev(qb), dev(x.k_bits), dev(vb), dev(x.do_bits)
    say(f"non-finite inputs: {w.name}, head {BH_BAD}: Q[{Q_ROW},{Q_COL}] = NaN, V[{V_ROW},{V_COL}] = +Inf")
    out, lse = xfa.forward(q, k, v, w.sm_scale, True)
    dq, dk, dv = xfa.backward(q, k, v, out, do, lse, w.sm_scale, True)
    torch.cuda.synchronize()                       # the calls return
    g = {n: t.float().cpu().numpy().reshape(w.BH, S, -1).astype(np.float64)
         for n, t in dict(out=out, dq=dq, dk=dk, dv=dv).items()}
    L = lse.cpu().numpy().reshape(w.BH, S).astype(np.float64)

    # the planted head: non-finite exactly where the definition puts it
    o5, l5 = g["out"][BH_BAD], L[BH_BAD]
    assert np.all(np.isnan(o5[Q_ROW])) and np.isnan(l5[Q_ROW])
    assert not np.any(np.isfinite(o5[V_ROW:, V_COL]))
    assert np.all(np.isnan(g["dq"][BH_BAD][Q_ROW]))
    assert not np.any(np.isfinite(g["dq"][BH_BAD][V_ROW:]))
    assert np.all(np.isnan(g["dk"][BH_BAD][:Q_ROW + 1])) and np.all(np.isnan(g["dv"][BH_BAD][:Q_ROW + 1]))
    # ... and finite, equal to the oracle on the clean head, where neither
    # planted value enters
    qc, kc, vc = (x.f64(n, BH_BAD) for n in ("q", "k", "v"))
    out_r, lse_r = attention_forward_head(qc, kc, vc, w.sm_scale, True)
    rows = np.array([i for i in range(S) if i != Q_ROW])
    assert np.all(np.isfinite(l5[rows]))
    assert np.abs(l5[rows] - lse_r[rows]).max() <= 2e-2
    clean = o5[rows][:, [d for d in range(hd) if d != V_COL]]
    ref = out_r[rows][:, [d for d in range(hd) if d != V_COL]]
    assert np.all(np.isfinite(clean)) and np.abs(clean - ref).max() <= 2e-2
    early = np.array([i for i in range(V_ROW - V_ROW % 128) if i != Q_ROW])
    assert np.all(np.isfinite(o5[early])) and np.abs(o5[early] - out_r[early]).max() <= 2e-2
    say(f"head {BH_BAD}: non-finite where defined, L and untouched outputs within 2e-2 of the oracle")

    # every other head matches the oracle
    for bh in range(w.BH):
        if bh == BH_BAD:
            continue
        a = [x.f64(n, bh) for n in ("q", "k", "v", "do")]
        o_r, l_r = attention_forward_head(*a[:3], w.sm_scale, True)
        grads_r = attention_backward_head(*a, w.sm_scale, True)[:3]
        assert np.all(np.isfinite(g["out"][bh])) and np.abs(g["out"][bh] - o_r).max() <= 2e-2, bh
        assert np.abs(L[bh] - l_r).max() <= 2e-2, bh
        for n, r in zip(("dq", "dk", "dv"), grads_r):
            got = g[n][bh]
            assert np.all(np.isfinite(got)), (bh, n)
            assert np.linalg.norm(got - r) / np.linalg.norm(r) <= 5e-2, (bh, n)
    say(f"other {w.BH - 1} heads match the oracle")
