"""The composed-attention comparator (comparator.py) computes the same
attention as the fused op: both against the CPU oracle on small bf16 and fp32
cases, so the benchmark A/B compares like with like."""

import numpy as np
import pytest

import workloads
from oracle import attention_backward_head, attention_forward_head

torch = pytest.importorskip("torch")
import comparator  # noqa: E402
import transformer_attention_xfa_amd as xfa  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("dtype,S,hd,causal", [("bf16", 256, 64, True), ("f32", 200, 32, False)])
def test_composed_matches_oracle_and_fused(dtype, S, hd, causal):
    w = workloads.Workload(f"cmp_{dtype}_{S}", dtype, 1, 2, S, hd, seed=13, causal=causal)
    x = workloads.make_inputs(w)
    say(f"comparator {w.name} causal={causal}")
    if dtype == "bf16":
        q, k, v, do = (torch.from_numpy(getattr(x, n + "_bits").view(np.int16)).view(torch.bfloat16).cuda()
                       for n in ("q", "k", "v", "do"))
    else:
        q, k, v, do = (torch.from_numpy(getattr(x, n)).cuda() for n in ("q", "k", "v", "do"))
    out_c, p = comparator.composed_forward(q, k, v, w.sm_scale, causal)
    grads_c = comparator.composed_backward(q, k, v, p, out_c, do, w.sm_scale)
    out_f, lse = xfa.forward(q, k, v, w.sm_scale, causal)
    grads_f = xfa.backward(q, k, v, out_f, do, lse, w.sm_scale, causal)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    for bh in range(w.BH):
        args = [x.f64(n, bh) for n in ("q", "k", "v")]
        o_r, _ = attention_forward_head(*args, w.sm_scale, causal)
        refs = (o_r,) + tuple(attention_backward_head(*args, x.f64("do", bh), w.sm_scale, causal)[:3])
        for name, c, f, r in zip(("out", "dq", "dk", "dv"), (out_c,) + tuple(grads_c), (out_f,) + tuple(grads_f), refs):
            den = max(np.abs(r).max(), 1e-2)
            ec = np.abs(c[0, bh].float().cpu().numpy() - r).max() / den
            ef = np.abs(f[0, bh].float().cpu().numpy() - r).max() / den
            say(f"  head {bh} {name}: composed {ec:.3g} fused {ef:.3g}")
            assert ec <= tol and ef <= tol, (name, ec, ef)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S,causal", [(256, True), (300, True), (200, False), (1, True)])
def test_causal_softmax_kernel(dtype, S, causal):
    # the comparator's softmax step against float64 NumPy on the same scores
    # (S = 300 and 200 take the kernel's unaligned per-element path)
    rng = np.random.default_rng(S)
    x = (rng.standard_normal((1, 2, S, S)) * 3).astype(np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xs = t.float().cpu().numpy().astype(np.float64) * 0.125
    if causal:
        xs = np.where(np.arange(S)[None, :] > np.arange(S)[:, None], -np.inf, xs)
    ref = np.exp(xs - xs.max(-1, keepdims=True))
    ref /= ref.sum(-1, keepdims=True)
    p = comparator.causal_softmax(t, 0.125, causal)
    torch.cuda.synchronize()
    got = p.float().cpu().numpy()
    err = np.abs(got - ref).max()
    say(f"causal_softmax {dtype} S={S} causal={causal}: max err {err:.3g}")
    assert err <= (4e-3 if dtype == "bf16" else 1e-6)
    if causal:
        assert np.all(got[..., np.triu_indices(S, 1)[0], np.triu_indices(S, 1)[1]] == 0)


@pytest.mark.parametrize("S,hd,causal", [(300, 64, True), (257, 32, False), (1024, 128, True)])
def test_atomic_floor_counts(S, hd, causal):
    say(f"atomic floor S={S} hd={hd} causal={causal}")
    acc = torch.zeros((2, 3, S, hd), dtype=torch.float32, device="cuda")
    comparator.dq_atomic_floor(acc, causal)
    torch.cuda.synchronize()
    exp = torch.from_numpy(comparator.dq_atomic_floor_expected(S, hd, causal)).cuda()
    assert torch.equal(acc, exp.expand_as(acc))
