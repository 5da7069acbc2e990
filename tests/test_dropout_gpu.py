"""GPU parity of attention-probabilities dropout: xfa_fwd_dropout and
xfa_bwd_dropout, called through the C ABI, against the CPU oracle
(``oracle.attention_dropout_forward_head`` / ``..._backward_head``).

Two kinds of check:
  * every element of every head against the oracle on seeded random inputs,
    with the plain parity tolerances (fp32: out and L 1e-5, gradients 1e-4
    of max |ref|; bf16: out and L 2e-2, gradients 5e-2 relative L2);
  * the keep decisions themselves, bit for bit: with Q = 0 every visible
    probability of row i is 1/n_i, and with V (and K) the first hd unit
    vectors, out, dV and dQ hold the mask of each kernel scaled by known
    factors, so the decision each kernel took for element (bh, i, j) is read
    back and compared with the oracle's keep_mask.  The flat indices go past
    2^32, where 32-bit index arithmetic would wrap.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import attention_dropout_backward_head, attention_dropout_forward_head, keep_mask

torch = pytest.importorskip("torch")
import transformer_attention_xfa_amd as xfa  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(out=1e-5, lse=1e-5, grad=1e-4), "bf16": dict(out=2e-2, lse=2e-2, grad=5e-2)}


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def to_dev(x, name):
    if x.w.dtype == "bf16":
        return torch.from_numpy(getattr(x, name + "_bits").view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(getattr(x, name)).to("cuda")


def run(q, k, v, do, scale, causal, p, seed):
    """Dropout forward, preprocess and backward through the C ABI."""
    B, H, S, hd = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    xfa.xfa_fwd_dropout(q, k, v, out, lse, scale, causal, p, seed)
    xfa.xfa_bwd_preprocess(out, do, delta, scale, causal)
    xfa.xfa_bwd_dropout(q, k, v, do, lse, delta, dq, dk, dv, scale, causal, p, seed)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy() for n, t in dict(out=out, lse=lse, delta=delta, dq=dq, dk=dk, dv=dv).items()}


def head(a, S, bh):
    return a.reshape(-1, S, *a.shape[3:])[bh].astype(np.float64)


def compare_head(x, g, bh, p, seed):
    w = x.w
    q, k, v, do = (x.f64(n, bh) for n in ("q", "k", "v", "do"))
    out_r, lse_r = attention_dropout_forward_head(q, k, v, w.sm_scale, w.causal, p, seed, bh)
    dq_r, dk_r, dv_r, dref = attention_dropout_backward_head(q, k, v, do, w.sm_scale, w.causal, p, seed, bh)
    tol = TOL[w.dtype]
    out, lse, delta = head(g["out"], w.S, bh), head(g["lse"], w.S, bh), head(g["delta"], w.S, bh)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    m = {"out": np.abs(out - out_r).max(), "lse": np.abs(lse - lse_r).max()}
    for n, ref in (("dq", dq_r), ("dk", dk_r), ("dv", dv_r)):
        got = head(g[n], w.S, bh)
        assert np.all(np.isfinite(got)), n
        if w.dtype == "f32":
            m[n] = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-2)
        else:
            m[n] = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-3 * math.sqrt(ref.size))
    # D = rowsum(dO * out) of the dropped output equals the oracle's rowsum(P o dP)
    slack = np.abs(do).sum(axis=1) * tol["out"] + 1e-5 * (1 + np.abs(dref))
    m["delta"] = np.abs(delta - dref).max()
    say(f"{w.name} p={p} head {bh}: " + " ".join(f"{n}={val:.3g}" for n, val in m.items()))
    assert np.all(np.abs(delta - dref) <= slack), m
    assert m["out"] <= tol["out"] and m["lse"] <= tol["lse"], m
    for n in ("dq", "dk", "dv"):
        assert m[n] <= tol["grad"], m


# ------------------------------------------------- element-wise against the oracle
CASES = [
    # dtype, B, H, S, hd, causal, p
    ("f32", 1, 2, 300, 64, True, 0.1),
    ("f32", 1, 2, 129, 128, False, 0.3),
    ("f32", 2, 1, 100, 16, True, 0.5),
    ("f32", 1, 2, 64, 32, False, 0.2),
    ("bf16", 1, 2, 300, 128, True, 0.1),
    ("bf16", 2, 1, 257, 64, False, 0.3),
    ("bf16", 1, 2, 100, 32, True, 0.5),
    ("bf16", 1, 2, 64, 16, False, 0.9),
    ("bf16", 1, 1, 1, 64, True, 0.5),
    ("bf16", 2, 4, 1024, 64, True, 0.1),
]


@pytest.mark.parametrize("dtype,B,H,S,hd,causal,p", CASES)
def test_dropout_matches_oracle(dtype, B, H, S, hd, causal, p):
    w = workloads.Workload(f"drop_{dtype}_s{S}_hd{hd}", dtype, B, H, S, hd, seed=2000 + S + hd, causal=causal,
                           do_std=1.0 if dtype == "f32" else 0.1)
    x = workloads.make_inputs(w)
    seed = 0xD1B54A32D192ED03 ^ (S * 1000003 + hd)
    say(f"run {w.name} B={B} H={H} causal={causal} p={p} seed={seed:#x}")
    g = run(*(to_dev(x, n) for n in ("q", "k", "v", "do")), w.sm_scale, causal, p, seed)
    for bh in range(w.BH):
        compare_head(x, g, bh, p, seed)


def test_dropout_c4_sampled_heads():
    # the bf16 [8, 16, 4096, 128] workload: flat indices up to 2^31 - 1
    w = workloads.C4
    x = workloads.make_inputs(w)
    p, seed = 0.1, 0x0123456789ABCDEF
    say(f"run {w.name} p={p}")
    g = run(*(to_dev(x, n) for n in ("q", "k", "v", "do")), w.sm_scale, True, p, seed)
    for bh in (0, w.BH - 1):
        compare_head(x, g, bh, p, seed)


# ---------------------------------------------------------- the keep bits, exactly
def _unit_rows(B, H, S, hd, dtype):
    """[B,H,S,hd] whose row j is the unit vector e_j for j < hd, else 0."""
    t = torch.zeros((B, H, S, hd), dtype=torch.float32)
    n = min(S, hd)
    t[:, :, torch.arange(n), torch.arange(n)] = 1.0
    return t.to(dtype).to("cuda")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,S,hd,causal,p", [
    (1, 3, 128, 128, False, 0.25),
    (1, 2, 300, 64, True, 0.5),
    (1, 20, 16384, 128, False, 0.25),     # flat indices up to 20 * 2^28 > 2^32
])
def test_keep_bits_of_every_kernel(dtype, B, H, S, hd, causal, p):
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    scale = 1.0 / math.sqrt(hd)
    seed = 0xFEDCBA9876543210
    say(f"keep bits {dtype} B={B} H={H} S={S} hd={hd} causal={causal} p={p}")
    q = torch.zeros((B, H, S, hd), dtype=tdt, device="cuda")
    ku = _unit_rows(B, H, S, hd, tdt)        # K and V: row j = e_j for j < hd
    n = min(S, hd)
    rows = np.arange(S)
    cnt = (rows + 1.0) if causal else np.full(S, float(S))       # visible keys of row i
    # run A: dO_i = e_i (i < hd) -> out[i, c] = M_ic / n_i and dV[j, c] = M_cj / n_c
    ga = run(q, ku, ku, ku, scale, causal, p, seed)
    # run B: dO = 1 -> dQ[i, c] = scale (M_ic - D_i) / n_i for c < hd
    gb = run(q, ku, ku, torch.ones_like(q), scale, causal, p, seed)
    vis = (np.arange(n)[None, :] <= rows[:, None]) if causal else np.ones((S, n), bool)
    bad = 0
    for bh in range(B * H):
        i = rows.astype(np.uint64)[:, None]
        c = np.arange(n, dtype=np.uint64)[None, :]
        ref_fwd = keep_mask(seed, (np.uint64(bh) * np.uint64(S) + i) * np.uint64(S) + c, p)    # keep(i, c)
        ref_key = keep_mask(seed, (np.uint64(bh) * np.uint64(S) + c) * np.uint64(S) + i, p)    # keep(c, j=i)
        out = head(ga["out"], S, bh)[:, :n]
        got_fwd = out * cnt[:, None] * (1 - p) > 0.5
        dv = head(ga["dv"], S, bh)[:, :n]                   # dv[j, c] = M_cj / n_c
        got_key = dv * cnt[None, :n] * (1 - p) > 0.5
        vis_key = (np.arange(n)[None, :] >= rows[:, None]) if causal else np.ones((S, n), bool)   # key j <= query c
        dq = head(gb["dq"], S, bh)[:, :n]
        d = head(gb["delta"], S, bh)
        got_q = (dq * cnt[:, None] / scale + d[:, None]) * (1 - p) > 0.5
        # invisible (causal) elements must be exactly zero wherever they show
        assert np.all(out[~vis] == 0) and np.all(dq[~vis] == 0) and np.all(dv[~vis_key] == 0)
        for name, got, ref, v in (("fwd", got_fwd, ref_fwd, vis), ("key", got_key, ref_key, vis_key),
                                  ("query", got_q, ref_fwd, vis)):
            wrong = int(np.count_nonzero((got != ref) & v))
            if wrong:
                say(f"head {bh} {name} kernel: {wrong} keep decisions differ")
            bad += wrong
        if bh == 0:
            rate = ref_fwd[vis].mean()
            say(f"head 0: keep rate {rate:.4f} over {int(vis.sum())} visible elements (1 - p = {1 - p})")
    assert bad == 0


# -------------------------------------------------------- reductions and contracts
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p_zero_is_bitwise_the_plain_path(dtype):
    w = workloads.Workload(f"p0_{dtype}", dtype, 1, 4, 300, 128, seed=31, do_std=1.0 if dtype == "f32" else 0.1)
    x = workloads.make_inputs(w)
    q, k, v, do = (to_dev(x, n) for n in ("q", "k", "v", "do"))
    g0 = run(q, k, v, do, w.sm_scale, True, 0.0, 12345)
    out, lse = xfa.forward(q, k, v, w.sm_scale, True)
    dq, dk, dv = xfa.backward(q, k, v, out, do, lse, w.sm_scale, True)
    torch.cuda.synchronize()
    for n, t in dict(out=out, lse=lse, dq=dq, dk=dk, dv=dv).items():
        np.testing.assert_array_equal(g0[n], t.float().cpu().numpy(), err_msg=n)


def test_same_seed_reproduces_and_other_seed_differs():
    w = workloads.C3.with_(B=1, H=2)
    x = workloads.make_inputs(w)
    args = [to_dev(x, n) for n in ("q", "k", "v", "do")]
    g1 = run(*args, w.sm_scale, True, 0.2, 99)
    g2 = run(*args, w.sm_scale, True, 0.2, 99)
    g3 = run(*args, w.sm_scale, True, 0.2, 100)
    for n in ("out", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(g1[n], g2[n], err_msg=n)
    np.testing.assert_array_equal(g1["lse"], g3["lse"])      # L does not see the mask
    for n in ("out", "dq", "dk", "dv"):
        assert np.mean(g1[n] != g3[n]) > 0.5, n


def test_autograd_with_dropout():
    # flash_attention(dropout_p, seed) differentiates through the same mask
    B, H, S, hd, p, seed = 1, 2, 200, 64, 0.2, 4242
    gen = torch.Generator().manual_seed(5)
    q, k, v = (torch.randn(B, H, S, hd, generator=gen) for _ in range(3))
    do = torch.randn(B, H, S, hd, generator=gen)
    qd, kd, vd = (t.cuda().requires_grad_(True) for t in (q, k, v))
    out = xfa.flash_attention(qd, kd, vd, causal=True, dropout_p=p, seed=seed)
    out.backward(do.cuda())
    scale = 1.0 / math.sqrt(hd)
    for bh in range(B * H):
        b, h = divmod(bh, H)
        args = [t[b, h].double().numpy() for t in (q, k, v)]
        out_r, _ = attention_dropout_forward_head(*args, scale, True, p, seed, bh)
        dq_r, dk_r, dv_r, _ = attention_dropout_backward_head(*args, do[b, h].double().numpy(), scale, True, p,
                                                              seed, bh)
        np.testing.assert_allclose(out[b, h].detach().cpu().double().numpy(), out_r, rtol=0, atol=1e-5)
        for got, ref in ((qd.grad, dq_r), (kd.grad, dk_r), (vd.grad, dv_r)):
            g = got[b, h].cpu().double().numpy()
            assert np.abs(g - ref).max() <= 1e-4 * max(np.abs(ref).max(), 1e-2)


def test_autograd_dropout_bf16_native_and_fp32_core():
    # bf16 tensors through the op with dropout, in both modes, against the oracle on the same mask
    B, H, S, hd, p, seed = 1, 2, 257, 128, 0.15, 31337
    gen = torch.Generator().manual_seed(9)
    q, k, v = (torch.randn(B, H, S, hd, generator=gen).to(torch.bfloat16) for _ in range(3))
    do = (torch.randn(B, H, S, hd, generator=gen) * 0.1).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(hd)
    for core in ("native", "fp32"):
        qd, kd, vd = (t.cuda().requires_grad_(True) for t in (q, k, v))
        out = xfa.flash_attention(qd, kd, vd, causal=True, dropout_p=p, seed=seed, core=core)
        out.backward(do.cuda())
        for bh in range(B * H):
            b, h = divmod(bh, H)
            args = [t[b, h].double().numpy() for t in (q, k, v)]
            out_r, _ = attention_dropout_forward_head(*args, scale, True, p, seed, bh)
            grads_r = attention_dropout_backward_head(*args, do[b, h].double().numpy(), scale, True, p, seed, bh)[:3]
            e_out = np.abs(out[b, h].detach().float().cpu().numpy() - out_r).max()
            errs = [np.linalg.norm(g[b, h].float().cpu().numpy() - r) / np.linalg.norm(r)
                    for g, r in zip((qd.grad, kd.grad, vd.grad), grads_r)]
            say(f"dropout autograd core={core} head {bh}: out {e_out:.3g} grads " + " ".join(f"{e:.3g}" for e in errs))
            assert e_out <= 2e-2 and max(errs) <= 5e-2
