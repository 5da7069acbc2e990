"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Both sides get identical seeded inputs from ``workloads``.  Tolerances:
  * fp32 workloads: max |out - ref| <= 1e-5, max |L - ref| <= 1e-5, and per
    gradient tensor max |g - ref| / max |ref| <= 1e-4;
  * bf16 workloads: max |out - ref| <= 2e-2, max |L - ref| <= 2e-2, and per
    gradient tensor ||g - ref||_2 / ||ref||_2 <= 5e-2.
Where a gradient is exactly zero (one key, S = 1) the relative measures have
no scale of their own: there dp - D cancels two independently rounded O(1)
dot products.  Their denominators are floored (fp32: max |ref| at 1e-2; bf16:
the root mean square of ref at 1e-3), one to two orders below the gradients'
magnitude for the unit-variance inputs used here.
D is checked against the oracle's row sums of P * dP, with the slack that the
stored O's own error allows.  At the full sizes the oracle runs on sampled
heads (every element of those heads) and properties that hold at any size are
checked on every head.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import attention_backward_head, attention_forward_head, attention_forward_rows

torch = pytest.importorskip("torch")
import transformer_attention_xfa_amd as xfa  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_F32 = dict(out=1e-5, lse=1e-5, grad=1e-4)
TOL_BF16 = dict(out=2e-2, lse=2e-2, grad=5e-2)


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def to_dev(x, name, stream=None):
    if x.w.dtype == "bf16":
        bits = getattr(x, name + "_bits")
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(getattr(x, name))
    return t.to("cuda")


def host(t):
    return t.float().cpu().numpy()


def run_gpu(x, stream=None):
    """Forward, preprocess and backward through the C ABI; host copies (fp32)."""
    w = x.w
    say(f"run {w.name} B={w.B} H={w.H} S={w.S} hd={w.hd} {w.dtype} causal={w.causal}")
    q, k, v, do = (to_dev(x, n) for n in ("q", "k", "v", "do"))
    B, H, S, hd = w.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ctx = torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream())
    with ctx:
        xfa.xfa_fwd(q, k, v, out, lse, w.sm_scale, w.causal)
        xfa.xfa_bwd_preprocess(out, do, delta, w.sm_scale, w.causal)
        xfa.xfa_bwd(q, k, v, do, lse, delta, dq, dk, dv, w.sm_scale, w.causal)
    torch.cuda.synchronize()
    res = {n: host(t) for n, t in dict(out=out, lse=lse, delta=delta, dq=dq, dk=dk, dv=dv).items()}
    del q, k, v, do, out, lse, delta, dq, dk, dv
    torch.cuda.empty_cache()
    return res


def head(a, w, bh):
    return a.reshape(w.BH, w.S, *a.shape[3:])[bh].astype(np.float64)


def compare_head(x, g, bh, row_block=None):
    """Every element of head bh against the oracle; returns the error metrics."""
    w = x.w
    q, k, v, do = (x.f64(n, bh) for n in ("q", "k", "v", "do"))
    out_r, lse_r = attention_forward_head(q, k, v, w.sm_scale, w.causal, row_block)
    dq_r, dk_r, dv_r, dref = attention_backward_head(q, k, v, do, w.sm_scale, w.causal, row_block)
    tol = TOL_F32 if w.dtype == "f32" else TOL_BF16
    out, lse, delta = head(g["out"], w, bh), head(g["lse"], w, bh), head(g["delta"], w, bh)
    m = {"out": np.abs(out - out_r).max(), "lse": np.abs(lse - lse_r).max()}
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    for n, ref in (("dq", dq_r), ("dk", dk_r), ("dv", dv_r)):
        got = head(g[n], w, bh)
        assert np.all(np.isfinite(got)), n
        if w.dtype == "f32":
            m[n] = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-2)
        else:
            m[n] = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-3 * math.sqrt(ref.size))
    # D: exact row sums up to the error the stored O carries
    slack = np.abs(do).sum(axis=1) * tol["out"] + 1e-5 * (1 + np.abs(dref))
    m["delta"] = np.abs(delta - dref).max()
    assert np.all(np.abs(delta - dref) <= slack), f"D off by {m['delta']}"
    say(f"{w.name} head {bh}: " + " ".join(f"{n}={v:.3g}" for n, v in m.items()))
    assert m["out"] <= tol["out"], m
    assert m["lse"] <= tol["lse"], m
    for n in ("dq", "dk", "dv"):
        assert m[n] <= tol["grad"], m
    return m


def check_invariants(x, g):
    """Per head: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, Q^T dQ = dK^T K."""
    w = x.w
    worst = dict(dk_sum=0.0, dv_sum=0.0, qdq=0.0)
    for bh in range(w.BH):
        q, k, do = x.f64("q", bh), x.f64("k", bh), x.f64("do", bh)
        dq, dk, dv = head(g["dq"], w, bh), head(g["dk"], w, bh), head(g["dv"], w, bh)
        worst["dk_sum"] = max(worst["dk_sum"], np.linalg.norm(dk.sum(0)) / np.linalg.norm(dk))
        worst["dv_sum"] = max(worst["dv_sum"],
                              np.linalg.norm(dv.sum(0) - do.sum(0)) / np.linalg.norm(do.sum(0)))
        a, b = q.T @ dq, dk.T @ k
        worst["qdq"] = max(worst["qdq"], np.linalg.norm(a - b) / np.linalg.norm(b))
    say(f"{w.name} invariants over {w.BH} heads: " + " ".join(f"{n}={v:.3g}" for n, v in worst.items()))
    lim = 1e-4 if w.dtype == "f32" else 5e-2
    assert worst["dk_sum"] <= lim and worst["dv_sum"] <= lim and worst["qdq"] <= lim, worst


_CACHE = {}


def gpu_result(w):
    if w.name not in _CACHE:
        x = workloads.make_inputs(w)
        _CACHE.clear()
        _CACHE[w.name] = (x, run_gpu(x))
    return _CACHE[w.name]


# ------------------------------------------------------------- the workloads
@pytest.mark.parametrize("w", [workloads.C1, workloads.C2, workloads.C3], ids=lambda w: w.name)
def test_small_workloads_every_head(w):
    x, g = gpu_result(w)
    for bh in range(w.BH):
        compare_head(x, g, bh)
    check_invariants(x, g)


def test_c4_sampled_heads_and_invariants():
    w = workloads.C4
    x, g = gpu_result(w)
    for bh in (0, 77, w.BH - 1):
        compare_head(x, g, bh)
    check_invariants(x, g)


def test_c5_one_head():
    w = workloads.C5
    x, g = gpu_result(w)
    compare_head(x, g, 13, row_block=2048)


def test_c5_lse_stability_and_invariants():
    w = workloads.C5
    x, g = gpu_result(w)
    assert np.all(np.isfinite(g["lse"])) and np.all(np.isfinite(g["out"]))
    rng = np.random.default_rng(0)
    for bh in (0, 31):
        q, k, v = x.f64("q", bh), x.f64("k", bh), x.f64("v", bh)
        lse = head(g["lse"], w, bh)
        worst = 0.0
        for r0 in range(0, w.S, 2048):
            s = (q[r0:r0 + 2048] @ k.T) * w.sm_scale
            rows = np.arange(r0, min(r0 + 2048, w.S))
            s[np.arange(w.S)[None, :] > rows[:, None]] = -np.inf
            mx = s.max(axis=1)
            lo = mx - lse[rows]
            hi = lse[rows] - mx - np.log(rows + 1.0)
            worst = max(worst, lo.max(), hi.max())
        say(f"{w.name} head {bh}: logsumexp bound violation {worst:.3g}")
        assert worst <= 1e-3
        rows = np.sort(rng.choice(w.S, 64, replace=False))
        out_r, lse_r = attention_forward_rows(q, k, v, rows, w.sm_scale, True)
        assert np.abs(head(g["out"], w, bh)[rows] - out_r).max() <= TOL_BF16["out"]
        assert np.abs(lse[rows] - lse_r).max() <= TOL_BF16["lse"]
    check_invariants(x, g)


@pytest.mark.parametrize("w", workloads.PAGE_SHAPES, ids=lambda w: w.name)
def test_page_shapes(w):
    x, g = gpu_result(w)
    for bh in (0, w.BH - 1):
        compare_head(x, g, bh)
    check_invariants(x, g)


# ---------------------------------------------------------------- edge cases
EDGE_S = [1, 17, 64, 100, 129, 300]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("hd", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_shapes(dtype, hd, causal):
    for S in EDGE_S:
        w = workloads.Workload(f"edge_{dtype}_hd{hd}_s{S}_{'c' if causal else 'f'}", dtype, 1, 2, S, hd,
                               seed=1000 + S + hd, causal=causal, do_std=1.0 if dtype == "f32" else 0.1)
        x = workloads.make_inputs(w)
        g = run_gpu(x)
        for bh in range(w.BH):
            compare_head(x, g, bh)


# A seeded sweep of shapes drawn at random (every dtype, head dim and mode,
# lengths with ragged tails, odd head counts): a random head and the last one
# of each against the oracle, the invariants over all heads.
def _sweep_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ("f32", "bf16")[i % 2]
        hd = (16, 32, 64, 128)[(i // 2) % 4]
        causal = bool((i // 8) % 2 == 0)
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 6))
        S = int(rng.integers(2, 701))
        cases.append((dtype, B, H, S, hd, causal, int(rng.integers(0, B * H))))
    return cases


@pytest.mark.parametrize("dtype,B,H,S,hd,causal,bh", _sweep_cases())
def test_random_shape_sweep(dtype, B, H, S, hd, causal, bh):
    w = workloads.Workload(f"sweep_{dtype}_b{B}h{H}_s{S}_hd{hd}_{'c' if causal else 'f'}", dtype, B, H, S, hd,
                           seed=5000 + 7 * S + hd, causal=causal, do_std=1.0 if dtype == "f32" else 0.1)
    x = workloads.make_inputs(w)
    g = run_gpu(x)
    for b in sorted({bh, w.BH - 1}):
        compare_head(x, g, b)
    check_invariants(x, g)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_query_is_uniform_attention(dtype):
    # Q = 0: out_i is the mean of V_0..V_i and L_i = ln(i+1)
    w = workloads.Workload(f"zeroq_{dtype}", dtype, 1, 2, 200, 64, seed=7)
    x = workloads.make_inputs(w)
    x.q[...] = 0.0
    if x.q_bits is not None:
        x.q_bits[...] = 0
    g = run_gpu(x)
    for bh in range(w.BH):
        compare_head(x, g, bh)
        lse = head(g["lse"], w, bh)
        np.testing.assert_allclose(lse, np.log(np.arange(1, w.S + 1)), rtol=0, atol=1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_peaky_logits(dtype):
    # logits with standard deviation 4 (fp32) / 16 (bf16).  fp32 rounding of a
    # 64-term dot product grows with the logits' size; at std 4 it stays well
    # inside the fp32 tolerance.
    std = 2.0 if dtype == "f32" else 4.0
    w = workloads.Workload(f"peaky_{dtype}", dtype, 1, 2, 257, 64, seed=8, q_std=std, k_std=std,
                           do_std=1.0 if dtype == "f32" else 0.1)
    x = workloads.make_inputs(w)
    g = run_gpu(x)
    for bh in range(w.BH):
        compare_head(x, g, bh)


def test_nondefault_stream_and_repeatability():
    w = workloads.C3.with_(B=1, H=4)
    x = workloads.make_inputs(w)
    g0 = run_gpu(x)
    s = torch.cuda.Stream()
    g1 = run_gpu(x, stream=s)
    # every output element is produced by one workgroup: bitwise reproducible
    for n in ("out", "lse", "delta", "dq", "dk", "dv"):
        np.testing.assert_array_equal(g0[n], g1[n], err_msg=n)
    for bh in range(w.BH):
        compare_head(x, g1, bh)


# fp32 cases keep scale * sqrt(hd) below 1, the logit size of the default
# scale, where the fp32 tolerances hold (the fp32 rounding of a score grows
# with its size); each differs from 1/sqrt(hd) by a factor of 2.5 or more.
@pytest.mark.parametrize("dtype,hd,causal,scale", [
    ("f32", 64, True, 0.05), ("f32", 128, False, 0.03), ("f32", 32, True, 0.07),
    ("bf16", 128, True, 0.03), ("bf16", 64, False, 0.3), ("bf16", 16, True, 1.0),
    ("bf16", 128, True, 2.0),
])
def test_scale_other_than_default(dtype, hd, causal, scale):
    # the softmax scale enters the exponent (scale * log2 e) and the dK and
    # dQ stores; the other tests use 1/sqrt(hd)
    w = workloads.Workload(f"scale{scale}_{dtype}_hd{hd}_{'c' if causal else 'f'}", dtype, 1, 3, 333, hd,
                           seed=6000 + hd, causal=causal, scale=scale, do_std=1.0 if dtype == "f32" else 0.1)
    x = workloads.make_inputs(w)
    g = run_gpu(x)
    for bh in range(w.BH):
        compare_head(x, g, bh)
    check_invariants(x, g)


def test_concurrent_calls_on_two_streams():
    # The entry points keep no state between calls: two problems enqueued on
    # two streams at once, nothing ordering one against the other, give each
    # the result it gives alone.
    xs = [workloads.make_inputs(workloads.Workload("conc_bf16_s1100_hd128", "bf16", 1, 3, 1100, 128, seed=71, do_std=0.1)),
          workloads.make_inputs(workloads.Workload("conc_f32_s700_hd64", "f32", 2, 1, 700, 64, seed=72,
                                                   causal=False, do_std=1.0))]
    alone = [run_gpu(x) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    live = []
    torch.cuda.synchronize()
    for x, s in zip(xs, streams):
        w = x.w
        say(f"enqueue {w.name} on its own stream")
        with torch.cuda.stream(s):
            q, k, v, do = (to_dev(x, n) for n in ("q", "k", "v", "do"))
            out = torch.empty_like(q)
            lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device="cuda")
            delta = torch.empty_like(lse)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
            xfa.xfa_fwd(q, k, v, out, lse, w.sm_scale, w.causal)
            xfa.xfa_bwd_preprocess(out, do, delta, w.sm_scale, w.causal)
            xfa.xfa_bwd(q, k, v, do, lse, delta, dq, dk, dv, w.sm_scale, w.causal)
        live.append(dict(out=out, lse=lse, delta=delta, dq=dq, dk=dk, dv=dv))
    torch.cuda.synchronize()
    for x, ts, ref in zip(xs, live, alone):
        got = {n: host(t) for n, t in ts.items()}
        for n in got:
            np.testing.assert_array_equal(got[n], ref[n], err_msg=f"{x.w.name} {n}")
        compare_head(x, got, x.w.BH - 1)


def test_preprocess_beyond_one_grid_pass():
    # D = rowsum(dO * O) over 33.6 M rows of bf16 hd 128: more rows than one
    # capped grid of preprocess workgroups covers (2^20 workgroups of 32
    # rows), so the rows past 2^25 come from a second pass of the grid.
    # Inputs are drawn on the device; sampled rows, all rows of the second
    # pass and the last rows are checked against float64 dot products.
    B, H, S, hd = 8, 1025, 4096, 128
    nrows = B * H * S
    first_pass = (1 << 20) * 32
    assert nrows > first_pass
    say(f"preprocess over {nrows} rows (bf16, hd {hd})")
    g = torch.Generator(device="cuda").manual_seed(91)
    out = torch.randn((B, H, S, hd), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    do = torch.randn((B, H, S, hd), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    delta = torch.full((B, H, S), float("nan"), device="cuda")
    xfa.xfa_bwd_preprocess(out, do, delta, 1.0 / math.sqrt(hd), True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, first_pass, 4096),
                                     np.arange(first_pass, nrows),
                                     np.arange(nrows - 64, nrows)]))
    idx = torch.from_numpy(rows).cuda()
    o = out.view(nrows, hd)[idx].float().cpu().numpy().astype(np.float64)
    d = do.view(nrows, hd)[idx].float().cpu().numpy().astype(np.float64)
    got = delta.view(nrows)[idx].cpu().numpy().astype(np.float64)
    ref = (o * d).sum(axis=1)
    err = np.abs(got - ref) / (1e-6 + np.abs(o * d).sum(axis=1))
    say(f"{len(rows)} rows checked, worst relative error {err.max():.3g}")
    assert np.all(np.isfinite(got)) and err.max() <= 3e-5
    del out, do, delta
    torch.cuda.empty_cache()


def test_binding_rejects_mismatched_tensors():
    # the binding checks layout, shape and dtype itself, before any launch
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((1, 2, 64), dtype=torch.float32, device="cuda")
    bad = [
        (q.transpose(2, 3), q, q, out, lse, "contiguous"),                      # non-contiguous q
        (q, torch.zeros((1, 2, 32, 64), dtype=q.dtype, device="cuda"), q, out, lse, "shape"),  # k of another length
        (q, q, q.float(), out, lse, "dtype"),                                   # v in another dtype
        (q, q, q, out[:, :1], lse, "shape"),                                    # out of another shape
        (q, q, q, out, lse.to(torch.bfloat16), "dtype"),                        # L not float32
        (q, q, q, out, lse.cpu(), "GPU"),                                       # L on the host
    ]
    for a, b, c, o, l, what in bad:
        with pytest.raises(ValueError, match=what):
            xfa.xfa_fwd(a, b, c, o, l)
    delta = torch.empty_like(lse)
    dq = torch.empty_like(q)
    with pytest.raises(ValueError, match="shape"):
        xfa.xfa_bwd(q, q, q, q, lse, delta, torch.empty((1, 2, 8, 64), dtype=q.dtype, device="cuda"), dq, dq)
    with pytest.raises(ValueError, match="contiguous"):
        xfa.xfa_bwd_preprocess(out, q.transpose(2, 3), delta)
    torch.cuda.synchronize()


def test_empty_and_error_paths():
    q = torch.zeros((1, 1, 0, 64), dtype=torch.bfloat16, device="cuda")
    out, lse = xfa.forward(q, q, q)
    assert out.shape == q.shape and lse.shape == (1, 1, 0)
    q = torch.zeros((1, 1, 8, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(xfa.XfaError):
        xfa.forward(q, q, q)
    q = torch.zeros((1, 1, 8, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(TypeError):
        xfa.forward(q, q, q)


# ------------------------------------------------ other kernels at scale
@pytest.mark.parametrize("dtype,B,H,S,hd,causal", [
    ("bf16", 2, 4, 4096, 128, False),     # non-causal at the C4 length
    ("bf16", 1, 4, 2048, 32, True),       # small head dim over many blocks
    ("bf16", 1, 4, 2047, 16, False),      # ragged end, smallest head dim
    ("f32", 1, 2, 1024, 128, True),       # fp32 kernels at hd 128 over many blocks
    ("f32", 1, 2, 1000, 64, False),
])
def test_other_shapes_at_scale(dtype, B, H, S, hd, causal):
    w = workloads.Workload(f"scale_{dtype}_s{S}_hd{hd}_{'c' if causal else 'f'}", dtype, B, H, S, hd,
                           seed=3000 + S + hd, causal=causal, do_std=1.0 if dtype == "f32" else 0.1)
    x = workloads.make_inputs(w)
    g = run_gpu(x)
    for bh in (0, w.BH - 1):
        compare_head(x, g, bh, row_block=1024)
    check_invariants(x, g)


# ------------------------------------- dispatch groups with a short last group
# Every kernel dispatches its tiles in groups of heads (up to four; three when
# a head has 66 tiles), the group's tiles interleaved; these head counts leave
# a short last group, whose heads must map to their own tiles like the rest.
@pytest.mark.parametrize("dtype,B,H,S,hd,causal", [
    ("bf16", 1, 5, 700, 64, True),       # 4 + 1 heads
    ("bf16", 3, 2, 1100, 128, True),     # 4 + 2
    ("f32", 1, 7, 300, 32, False),       # 4 + 3
    ("bf16", 1, 4, 8448, 64, True),      # 66 tiles per head: groups of 3, 3 + 1
])
def test_dispatch_group_remainders(dtype, B, H, S, hd, causal):
    w = workloads.Workload(f"groups_{dtype}_b{B}h{H}_s{S}_hd{hd}_{'c' if causal else 'f'}", dtype, B, H, S, hd,
                           seed=4000 + S + hd, causal=causal, do_std=1.0 if dtype == "f32" else 0.1)
    x = workloads.make_inputs(w)
    g = run_gpu(x)
    for bh in (range(w.BH) if S <= 2048 else (0, w.BH - 1)):
        compare_head(x, g, bh, row_block=1024)
    check_invariants(x, g)
