"""The differentiable op (transformer_attention_xfa_amd.flash_attention) on
the GPU: gradients through torch.autograd against the CPU oracle, and the
memory it saves for the backward against attention composed of torch ops
(which keeps the S x S probabilities)."""

import math

import numpy as np
import pytest

import workloads
from oracle import attention_backward_head, attention_forward_head

torch = pytest.importorskip("torch")
import transformer_attention_xfa_amd as xfa  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)


CASES = [
    ("f32", 1, 2, 100, 64, True),
    ("f32", 1, 2, 77, 32, False),
    ("bf16", 1, 2, 300, 128, True),
    ("bf16", 2, 1, 129, 64, False),
]


@pytest.mark.parametrize("dtype,B,H,S,hd,causal", CASES)
def test_gradients_through_autograd(dtype, B, H, S, hd, causal):
    w = workloads.Workload(f"ag_{dtype}_{S}_{hd}", dtype, B, H, S, hd, seed=11, causal=causal)
    x = workloads.make_inputs(w)
    say(f"autograd {w.name} B={B} H={H} causal={causal}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def dev(n):
        if dtype == "bf16":
            return torch.from_numpy(getattr(x, n + "_bits").view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(getattr(x, n)).cuda()

    q, k, v = (dev(n).requires_grad_(True) for n in ("q", "k", "v"))
    do = dev("do")
    out = xfa.flash_attention(q, k, v, causal=causal)
    assert out.dtype == tdt and out.shape == q.shape
    dq, dk, dv = torch.autograd.grad(out, (q, k, v), grad_outputs=do)
    tol = dict(out=1e-5, grad=1e-4) if dtype == "f32" else dict(out=2e-2, grad=5e-2)
    for bh in range(w.BH):
        b_, h_ = divmod(bh, H)
        args = [x.f64(n, bh) for n in ("q", "k", "v")]
        o_r, _ = attention_forward_head(*args, w.sm_scale, causal)
        dq_r, dk_r, dv_r, _ = attention_backward_head(*args, x.f64("do", bh), w.sm_scale, causal)
        err = np.abs(out[b_, h_].detach().float().cpu().numpy() - o_r).max()
        assert err <= tol["out"], err
        for name, got, ref in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
            g = got[b_, h_].float().cpu().numpy()
            if dtype == "f32":
                m = np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-2)
            else:
                m = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-3 * math.sqrt(ref.size))
            say(f"  head {bh} {name}: {m:.3g}")
            assert m <= tol["grad"], (name, m)


def test_lse_is_returned_and_not_differentiable():
    torch.manual_seed(0)
    q, k, v = (torch.randn(1, 2, 64, 64, device="cuda", requires_grad=True) for _ in range(3))
    out, lse = xfa.flash_attention(q, k, v, return_lse=True)
    assert lse.shape == (1, 2, 64) and lse.dtype == torch.float32 and not lse.requires_grad
    (out.sum()).backward()
    assert q.grad is not None and k.grad is not None and v.grad is not None


def _composed(q, k, v, scale, causal):
    """Attention from torch ops in fp32; autograd keeps the S x S probabilities."""
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
    if causal:
        S = q.shape[-2]
        mask = torch.ones(S, S, dtype=torch.bool, device=q.device).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    return torch.matmul(torch.softmax(s, dim=-1), v)


def _peak(fn):
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    fn()
    torch.cuda.synchronize()
    return torch.cuda.max_memory_allocated() - base


def test_peak_memory_flash_vs_composed():
    """fp32, B=1, H=8, S=2048, hd=64: forward + backward of each path."""
    torch.manual_seed(1)
    B, H, S, hd = 1, 8, 2048, 64
    scale = 1 / math.sqrt(hd)
    q, k, v = (torch.randn(B, H, S, hd, device="cuda", requires_grad=True) for _ in range(3))
    do = torch.randn(B, H, S, hd, device="cuda")
    res = {}

    def run(fn, tag):
        def go():
            out = fn()
            res[tag] = (out.detach(),) + torch.autograd.grad(out, (q, k, v), grad_outputs=do)
        return go

    peak_c = _peak(run(lambda: _composed(q, k, v, scale, True), "composed"))
    peak_f = _peak(run(lambda: xfa.flash_attention(q, k, v, scale, True), "flash"))
    say(f"peak memory above inputs, fwd+bwd: composed {peak_c / 2**20:.1f} MiB, flash {peak_f / 2**20:.1f} MiB "
        f"(one S x S fp32 matrix per head: {B * H * S * S * 4 / 2**20:.0f} MiB)")
    # composed keeps at least the probabilities; flash keeps O(S) per row
    assert peak_c >= B * H * S * S * 4
    assert peak_f < peak_c / 4
    # and both compute the same thing
    for a, b in zip(res["composed"], res["flash"]):
        assert torch.allclose(a, b, atol=2e-4, rtol=2e-4), (a - b).abs().max().item()


@pytest.mark.parametrize("B,H,S,hd,causal", [(1, 2, 300, 128, True), (2, 1, 129, 64, False)])
def test_fp32_core_mode(B, H, S, hd, causal):
    """core="fp32" on bf16 tensors (the pages' numerics: casts at the
    boundary, fp32 kernels inside) against the oracle on the same bf16
    inputs.  Only the bf16 rounding of out and of the gradients remains, so
    its errors are within a few bf16 ulps and no larger than the native
    bf16 path's, which also rounds P and dS to bf16."""
    w = workloads.Workload(f"core_{S}_{hd}", "bf16", B, H, S, hd, seed=12, causal=causal)
    x = workloads.make_inputs(w)
    say(f"fp32 core {w.name} B={B} H={H} causal={causal}")

    def dev(n):
        return torch.from_numpy(getattr(x, n + "_bits").view(np.int16)).view(torch.bfloat16).cuda()

    errs = {}
    for core in ("fp32", "native"):
        q, k, v = (dev(n).requires_grad_(True) for n in ("q", "k", "v"))
        out = xfa.flash_attention(q, k, v, causal=causal, core=core)
        assert out.dtype == torch.bfloat16
        grads = torch.autograd.grad(out, (q, k, v), grad_outputs=dev("do"))
        e = dict(out=0.0, dq=0.0, dk=0.0, dv=0.0)
        for bh in range(w.BH):
            b_, h_ = divmod(bh, H)
            args = [x.f64(n, bh) for n in ("q", "k", "v")]
            o_r, _ = attention_forward_head(*args, w.sm_scale, causal)
            refs = attention_backward_head(*args, x.f64("do", bh), w.sm_scale, causal)[:3]
            e["out"] = max(e["out"], float(np.abs(out[b_, h_].detach().float().cpu().numpy() - o_r).max()))
            for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
                g = got[b_, h_].float().cpu().numpy()
                e[name] = max(e[name], float(np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-2)))
        errs[core] = e
        say(f"  core={core}: " + ", ".join(f"{k_} {v_:.3g}" for k_, v_ in e.items()))
    # bf16 has an 8-bit significand: one rounding is at most 2^-9 relative
    assert errs["fp32"]["out"] <= 2.0 ** -7 * 4, errs["fp32"]
    for name in ("dq", "dk", "dv"):
        assert errs["fp32"][name] <= 2.0 ** -7, (name, errs["fp32"])
    for name in errs["fp32"]:
        assert errs["fp32"][name] <= errs["native"][name] * 1.05 + 1e-6, (name, errs)


def test_double_backward_is_refused():
    # the backward is not itself differentiable: asking for it raises instead of returning wrong values
    q, k, v = (torch.randn(1, 1, 64, 32, device="cuda", requires_grad=True) for _ in range(3))
    out = xfa.flash_attention(q, k, v)
    g, = torch.autograd.grad(out.sum(), q, create_graph=True)
    with pytest.raises(RuntimeError):
        g.sum().backward()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_views_of_a_packed_projection(dtype):
    # q, k, v as strided views of one [B, S, 3, H, hd] projection (the usual
    # head split): the op takes them as they are, and the gradient reaching
    # the packed tensor equals that of the same op on contiguous copies
    B, S, H, hd = 2, 200, 3, 64
    g = torch.Generator(device="cuda").manual_seed(17)
    qkv = torch.randn((B, S, 3, H, hd), generator=g, device="cuda").to(dtype).requires_grad_(True)
    do = torch.randn((B, H, S, hd), generator=g, device="cuda").to(dtype)
    q, k, v = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    assert not q.is_contiguous()
    out = xfa.flash_attention(q, k, v)
    (gp,) = torch.autograd.grad(out, (qkv,), grad_outputs=do)
    ref = qkv.detach().clone().requires_grad_(True)
    qc, kc, vc = (ref[:, :, i].permute(0, 2, 1, 3).contiguous() for i in range(3))
    out_c = xfa.flash_attention(qc, kc, vc)
    (gr,) = torch.autograd.grad(out_c, (ref,), grad_outputs=do)
    assert torch.equal(out, out_c)
    assert torch.equal(gp, gr)
