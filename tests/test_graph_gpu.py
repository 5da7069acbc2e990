"""The three entry points captured in one HIP graph (torch.cuda.CUDAGraph on
a capture stream) and replayed: the library launches kernels only (no
allocation, memset or synchronisation), so the captured step is the eager
step.  Each replay runs on fresh inputs copied into the captured buffers,
with eager work and synchronisations in between, and must match the eager
results bit for bit (every output element is produced by one workgroup in
a fixed order)."""

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
import transformer_attention_xfa_amd as xfa  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("dtype,dropout", [("bf16", 0.0), ("f32", 0.0), ("bf16", 0.2)])
def test_step_in_a_hip_graph_replays_exactly(dtype, dropout):
    B, H, S, hd = 1, 4, 300, 128
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    scale, causal, seed = 1.0 / np.sqrt(hd), True, 77
    gen = torch.Generator(device="cuda").manual_seed(3)

    def fresh():
        return [torch.randn(B, H, S, hd, generator=gen, device="cuda").to(tdt) for _ in range(4)]

    q, k, v, do = fresh()
    out = torch.empty_like(q)
    lse = torch.empty(B, H, S, device="cuda")
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)

    def step():
        if dropout:
            xfa.xfa_fwd_dropout(q, k, v, out, lse, scale, causal, dropout, seed)
        else:
            xfa.xfa_fwd(q, k, v, out, lse, scale, causal)
        xfa.xfa_bwd_preprocess(out, do, delta, scale, causal)
        if dropout:
            xfa.xfa_bwd_dropout(q, k, v, do, lse, delta, dq, dk, dv, scale, causal, dropout, seed)
        else:
            xfa.xfa_bwd(q, k, v, do, lse, delta, dq, dk, dv, scale, causal)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.synchronize()
    say(f"captured the {dtype} step (dropout {dropout}) in a graph")
    for r in range(3):
        for t, n in zip((q, k, v, do), fresh()):
            t.copy_(n)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (out, lse, delta, dq, dk, dv)]
        step()                                  # the same step, eager, on the same inputs
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "delta", "dq", "dk", "dv"), got, (out, lse, delta, dq, dk, dv)):
            assert torch.equal(a, b), (r, name)
        assert torch.isfinite(got[0]).all() and torch.isfinite(got[3]).all()
        say(f"replay {r}: bitwise equal to the eager step")
