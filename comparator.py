"""The composed attention path on MI355X, as a benchmark comparator for the
fused op (T14 flash-attention design doc: the composed path the fused kernel
replaces, and its measured-results section, which compares the two on
throughput and peak memory).

Composed attention materialises the scores: S = Q K^T by a batched library
GEMM (hipBLASLt through torch), then a causal row softmax written as a HIP
kernel of its own (comparator_kernels/causal_softmax.hip: scale, mask and
softmax in one pass over the scores, writing the [B, H, S, S] probabilities
P in the inputs' dtype), then out = P V by a second GEMM; the backward keeps
P and forms dV, dP, dS, dQ, dK with three more GEMMs and elementwise work on
S x S tensors.  This is a comparator, not a second implementation of the op:
it computes all S*S products where the fused op skips the masked half.
Every batched product is given contiguous operands (the transposes are
formed as small [.., hd, S] copies).

dq_atomic_floor_record() times the other comparator in the same library
(comparator_kernels/dq_atomic_floor.hip): the fp32 atomic traffic alone that
summing dQ across key workgroups would need, the alternative to the fused
op's separate query-outer dQ kernel.
"""
from __future__ import annotations

import time

import numpy as np


_softmax_lib = None


def _softmax():
    """xfa_comparator_causal_softmax from comparator_kernels/libcomposed.so."""
    global _softmax_lib
    if _softmax_lib is None:
        import ctypes
        import os

        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "comparator_kernels", "libcomposed.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(path)
        fn = lib.xfa_comparator_causal_softmax
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                       ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        _softmax_lib = fn
    return _softmax_lib


_floor_fn = None


def _floor():
    """xfa_comparator_dq_atomic_floor from comparator_kernels/libcomposed.so."""
    global _floor_fn
    if _floor_fn is None:
        import ctypes

        _softmax()                          # loads (or reports) the library
        import os

        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "comparator_kernels", "libcomposed.so")
        fn = ctypes.CDLL(path).xfa_comparator_dq_atomic_floor
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                       ctypes.c_void_p]
        _floor_fn = fn
    return _floor_fn


def dq_atomic_floor(acc, causal):
    """One launch of the atomic-floor kernel on a [B, H, S, hd] fp32 buffer."""
    import torch

    B, H, S, hd = acc.shape
    assert acc.is_contiguous() and acc.dtype == torch.float32 and acc.is_cuda
    st = _floor()(acc.data_ptr(), B * H, S, hd, int(bool(causal)), torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise RuntimeError(f"xfa_comparator_dq_atomic_floor failed (status {st})")


def dq_atomic_floor_expected(S, hd, causal):
    """acc[bh, q, d] after one launch on zeros: the key workgroups (128 keys)
    that see query q."""
    nkt = (S + 127) // 128
    rows = (np.arange(S) // 128 + 1) if causal else np.full(S, nkt)
    return np.repeat(rows[:, None].astype(np.float32), hd, axis=1)


def dq_atomic_floor_record(w, steps, bwd_ms=None):
    """Time of the minimum fp32 atomic traffic the atomic dQ design needs on
    workload w, checked once for its counts; bwd_ms is the fused backward's
    time for comparison."""
    import torch

    B, H, S, hd = w.shape
    acc = torch.zeros((B, H, S, hd), dtype=torch.float32, device="cuda")
    dq_atomic_floor(acc, w.causal)
    torch.cuda.synchronize()
    exp = torch.from_numpy(dq_atomic_floor_expected(S, hd, w.causal)).cuda()
    ok = bool(torch.equal(acc, exp.expand_as(acc)))
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(steps):
        acc.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dq_atomic_floor(acc, w.causal)
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in times]))
    nkt = (S + 127) // 128
    nb = (S + 31) // 32
    blocks = sum(nb - 4 * kt for kt in range(nkt)) if w.causal else nkt * nb
    ops = B * H * blocks * 32 * hd
    rec = {
        "kind": "fp32 atomic adds of the atomic dQ design alone: one per dQ element per "
                "(128-key workgroup, 32-query block) pair, no loads or matrix work",
        "kernel": "dq_atomic_floor_kernel", "atomic_lane_ops": int(ops), "avg_ms": round(ms, 4),
        "g_atomics_per_s": round(ops / (ms * 1e-3) / 1e9, 1), "counts_exact": ok,
    }
    if bwd_ms:
        rec["fused_bwd_ms"] = round(bwd_ms, 4)
        rec["floor_over_fused_bwd"] = round(ms / bwd_ms, 2)
    return rec


def causal_softmax(s, scale, causal):
    """P = softmax(mask(s * scale)) row by row for contiguous [..., S, S]
    scores (bf16 or fp32) on the GPU, by the comparator's HIP kernel."""
    import torch

    S = s.shape[-1]
    assert s.is_contiguous() and s.shape[-2] == S and s.dtype in (torch.bfloat16, torch.float32)
    p = torch.empty_like(s)
    st = _softmax()(s.data_ptr(), p.data_ptr(), s.numel() // (S * S), S, float(scale), int(bool(causal)),
                    1 if s.dtype == torch.bfloat16 else 0, torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise RuntimeError(f"xfa_comparator_causal_softmax failed (status {st})")
    return p


def composed_forward(q, k, v, scale, causal):
    """out, P for [B, H, S, hd] q, k, v (P kept for the backward)."""
    import torch

    s = torch.matmul(q, k.transpose(-1, -2).contiguous())
    p = causal_softmax(s, scale, causal)
    del s
    return torch.matmul(p, v), p


def composed_backward(q, k, v, p, out, do, scale):
    """dq, dk, dv of sum(do * out) from the kept probabilities p."""
    import torch

    dv = torch.matmul(do.transpose(-1, -2).contiguous(), p).transpose(-1, -2)      # (dO^T P)^T = P^T dO
    dp = torch.matmul(do, v.transpose(-1, -2).contiguous()).float()
    delta = (do.float() * out.float()).sum(-1, keepdim=True)
    ds = (p.float() * (dp - delta) * scale).to(q.dtype)
    del dp
    dq = torch.matmul(ds, k)
    dk = torch.matmul(q.transpose(-1, -2).contiguous(), ds).transpose(-1, -2)     # (Q^T dS)^T = dS^T Q
    return dq, dk.contiguous(), dv.contiguous()


def bench_composed(q, k, v, do, scale, causal, steps, warmup):
    """Average fwd and bwd times (HIP events on the current stream) and the
    peak memory above the inputs of one fwd + bwd step, for the composed path
    and for the fused op (its outputs and O(S) buffers allocated inside the
    measured step the same way)."""
    import torch

    import transformer_attention_xfa_amd as xfa

    stream = torch.cuda.current_stream()

    def composed_step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        out, p = composed_forward(q, k, v, scale, causal)
        if ev is not None:
            ev[1].record(stream)
        grads = composed_backward(q, k, v, p, out, do, scale)
        if ev is not None:
            ev[2].record(stream)
        return out, grads

    def fused_step():
        out, lse = xfa.forward(q, k, v, scale, causal)
        return out, xfa.backward(q, k, v, out, do, lse, scale, causal)

    def peak(fn):
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        r = fn()
        torch.cuda.synchronize()
        p_ = torch.cuda.max_memory_allocated() - base
        del r
        return p_

    for _ in range(warmup):
        composed_step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        composed_step(events[i])
    torch.cuda.synchronize()
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    peak_c = peak(composed_step)
    peak_f = peak(fused_step)
    return {"fwd_ms": fwd, "bwd_ms": bwd, "peak_bytes": int(peak_c), "fused_peak_bytes": int(peak_f)}


def comparator_record(x, steps, warmup, fused_ms_step):
    """The comparator object of bench.py's JSON line for inputs x."""
    import torch

    w = x.w
    dev = torch.device("cuda", 0)
    if w.dtype == "bf16":
        q, k, v, do = (torch.from_numpy(getattr(x, n + "_bits").view(np.int16)).view(torch.bfloat16).to(dev)
                       for n in ("q", "k", "v", "do"))
    else:
        q, k, v, do = (torch.from_numpy(getattr(x, n)).to(dev) for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    r = bench_composed(q, k, v, do, w.sm_scale, w.causal, steps, warmup)
    flop = w.fwd_flop + w.bwd_flop
    ms = r["fwd_ms"] + r["bwd_ms"]
    return {
        "kind": "composed attention (library GEMMs, HIP causal-softmax kernel, [B,H,S,S] probabilities kept "
                "for the backward)",
        "fwd_ms": round(r["fwd_ms"], 3), "bwd_ms": round(r["bwd_ms"], 3), "ms_per_step": round(ms, 3),
        "value": round(flop / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "note": "same algorithmic flop count as the fused op; the composed path computes all S*S products",
        "speedup_fused": round(ms / fused_ms_step, 2),
        "peak_mib_composed": round(r["peak_bytes"] / 2**20, 1),
        "peak_mib_fused": round(r["fused_peak_bytes"] / 2**20, 1),
        "seconds": round(time.perf_counter() - t0, 1),
    }
