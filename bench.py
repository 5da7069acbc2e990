"""Throughput of the fused causal attention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--comparator]
                    [--dropout P] [--graph] [--autograd] [--dq-atomic-floor]

One step is one pass of the whole path over one batch: xfa_fwd, then
xfa_bwd_preprocess, then xfa_bwd, with inputs resident in HBM.  The default
workload is causal bf16 attention, B=8, H=16, S=4096, hd=128.  The printed
JSON line carries the whole-step throughput in algorithmic TFLOP/s (only
unmasked query/key pairs count: 4*hd flop per pair forward, 10*hd backward),
each kernel's average duration from HIP events recorded on the stream the
kernels run on, the roofline of the dominant kernel, and the CPU oracle timed
on a bounded sample of the same workload.  --comparator adds composed
attention (comparator.py) on the same inputs: its time and both paths' peak
memory.  --dropout P adds the same step with dropout on the attention
probabilities (xfa_fwd_dropout / xfa_bwd_dropout) and its cost over the plain
step; the headline value is always the plain step.  --graph adds the step
captured once in a HIP graph and replayed (the same kernels, without the
per-launch host overhead that dominates the small workloads).  --autograd
adds the differentiable op (flash_attention, forward then backward through
torch autograd) in its native mode and in the fp32-core mode (bf16 tensors
cast at the boundary, the fp32 kernels inside).  --dq-atomic-floor adds the
time of the fp32 atomic adds alone that summing dQ across key workgroups
would take (comparator_kernels/dq_atomic_floor.hip), beside the backward.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "causal attention fwd+bwd TFLOP/s at 1 MI355X (and % of MFMA peak)"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = {
    "bwd": "transformer_attention_xfa_amd/csrc/xfa_bwd.hip",
    "fwd": "transformer_attention_xfa_amd/csrc/xfa_fwd.hip",
    "pre": "transformer_attention_xfa_amd/csrc/xfa_pre.hip",
}
KERNEL_NAME = {"fwd": "fwd_kernel", "pre": "bwd_pre_kernel", "bwd": "bwd_key_kernel + bwd_query_kernel"}


def source_digest(phase: str) -> str:
    h = hashlib.sha256()
    for rel in (KERNEL_SRC[phase], "transformer_attention_xfa_amd/csrc/xfa_common.h",
                "transformer_attention_xfa_amd/csrc/xfa_stage.h", "transformer_attention_xfa_amd/build.py"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(phase: str, w) -> float | None:
    """HBM bytes per launch from the committed counter runs, if they were
    taken on the current kernel source and this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(phase)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != source_digest(phase) or rec.get("workload") != w.name:
        return None
    return float(rec["hbm_bytes_per_launch"])


PHASE_KERNELS = {"fwd": ("fwd_kernel",), "pre": ("bwd_pre_kernel",), "bwd": ("bwd_key_kernel", "bwd_query_kernel")}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 2 ** 30     # what --copy-calibration copies per dispatch


def _counter_means(path: str) -> dict:
    """Mean Counter_Value per kernel (by the kernel's unqualified name) of a
    rocprofv3 --pmc csv with one counter."""
    import csv

    acc = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            for base in [k for ks in PHASE_KERNELS.values() for k in ks] + [COPY_KERNEL]:
                if base in name:
                    acc.setdefault(base, []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def ingest_pmc(fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str, workload: str) -> dict:
    """profiles/traffic.json from two counter runs of bench.py (FETCH_SIZE,
    WRITE_SIZE) and the same two counters over --copy-calibration: each
    counter is scaled by the bytes a 1 GiB copy moves per unit of it, per
    launch, and stamped with the digest of the sources it was taken on."""
    fetch, write = _counter_means(fetch_csv), _counter_means(write_csv)
    cf, cw = _counter_means(copy_fetch_csv)[COPY_KERNEL], _counter_means(copy_write_csv)[COPY_KERNEL]
    ff, fw = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    out = {"_note": "HBM bytes per launch on the named workload, from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
                    "(KiB per dispatch, mean over the dispatches of each kernel), scaled by what a 1 GiB "
                    "device-to-device copy (bench.py --copy-calibration) reads and writes on the same counters; "
                    "the bwd phase is its two kernels' sum.  Written by bench.py --ingest-pmc.",
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                           "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)}}
    for phase, kernels in PHASE_KERNELS.items():
        if not all(k in fetch and k in write for k in kernels):
            continue
        rd = sum(fetch[k] for k in kernels) * 1024 * ff
        wr = sum(write[k] for k in kernels) * 1024 * fw
        out[phase] = {"kernels": {k: {"fetch_kib": fetch[k], "write_kib": write[k]} for k in kernels},
                      "workload": workload, "source_digest": source_digest(phase),
                      "read_bytes": round(rd), "write_bytes": round(wr), "hbm_bytes_per_launch": round(rd + wr)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def gpu_bench(x, steps: int, warmup: int, dropout_p: float = 0.0, seed: int = 0x5EED):
    import torch

    import transformer_attention_xfa_amd as xfa

    w = x.w
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if w.dtype == "bf16":
        q, k, v, do = (torch.from_numpy(getattr(x, n + "_bits").view(np.int16)).view(torch.bfloat16).to(dev)
                       for n in ("q", "k", "v", "do"))
    else:
        q, k, v, do = (torch.from_numpy(getattr(x, n)).to(dev) for n in ("q", "k", "v", "do"))
    B, H, S, hd = w.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    scale, causal = w.sm_scale, w.causal
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if dropout_p:
            xfa.xfa_fwd_dropout(q, k, v, out, lse, scale, causal, dropout_p, seed, stream)
        else:
            xfa.xfa_fwd(q, k, v, out, lse, scale, causal, stream)
        if ev is not None:
            ev[1].record(stream)
        xfa.xfa_bwd_preprocess(out, do, delta, scale, causal, stream)
        if ev is not None:
            ev[2].record(stream)
        if dropout_p:
            xfa.xfa_bwd_dropout(q, k, v, do, lse, delta, dq, dk, dv, scale, causal, dropout_p, seed, stream)
        else:
            xfa.xfa_bwd(q, k, v, do, lse, delta, dq, dk, dv, scale, causal, stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = {"fwd": [], "pre": [], "bwd": []}
    for ev in events:
        ms["fwd"].append(ev[0].elapsed_time(ev[1]))
        ms["pre"].append(ev[1].elapsed_time(ev[2]))
        ms["bwd"].append(ev[2].elapsed_time(ev[3]))
    assert torch.isfinite(out).all() and torch.isfinite(dq).all(), "non-finite output"
    name = torch.cuda.get_device_name(dev)
    stats = {"mean": {p: float(np.mean(v)) for p, v in ms.items()},
             "median": {p: float(np.median(v)) for p, v in ms.items()},
             "min": {p: float(np.min(v)) for p, v in ms.items()}}
    return (t1 - t0) * 1e3 / steps, stats, name


def graph_bench(x, steps: int, warmup: int):
    """ms per step of the plain step captured in one HIP graph and replayed."""
    import torch

    import transformer_attention_xfa_amd as xfa

    w = x.w
    dev = torch.device("cuda", 0)
    if w.dtype == "bf16":
        q, k, v, do = (torch.from_numpy(getattr(x, n + "_bits").view(np.int16)).view(torch.bfloat16).to(dev)
                       for n in ("q", "k", "v", "do"))
    else:
        q, k, v, do = (torch.from_numpy(getattr(x, n)).to(dev) for n in ("q", "k", "v", "do"))
    B, H, S, hd = w.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)

    def step():
        xfa.xfa_fwd(q, k, v, out, lse, w.sm_scale, w.causal)
        xfa.xfa_bwd_preprocess(out, do, delta, w.sm_scale, w.causal)
        xfa.xfa_bwd(q, k, v, do, lse, delta, dq, dk, dv, w.sm_scale, w.causal)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def autograd_bench(x, steps: int, warmup: int, core: str):
    """Mean fwd and bwd ms of flash_attention(...).backward() on x, for one core mode."""
    import torch

    import transformer_attention_xfa_amd as xfa

    w = x.w
    dev = torch.device("cuda", 0)
    if w.dtype == "bf16":
        q, k, v, do = (torch.from_numpy(getattr(x, n + "_bits").view(np.int16)).view(torch.bfloat16).to(dev)
                       for n in ("q", "k", "v", "do"))
    else:
        q, k, v, do = (torch.from_numpy(getattr(x, n)).to(dev) for n in ("q", "k", "v", "do"))
    q, k, v = (t.requires_grad_(True) for t in (q, k, v))
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        out = xfa.flash_attention(q, k, v, w.sm_scale, w.causal, core=core)
        if ev is not None:
            ev[1].record(stream)
        out.backward(do)
        if ev is not None:
            ev[2].record(stream)
        q.grad = k.grad = v.grad = None

    for _ in range(warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    flop = w.fwd_flop + w.bwd_flop
    return {"fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4), "ms_per_step": round(fwd + bwd, 4),
            "value": round(flop / ((fwd + bwd) * 1e-3) / 1e12, 2), "unit": "TFLOP/s"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


# The host share of one GPU on the measurement machines: worker pools stay
# within it whatever the affinity mask shows.
HOST_WORKERS_MAX = 16
_BLAS_ENV = ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS")


def _oracle_job(job):
    """One head of the oracle in a pool worker: (phase, q, k, v, do, scale, causal) -> seconds."""
    from oracle import attention_backward_head, attention_forward_head

    phase, q, k, v, do, scale, causal = job
    t0 = time.perf_counter()
    if phase == "fwd":
        attention_forward_head(q, k, v, scale, causal, row_block=1024)
    else:
        attention_backward_head(q, k, v, do, scale, causal, row_block=1024)
    return time.perf_counter() - t0


def _oracle_ready(_):
    import oracle  # noqa: F401  (imports done before the timed maps)
    time.sleep(0.25)   # long enough that every worker takes one of these
    return os.getpid()


def cpu_baseline(x, n_heads: int):
    """The oracle, untuned, on the first n_heads heads of the workload, one
    head per task in a pool of single-threaded worker processes (one per
    available host core, at most HOST_WORKERS_MAX); the forward of all
    sampled heads, then their backward, each timed as wall time around the
    pool's map.  Workers are started fresh (spawn) with one BLAS thread; a
    worker that dies breaks the pool with an error instead of a hang."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    w = x.w
    n_heads = max(1, min(n_heads, w.BH))
    workers = max(1, min(len(os.sched_getaffinity(0)), HOST_WORKERS_MAX, n_heads))
    heads = [[x.f64(n, h) for n in ("q", "k", "v", "do")] for h in range(n_heads)]
    saved = {k: os.environ.get(k) for k in _BLAS_ENV}
    os.environ.update({k: "1" for k in _BLAS_ENV})   # inherited by the spawned workers
    try:
        with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as pool:
            pids = set(pool.map(_oracle_ready, range(workers), timeout=300))
            wall = {}
            busy = {}
            for phase in ("fwd", "bwd"):
                jobs = [(phase, q, k, v, do, w.sm_scale, w.causal) for q, k, v, do in heads]
                t0 = time.perf_counter()
                per_head = list(pool.map(_oracle_job, jobs, timeout=900))
                wall[phase] = time.perf_counter() - t0
                busy[phase] = float(sum(per_head))
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    t_fwd, t_bwd = wall["fwd"], wall["bwd"]
    dt = t_fwd + t_bwd
    frac = n_heads / w.BH
    flop = (w.fwd_flop + w.bwd_flop) * frac
    return {
        "value": round(flop / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{n_heads} of {w.BH} heads of {w.name}, forward then backward, float64 NumPy composed "
                  f"attention (it computes all S*S products; the rate uses the same algorithmic flop count "
                  f"as the GPU), one head per task on a pool of {workers} single-threaded worker processes "
                  f"({len(pids)} started), wall time {dt:.1f} s on {_cpu_model()}",
        "seconds": round(dt, 2),
        "fwd_seconds": round(t_fwd, 2),
        "bwd_seconds": round(t_bwd, 2),
        "fwd_tflops": round(w.fwd_flop * frac / t_fwd / 1e12, 6),
        "bwd_tflops": round(w.bwd_flop * frac / t_bwd / 1e12, 6),
        "worker_busy_seconds": round(busy["fwd"] + busy["bwd"], 2),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=workloads.C4.name, choices=sorted(workloads.BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=128,
                    help="heads of the workload the CPU oracle runs (default 128: all of C4's)")
    ap.add_argument("--comparator", action="store_true",
                    help="also time composed attention (library GEMMs + softmax) and both paths' peak memory")
    ap.add_argument("--autograd", action="store_true",
                    help="also time flash_attention forward + backward through autograd, native and fp32-core modes")
    ap.add_argument("--graph", action="store_true",
                    help="also time the plain step captured in a HIP graph and replayed")
    ap.add_argument("--dq-atomic-floor", action="store_true",
                    help="also time the fp32 atomic traffic alone that summing dQ across key workgroups "
                         "would need (the alternative to the separate dQ kernel)")
    ap.add_argument("--ingest-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 --pmc csv files of bench.py (FETCH_SIZE, "
                         "WRITE_SIZE, on --workload) and of --copy-calibration (same counters), then exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three 1 GiB device-to-device copies (the reference kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    ap.add_argument("--dropout", type=float, default=0.0, metavar="P",
                    help="also time the step with dropout probability P on the attention probabilities")
    args = ap.parse_args(argv)
    if not 0.0 <= args.dropout < 1.0:
        ap.error("--dropout must be in [0, 1)")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the attention path is independent per head, and "
              "sharding heads across GPUs needs no communication, so run it with --gpus 1.",
              file=sys.stderr)
        return 2

    if args.ingest_pmc:
        print(json.dumps(ingest_pmc(*args.ingest_pmc, workload=args.workload)), flush=True)
        return 0
    if args.copy_calibration:
        import torch
        a = torch.ones(2 ** 28, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": a.numel() * 4, "copies": 3}), flush=True)
        return 0
    w = workloads.BY_NAME[args.workload]
    x = workloads.make_inputs(w)
    # the oracle's worker pool runs before this process touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(x, args.cpu_heads)
    ms_step, stats, device = gpu_bench(x, args.steps, args.warmup)
    ms_mean, ms_med, ms_min = stats["mean"], stats["median"], stats["min"]
    flop = w.fwd_flop + w.bwd_flop
    value = flop / (ms_step * 1e-3) / 1e12

    # the dominant kernel: the one with the longest average duration
    phase_flop = {"fwd": w.fwd_flop, "bwd": w.bwd_flop}
    dom = max(("fwd", "bwd"), key=lambda p: ms_mean[p])
    achieved = phase_flop[dom] / (ms_mean[dom] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    roofline = {
        "bound": "mfma", "kernel": KERNEL_NAME[dom], "achieved": round(achieved, 2), "peak": peak,
        "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
        "traffic": measured_traffic(dom, w),
        "avg_launch_ms": round(ms_mean[dom], 4),
    }
    el = 2 if w.dtype == "bf16" else 4
    pre_bytes = w.BH * w.S * (2 * w.hd * el + 4)   # read O, dO; write D
    phases = {
        "fwd": {"kernel": KERNEL_NAME["fwd"], "avg_ms": round(ms_mean["fwd"], 4), "median_ms": round(ms_med["fwd"], 4),
                "min_ms": round(ms_min["fwd"], 4), "tflops": round(w.fwd_flop / (ms_mean["fwd"] * 1e-3) / 1e12, 2)},
        "bwd_preprocess": {"kernel": KERNEL_NAME["pre"], "avg_ms": round(ms_mean["pre"], 4),
                           "median_ms": round(ms_med["pre"], 4), "min_ms": round(ms_min["pre"], 4),
                           "gbs": round(pre_bytes / (ms_mean["pre"] * 1e-3) / 1e9, 1),
                           "frac_hbm": round(pre_bytes / (ms_mean["pre"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "bwd": {"kernel": KERNEL_NAME["bwd"], "avg_ms": round(ms_mean["bwd"], 4), "median_ms": round(ms_med["bwd"], 4),
                "min_ms": round(ms_min["bwd"], 4), "tflops": round(w.bwd_flop / (ms_mean["bwd"] * 1e-3) / 1e12, 2)},
    }
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "hd": w.hd, "causal": w.causal,
                   "scale": w.sm_scale, "global_batch": w.B, "seq_len": w.S, "parallelism": "none"},
        "frac_of_peak": round(value / PEAK_TFLOPS[w.dtype], 4),
        "roofline": roofline,
        "phases": phases,
        "device": device,
    }
    if args.autograd:
        nat = autograd_bench(x, args.steps, args.warmup, "native")
        f32 = autograd_bench(x, args.steps, args.warmup, "fp32")
        f32["frac_of_fp32_peak"] = round(f32["value"] / PEAK_TFLOPS["f32"], 4)
        rec["autograd"] = {
            "op": "flash_attention(q, k, v).backward(dout), events around forward and backward",
            "native": nat,
            "fp32_core": dict(f32, note="bf16 tensors cast to fp32 at the boundary, fp32 kernels inside, "
                                        "results cast back; the rate uses the same algorithmic flops"),
        }
    if args.graph:
        g_ms = graph_bench(x, args.steps, args.warmup)
        rec["graph"] = {"ms_per_step": round(g_ms, 4), "value": round(flop / (g_ms * 1e-3) / 1e12, 2),
                        "unit": "TFLOP/s", "note": "the same step captured once in a HIP graph and replayed"}
    if args.dropout:
        d_step, d_stats, _ = gpu_bench(x, args.steps, args.warmup, dropout_p=args.dropout)
        d_mean = d_stats["mean"]
        rec["dropout"] = {
            "p": args.dropout, "kernels": "fwd_kernel, bwd_key_kernel + bwd_query_kernel with in-kernel keep bits",
            "ms_per_step": round(d_step, 4), "fwd_ms": round(d_mean["fwd"], 4), "bwd_ms": round(d_mean["bwd"], 4),
            "value": round(flop / (d_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "step_cost_vs_plain": round(d_step / ms_step, 3),
            "fwd_cost_vs_plain": round(d_mean["fwd"] / ms_mean["fwd"], 3),
            "bwd_cost_vs_plain": round(d_mean["bwd"] / ms_mean["bwd"], 3),
        }
    if args.dq_atomic_floor:
        import comparator
        rec["dq_atomic_floor"] = comparator.dq_atomic_floor_record(w, args.steps, ms_mean["bwd"])
    if args.comparator:
        import comparator
        rec["comparator"] = comparator.comparator_record(x, max(1, args.steps // 4), 1, ms_step)
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
