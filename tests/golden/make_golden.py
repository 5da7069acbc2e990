"""Writes tests/golden/c1_oracle.json: the smallest workload's input digests
and oracle outputs at sampled positions.

It calls only the oracle and the input generator.  The stored values freeze
the input recipe and the oracle's results so that a silent change to either
shows up as a failing CPU test; they are not a pin of the oracle by
themselves (the pins are in tests/test_oracle_pins.py).

Run from the repository root:  python tests/golden/make_golden.py
"""

import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402
from oracle import attention_backward_head, attention_forward_head  # noqa: E402

SAMPLES = [(0, 0), (1, 3), (17, 5), (31, 15), (32, 0), (63, 7), (63, 15)]


def build():
    w = workloads.C1
    x = workloads.make_inputs(w)
    digests = {n: hashlib.sha256(np.ascontiguousarray(getattr(x, n)).tobytes()).hexdigest()
               for n in ("q", "k", "v", "do")}
    q, k, v, do = (x.f64(n, 0) for n in ("q", "k", "v", "do"))
    out, lse = attention_forward_head(q, k, v, w.sm_scale, True)
    dq, dk, dv, dref = attention_backward_head(q, k, v, do, w.sm_scale, True)
    samp = {}
    for name, a in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        samp[name] = [[i, d, float(a[i, d])] for i, d in SAMPLES]
        samp[name + "_sum"] = float(a.sum())
    samp["lse"] = [[i, float(lse[i])] for i, _ in SAMPLES]
    samp["dref"] = [[i, float(dref[i])] for i, _ in SAMPLES]
    return {"workload": w.name, "input_sha256": digests, "oracle": samp}


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_oracle.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=1)
        f.write("\n")
    print("wrote", path)
