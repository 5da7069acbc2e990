"""Compile libxfa.so (gfx950) in-tree with hipcc.

    python -m transformer_attention_xfa_amd.build

Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` at the
repository root and the objects are linked into
``transformer_attention_xfa_amd/libxfa.so``.  It always recompiles.
``build_comparator()`` compiles the benchmark comparator's softmax kernel
(``comparator_kernels/``) into ``comparator_kernels/libcomposed.so``, a
library of its own: it is not part of the attention path.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libxfa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# Per-file additions.  The backward key kernel keeps dK and dV of its keys in
# registers for the whole sweep and needs more than the 256 architectural
# VGPRs; left to its heuristics the compiler then puts every matrix-core
# result in accumulation registers and copies each score tile out with
# v_accvgpr_read before the vector math (32 copies per 32-query block).
# Asking for matrix-core results in VGPRs keeps the score tiles there and
# uses the accumulation registers for other values: no copies in the loop,
# about 3 % less time for the key kernel on the [8, 16, 4096, 128] bf16 case.
FILE_FLAGS = {
    "xfa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC, "-c", src,
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


COMPARATOR_DIR = os.path.join(ROOT, "comparator_kernels")
COMPARATOR_LIB = os.path.join(COMPARATOR_DIR, "libcomposed.so")


def build_comparator(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(COMPARATOR_DIR, "*.hip")))
    tmp = COMPARATOR_LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-shared", "-o", tmp, *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on the comparator kernels:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, COMPARATOR_LIB)
    if verbose:
        print("built", COMPARATOR_LIB, file=sys.stderr)
    return COMPARATOR_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_comparator(verbose=True)
