"""Named attention workloads and their seeded synthetic inputs.

This module holds no attention arithmetic. It only fixes the workload shapes
and draws the inputs, so that the GPU path and the CPU oracle receive exactly
the same values. Both sides import it; neither imports the other.

Input recipe (the same for every workload):
  * ``rng = numpy.random.default_rng(seed)``;
  * Q, K, V, dO are drawn in that order as float32 standard normals of shape
    ``[B, H, S, hd]``, each multiplied by its standard deviation;
  * for bf16 workloads each value is rounded to bfloat16 (round to nearest,
    ties to even) and both sides use the rounded values: the GPU as raw bf16
    bits, the oracle upcast to float64.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32" or "bf16": storage type of Q, K, V, O, dO, dQ, dK, dV
    B: int
    H: int
    S: int
    hd: int
    seed: int
    q_std: float = 1.0
    k_std: float = 1.0
    v_std: float = 1.0
    do_std: float = 1.0
    causal: bool = True
    scale: float | None = None  # None: 1/sqrt(hd)

    @property
    def BH(self) -> int:
        return self.B * self.H

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.hd) if self.scale is None else float(self.scale)

    @property
    def shape(self) -> tuple[int, int, int, int]:
        return (self.B, self.H, self.S, self.hd)

    @property
    def pairs_per_head(self) -> int:
        """Unmasked (query, key) pairs of one head."""
        return self.S * (self.S + 1) // 2 if self.causal else self.S * self.S

    @property
    def fwd_flop(self) -> float:
        """Algorithmic forward work: Q.K^T and P.V, 2*hd flop each per pair."""
        return 4.0 * self.hd * self.pairs_per_head * self.BH

    @property
    def bwd_flop(self) -> float:
        """Algorithmic backward work: recomputed Q.K^T, dO.V^T, P^T.dO, dS.K,
        dS^T.Q, 2*hd flop each per pair."""
        return 10.0 * self.hd * self.pairs_per_head * self.BH

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the method is checked and measured on.  C4 is the
# throughput workload; C1 is the smallest one.
C1 = Workload("c1_f32_s64_hd16", "f32", 1, 1, 64, 16, seed=0)
C2 = Workload("c2_f32_s256_hd64", "f32", 2, 4, 256, 64, seed=1)
C3 = Workload("c3_bf16_s1024_hd64", "bf16", 4, 8, 1024, 64, seed=2, do_std=0.1)
C4 = Workload("c4_bf16_s4096_hd128", "bf16", 8, 16, 4096, 128, seed=3, do_std=0.1)
C5 = Workload("c5_bf16_s16384_hd128", "bf16", 1, 32, 16384, 128, seed=4,
              q_std=1.5, k_std=1.5, do_std=0.1)
CONFIGS = (C1, C2, C3, C4, C5)

# Attention shapes of the page's dim768 model (12 heads x 64) at its two
# measured batch/sequence settings, with C3's value distributions.
PA = Workload("pa_bf16_b8_s1024_hd64", "bf16", 8, 12, 1024, 64, seed=5, do_std=0.1)
PB = Workload("pb_bf16_b2_s2048_hd64", "bf16", 2, 12, 2048, 64, seed=6, do_std=0.1)
PAGE_SHAPES = (PA, PB)

BY_NAME = {w.name: w for w in CONFIGS + PAGE_SHAPES}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs here are finite Gaussians, so NaN handling is not needed; an
    infinite or NaN input raises.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_bf16_bits expects finite values")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """One workload's inputs.

    ``q, k, v, do`` are float32 arrays holding the exact stored values (for
    bf16 workloads: the bf16-rounded values).  ``*_bits`` hold the raw bf16
    patterns for bf16 workloads and are None for f32 workloads.
    """
    w: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    do_bits: np.ndarray | None = None

    def f64(self, name: str, bh: int | None = None) -> np.ndarray:
        """A tensor (or one head of it, ``[S, hd]``) as float64 for the oracle."""
        a = getattr(self, name)
        if bh is not None:
            a = a.reshape(self.w.BH, self.w.S, self.w.hd)[bh]
        return a.astype(np.float64)


def make_inputs(w: Workload) -> Inputs:
    rng = np.random.default_rng(w.seed)
    arrs = []
    for std in (w.q_std, w.k_std, w.v_std, w.do_std):
        a = rng.standard_normal(w.shape, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        arrs.append(a)
    if w.dtype == "f32":
        return Inputs(w, *arrs)
    if w.dtype != "bf16":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    bits = [round_to_bf16_bits(a) for a in arrs]
    vals = [bf16_bits_to_f32(b) for b in bits]
    return Inputs(w, *vals, *bits)
