"""Seeded synthetic inputs for the ternary BitLinear path.

This module only draws numbers: shapes, distributions and seeds of the five
benchmark workloads plus a generic random case for tests.  It holds none of the
method's arithmetic (no quantisation, no packing, no accumulation), so the CPU
oracle under ``oracle/`` and the HIP library can both be fed from it without
sharing any code with each other.

Seeding: NumPy PCG64 through ``SeedSequence([workload_id, role])`` for weights,
scales and outlier channels, and ``SeedSequence([workload_id, role, M])`` for
activations.  Weights are therefore identical across an M sweep.

bf16 inputs are produced by rounding fp32 N(0,1) draws to the nearest bf16
(ties to even) and are returned as raw uint16 bit patterns.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

# roles (second element of the seed sequence)
ROLE_W = 0
ROLE_BETA = 1
ROLE_X = 2
ROLE_OUTLIER = 3
ROLE_W_GATE = 10
ROLE_W_UP = 11
ROLE_W_DOWN = 12
ROLE_BETA_GATE = 20
ROLE_BETA_UP = 21
ROLE_BETA_DOWN = 22

# ternary distributions as lookup tables over a uniform integer draw:
# every entry is equally likely, so the table fixes P(-1), P(0), P(+1)
TERNARY_UNIFORM = (-1, 0, 1)            # 1/3 each
TERNARY_HALF_ZERO = (0, 0, -1, 1)       # P(0)=0.5, P(+-1)=0.25
TERNARY_SPARSE60 = (0, 0, 0, -1, 1)     # P(0)=0.6, P(+-1)=0.2


@dataclass(frozen=True)
class Workload:
    """One benchmark workload: shapes, distributions and the M sweep."""

    wid: int
    name: str
    ms: Sequence[int]
    K: int
    N: int
    table: Sequence[int]
    beta: Optional[float]            # fixed fp32 beta, or None -> U(lo, hi)
    beta_range: Optional[tuple] = None
    act: str = "normal_f32"          # normal_f32 | normal_bf16 | student_t3_outliers
    rms: bool = False
    rms_eps: float = 1e-6
    glu_f: int = 0                   # hidden width of the GLU (0 = plain layer)
    extra: Dict[str, float] = field(default_factory=dict)


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "gemv_k2048_n2048", (1,), 2048, 2048, TERNARY_UNIFORM, 0.02),
    2: Workload(2, "decode_ffn_up_k4096_n11008", (1, 4, 16), 4096, 11008,
                TERNARY_HALF_ZERO, None, beta_range=(0.01, 0.05)),
    3: Workload(3, "prefill_m2048_k4096_n11008", (2048,), 4096, 11008,
                TERNARY_UNIFORM, 0.02, act="normal_bf16"),
    4: Workload(4, "glu_d2560_f6912", (1, 512), 2560, 6912, TERNARY_UNIFORM,
                0.02, rms=True, rms_eps=1e-6, glu_f=6912),
    5: Workload(5, "sweep_k8192_n28672", (1, 8, 64, 512), 8192, 28672,
                TERNARY_SPARSE60, 0.02, act="student_t3_outliers",
                extra={"outlier_frac": 0.001, "outlier_scale": 50.0}),
}


def rng_for(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def ternary(rng: np.random.Generator, N: int, K: int,
            table: Sequence[int] = TERNARY_UNIFORM) -> np.ndarray:
    """int8 [N][K] with entries drawn uniformly from ``table``."""
    lut = np.asarray(table, dtype=np.int8)
    out = np.empty((N, K), dtype=np.int8)
    rows = max(1, (1 << 24) // max(K, 1))          # draw in ~16 MB slabs
    for r0 in range(0, N, rows):
        r1 = min(N, r0 + rows)
        idx = rng.integers(0, len(lut), size=(r1 - r0, K), dtype=np.uint8)
        out[r0:r1] = lut[idx]
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (input preparation only)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def workload_weights(wid: int, role: int = ROLE_W, N: Optional[int] = None,
                     K: Optional[int] = None) -> np.ndarray:
    w = WORKLOADS[wid]
    return ternary(rng_for(wid, role), N if N is not None else w.N,
                   K if K is not None else w.K, w.table)


def workload_beta(wid: int, role: int = ROLE_BETA) -> np.float32:
    w = WORKLOADS[wid]
    if w.beta is not None:
        return np.float32(w.beta)
    lo, hi = w.beta_range
    return np.float32(rng_for(wid, role).uniform(lo, hi))


def outlier_channels(wid: int, K: int) -> np.ndarray:
    w = WORKLOADS[wid]
    n = int(round(w.extra["outlier_frac"] * K))
    return np.sort(rng_for(wid, ROLE_OUTLIER).choice(K, size=n, replace=False))


def workload_activations(wid: int, M: int, K: Optional[int] = None) -> np.ndarray:
    """Activations of workload ``wid`` at ``M`` tokens.

    fp32 [M][K] for the fp32 workloads; uint16 bf16 bits [M][K] for the bf16
    workload.
    """
    w = WORKLOADS[wid]
    K = K if K is not None else w.K
    rng = rng_for(wid, ROLE_X, M)
    if w.act == "normal_f32":
        return rng.standard_normal((M, K), dtype=np.float32)
    if w.act == "normal_bf16":
        return f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    if w.act == "student_t3_outliers":
        x = rng.standard_t(3, size=(M, K))
        x[:, outlier_channels(wid, K)] *= w.extra["outlier_scale"]
        return x.astype(np.float32)
    raise ValueError(w.act)


def glu_weights(wid: int = 4):
    """(w_gate [F][D], w_up [F][D], w_down [D][F]) of the GLU workload."""
    w = WORKLOADS[wid]
    D, F = w.K, w.glu_f
    return (ternary(rng_for(wid, ROLE_W_GATE), F, D, w.table),
            ternary(rng_for(wid, ROLE_W_UP), F, D, w.table),
            ternary(rng_for(wid, ROLE_W_DOWN), D, F, w.table))


def glu_betas(wid: int = 4):
    w = WORKLOADS[wid]
    return tuple(np.float32(w.beta) for _ in range(3))


def random_case(seed: int, M: int, N: int, K: int,
                table: Sequence[int] = TERNARY_UNIFORM, act: str = "normal_f32"):
    """Generic seeded case for tests: (x, w, beta)."""
    rng = rng_for(9000, seed, M, N, K)
    w = ternary(rng, N, K, table)
    beta = np.float32(rng.uniform(0.01, 0.05))
    if act == "normal_f32":
        x = rng.standard_normal((M, K), dtype=np.float32)
    elif act == "student_t3":
        x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    elif act == "normal_bf16":
        x = f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    else:
        raise ValueError(act)
    return x, w, beta


def workload_list() -> List[Workload]:
    return [WORKLOADS[i] for i in sorted(WORKLOADS)]
