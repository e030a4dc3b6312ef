"""Seeded synthetic inputs for the scaled FP8 GEMM workloads.

This module is shared by the CPU oracle, the tests and the benchmark.  It only
draws random fp32 operands and expert row counts; it holds none of the method's
arithmetic (no amax, scaling, rounding or matrix products).

Every workload is drawn with ``numpy.random.default_rng(seed)`` (PCG64).  Draw
order is fixed: operand A first, then operand B (dense), or expert counts, then
activations, then the expert weights one expert at a time (grouped).  B is
always returned as ``[N, K]`` float32: N rows of K contiguous values, which is the
column-major ``[K, N]`` operand the GEMM consumes.

The five workloads follow the FP8 GEMM shapes the pages discuss: a small
per-tensor case, the M=128 / N=K=4096 decode-like shape whose memory throughput
is tabulated in "Hopper/Blackwell architecture features" §12.2.4, row-wise
scaling with outliers (the FP8 row-wise GEMM of §12.3.4), a 32-element
microscaled (MXFP8) case (§12.6.1 table, "2nd-gen Transformer Engine" row) and
the mixture-of-experts grouped form of the JAX/Triton Blackwell FP8 GEMM post.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "normal", "with_outliers", "block_scaled_normal",
    "dense_inputs", "grouped_counts", "grouped_inputs", "random_inputs",
]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int          # rows of A (grouped: total rows over all experts)
    N: int
    K: int
    mode: str       # "tensor" | "rowwise" | "mx32"
    out: str        # "f16" | "bf16"
    seed: int
    dist: str       # "normal" | "outlier" | "mx_block"
    groups: int = 0  # >0: grouped (MoE) workload with this many experts
    weight_std: float = 1.0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    "pertensor256": Workload("pertensor256", 256, 256, 256, "tensor", "f16", 1, "normal"),
    "skinny128": Workload("skinny128", 128, 4096, 4096, "tensor", "bf16", 2, "normal"),
    "rowwise4096": Workload("rowwise4096", 4096, 4096, 4096, "rowwise", "bf16", 3, "outlier"),
    "mx8192": Workload("mx8192", 8192, 8192, 8192, "mx32", "bf16", 4, "mx_block"),
    "grouped_moe": Workload("grouped_moe", 16384, 14336, 4096, "rowwise", "bf16", 5, "normal",
                            groups=8, weight_std=0.02),
}


def normal(rng: np.random.Generator, rows: int, k: int, std: float = 1.0) -> np.ndarray:
    """rows x k float32 draws from N(0, std^2)."""
    x = rng.standard_normal((rows, k), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def with_outliers(rng: np.random.Generator, rows: int, k: int, p: float = 0.01,
                  factor: float = 20.0) -> np.ndarray:
    """N(0,1) with each entry independently multiplied by ``factor`` with probability p."""
    x = rng.standard_normal((rows, k), dtype=np.float32)
    mask = rng.random((rows, k), dtype=np.float32) < np.float32(p)
    x[mask] *= np.float32(factor)
    return x


def block_scaled_normal(rng: np.random.Generator, rows: int, k: int, block: int = 32,
                        lo: float = 0.1, hi: float = 10.0) -> np.ndarray:
    """N(0,1) times one U(lo, hi) multiplier per (row, ``block`` contiguous K) block."""
    if k % block:
        raise ValueError("k must be a multiple of the block length")
    x = rng.standard_normal((rows, k), dtype=np.float32)
    u = rng.uniform(lo, hi, size=(rows, k // block)).astype(np.float32)
    x.reshape(rows, k // block, block)[...] *= u[:, :, None]
    return x


_DISTS = {"normal": normal, "outlier": with_outliers, "mx_block": block_scaled_normal}


def random_inputs(M: int, N: int, K: int, seed: int, dist: str = "normal"):
    """A [M,K] and B [N,K] float32 with the named distribution (A drawn first)."""
    rng = np.random.default_rng(seed)
    gen = _DISTS[dist]
    A = gen(rng, M, K)
    B = gen(rng, N, K)
    return A, B


def dense_inputs(w: Workload):
    """The A [M,K] and B [N,K] operands of a dense workload."""
    if w.groups:
        raise ValueError("grouped workload: use grouped_inputs")
    return random_inputs(w.M, w.N, w.K, w.seed, w.dist)


def grouped_counts(rng: np.random.Generator, total: int, groups: int) -> np.ndarray:
    """Rows per expert ~ Multinomial(total, uniform over experts)."""
    return rng.multinomial(total, [1.0 / groups] * groups).astype(np.int64)


def grouped_inputs(w: Workload, experts: tuple | None = None):
    """counts [G] int64, A [M,K] float32 (rows sorted by expert), W [G,N,K] float32.

    With ``experts`` given, W holds only those experts' weights (in that order);
    the draws of the other experts are still consumed so values do not depend on
    the selection.
    """
    if not w.groups:
        raise ValueError("dense workload: use dense_inputs")
    rng = np.random.default_rng(w.seed)
    counts = grouped_counts(rng, w.M, w.groups)
    A = normal(rng, w.M, w.K)
    keep = list(range(w.groups)) if experts is None else list(experts)
    W = np.empty((len(keep), w.N, w.K), dtype=np.float32)
    for g in range(w.groups):
        wg = normal(rng, w.N, w.K, w.weight_std)
        for slot, e in enumerate(keep):
            if e == g:
                W[slot] = wg
    return counts, A, W
