"""The scaled FP8 GEMM reference, its error bound and the grouped (MoE) form.

TEST INFRASTRUCTURE (see the package docstring).

Definition.  With e4m3fn operand codes qa [M,K] and qb [N,K] (B column-major,
stored as its N x K transpose) and their scales, the GEMM is

    C[m,n] = sum_k dq_a[m,k] * dq_b[n,k]

where dq is the dequantised operand: ``s * decode(q)`` per tensor, per row of A
and per column of B (row-wise), or ``2^(code-127) * decode(q)`` per 32-element
K block (MX).  The kernels the pages show accumulate ``tl.dot`` products in an
fp32 ``acc`` and cast it on store (``acc.to(tl.float16)`` in the JAX/Triton
Blackwell FP8 GEMM post's kernel pseudocode; ``acc.to(tl.bfloat16)`` in
"Hopper/Blackwell architecture features" §12.7.1/§12.7.2), so the result is
delivered in fp16 or bf16 after fp32 accumulation.

This reference evaluates the sum in float64.  Every decoded e4m3 value is
i * 2^j with |i| <= 15 and -9 <= j <= 5, so for per-tensor and row-wise scaling
the inner sum sum_k decode*decode is an integer multiple of 2^-18 below 2^50
units and float64 holds it exactly in any summation order; only the final
multiplication by the scales rounds.  For MX each term carries a power-of-two
block factor, which float64 also represents exactly; only the sum across blocks
rounds (relative error near 1e-15 of sum |a*b|).

Acceptance bound (read from the target statement of this GEMM):
    |C - C_ref| <= 1e-3 * sum_k |dq_a[m,k] * dq_b[n,k]| + ulp_out(|C_ref|)
with ulp_out the spacing of the output format (fp16: 11 significant bits,
bf16: 8) at |C_ref|, never below that format's subnormal spacing.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_e4m3, decode_e8m0
from .quant import MX_BLOCK

_OUT_FORMATS = {
    # name: (significand bits incl. hidden, minimum normal exponent, largest finite)
    "f16": (11, -14, 65504.0),
    "bf16": (8, -126, float.fromhex("0x1.fep127")),
}


def dequantize(q: np.ndarray, scale, mode: str) -> np.ndarray:
    """float64 values represented by codes q [R,K] and their scales."""
    v = decode_e4m3(q)
    if mode == "tensor":
        return v * float(np.asarray(scale, dtype=np.float32))
    if mode == "rowwise":
        return v * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]
    if mode == "mx32":
        R, K = v.shape
        f = decode_e8m0(np.asarray(scale, dtype=np.uint8))            # [R, K/32]
        return (v.reshape(R, K // MX_BLOCK, MX_BLOCK) * f[:, :, None]).reshape(R, K)
    raise ValueError(f"unknown scale mode {mode!r}")


def _select(x, idx):
    return x if idx is None else x[np.asarray(idx)]


def gemm_reference(qa, sa, qb, sb, mode: str, rows=None, cols=None):
    """(C_ref, abs_ref) in float64 for the selected rows of A and columns of C.

    qa: uint8 [M,K]; qb: uint8 [N,K] (column-major B).  Scales: "tensor" ->
    float32 scalars; "rowwise" -> float32 [M] and [N]; "mx32" -> uint8 E8M0
    [M,K/32] and [N,K/32].  ``rows``/``cols`` pick a sub-block (default all).
    """
    qa_s = _select(qa, rows)
    qb_s = _select(qb, cols)
    if mode == "tensor":
        da, db = decode_e4m3(qa_s), decode_e4m3(qb_s)
        f = float(np.float32(sa)) * float(np.float32(sb))
        inner = da @ db.T                        # exact: multiples of 2^-18 below 2^50 units
        absin = np.abs(da) @ np.abs(db).T
        return inner * f, absin * abs(f)
    if mode == "rowwise":
        da, db = decode_e4m3(qa_s), decode_e4m3(qb_s)
        fa = _select(np.asarray(sa, np.float32), rows).astype(np.float64)
        fb = _select(np.asarray(sb, np.float32), cols).astype(np.float64)
        inner = da @ db.T
        absin = np.abs(da) @ np.abs(db).T
        outer = fa[:, None] * fb[None, :]
        return inner * outer, absin * np.abs(outer)
    if mode == "mx32":
        da = dequantize(qa_s, _select(sa, rows), "mx32")
        db = dequantize(qb_s, _select(sb, cols), "mx32")
        return da @ db.T, np.abs(da) @ np.abs(db).T
    raise ValueError(f"unknown scale mode {mode!r}")


def grouped_reference(qa, sa, offsets, qb, sb, mode: str, rows=None, cols=None):
    """Grouped GEMM reference: rows [offsets[g], offsets[g+1]) of A use expert g.

    qa: uint8 [total_m, K] sorted by expert; offsets: int [G+1] with
    offsets[0] = 0 and offsets[G] = total_m; qb: uint8 [G, N, K].  Scales:
    "tensor" -> sa float32 scalar, sb float32 [G]; "rowwise" -> sa [total_m],
    sb [G, N]; "mx32" -> sa uint8 [total_m, K/32], sb uint8 [G, N, K/32].
    Returns (C_ref, abs_ref) for the selected rows (default all) and columns.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    total_m = qa.shape[0]
    rows = np.arange(total_m) if rows is None else np.asarray(rows, dtype=np.int64)
    N = qb.shape[1] if cols is None else len(cols)
    C = np.zeros((len(rows), N), dtype=np.float64)
    A = np.zeros((len(rows), N), dtype=np.float64)
    group_of = np.searchsorted(offsets, rows, side="right") - 1
    for g in range(len(offsets) - 1):
        sel = np.nonzero(group_of == g)[0]
        if sel.size == 0:
            continue
        r = rows[sel]
        if mode == "tensor":
            c, a = gemm_reference(qa[r], sa, qb[g], np.asarray(sb)[g], mode, cols=cols)
        else:
            c, a = gemm_reference(qa[r], np.asarray(sa)[r], qb[g], np.asarray(sb)[g], mode,
                                  cols=cols)
        C[sel] = c
        A[sel] = a
    return C, A


def output_ulp(x: np.ndarray, out: str) -> np.ndarray:
    """Spacing of the output format at |x| (subnormal spacing near zero)."""
    p, emin, _ = _OUT_FORMATS[out]
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(a)                       # a = f * 2^ex, floor(log2 a) = ex - 1
    e = np.where(a > 0, ex.astype(np.int64) - 1, emin)
    e = np.maximum(e, emin)
    return np.ldexp(1.0, e - (p - 1))


def tolerance(C_ref: np.ndarray, abs_ref: np.ndarray, out: str) -> np.ndarray:
    """1e-3 * sum_k |a*b| + one output ulp at |C_ref|."""
    return 1e-3 * np.asarray(abs_ref, np.float64) + output_ulp(C_ref, out)


def within_bound(C_test, C_ref, abs_ref, out: str) -> np.ndarray:
    """Boolean mask: which outputs satisfy the acceptance bound."""
    err = np.abs(np.asarray(C_test, np.float64) - np.asarray(C_ref, np.float64))
    return err <= tolerance(C_ref, abs_ref, out)


def round_to_output(x: np.ndarray, out: str) -> np.ndarray:
    """Round-to-nearest-even of float64 values onto the output format (diagnostics).

    Values whose rounding exceeds the largest finite number become +-inf.
    """
    p, emin, fmax = _OUT_FORMATS[out]
    x = np.asarray(x, dtype=np.float64)
    q = output_ulp(x, out)
    r = np.rint(x / q) * q                    # x / q is exact (power of two); rint is RNE
    return np.where(np.abs(r) > fmax, np.copysign(np.inf, x), r)
