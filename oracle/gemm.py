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

Either operand may hold e4m3fn or e5m2 codes (the JAX/Triton Blackwell FP8
GEMM post names both formats; mixed E4M3 x E5M2 products are the usual
gradient GEMM).

This reference evaluates the sum in float64.  Every decoded e4m3 value is
i * 2^j with |i| <= 15 and -9 <= j <= 5, so for per-tensor and row-wise scaling
of two e4m3 operands the inner sum sum_k decode*decode is an integer multiple of
2^-18 below 2^50 units and float64 holds it exactly in any summation order; only
the final multiplication by the scales rounds.  e5m2 values span 2^-16 to
57344, so sums with an e5m2 operand, like MX sums (each term carries a
power-of-two block factor), may round in float64: relative error near 1e-15 of
sum |a*b|, far inside the acceptance bound.

Acceptance bound (read from the target statement of this GEMM):
    |C - C_ref| <= 1e-3 * sum_k |dq_a[m,k] * dq_b[n,k]| + ulp_out(|C_ref|)
with ulp_out the spacing of the output format (fp16: 11 significant bits,
bf16: 8) at |C_ref|, never below that format's subnormal spacing.
"""
from __future__ import annotations

import numpy as np

from .formats import decode, decode_e8m0
from .quant import MX_BLOCK

_OUT_FORMATS = {
    # name: (significand bits incl. hidden, minimum normal exponent, largest finite)
    "f16": (11, -14, 65504.0),
    "bf16": (8, -126, float.fromhex("0x1.fep127")),
}


def dequantize(q: np.ndarray, scale, mode: str, fmt: str = "e4m3") -> np.ndarray:
    """float64 values represented by codes q [R,K] (element format fmt) and their scales."""
    v = decode(q, fmt)
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


def gemm_reference(qa, sa, qb, sb, mode: str, rows=None, cols=None, fmt_a: str = "e4m3",
                   fmt_b: str = "e4m3"):
    """(C_ref, abs_ref) in float64 for the selected rows of A and columns of C.

    qa: uint8 [M,K]; qb: uint8 [N,K] (column-major B); fmt_a / fmt_b: their
    element formats ("e4m3" or "e5m2").  Scales: "tensor" -> float32 scalars;
    "rowwise" -> float32 [M] and [N]; "mx32" -> uint8 E8M0 [M,K/32] and
    [N,K/32].  ``rows``/``cols`` pick a sub-block (default all).
    """
    qa_s = _select(qa, rows)
    qb_s = _select(qb, cols)
    if mode == "tensor":
        da, db = decode(qa_s, fmt_a), decode(qb_s, fmt_b)
        f = float(np.float32(sa)) * float(np.float32(sb))
        inner = da @ db.T                        # e4m3 x e4m3: exact (see above)
        absin = np.abs(da) @ np.abs(db).T
        return inner * f, absin * abs(f)
    if mode == "rowwise":
        da, db = decode(qa_s, fmt_a), decode(qb_s, fmt_b)
        fa = _select(np.asarray(sa, np.float32), rows).astype(np.float64)
        fb = _select(np.asarray(sb, np.float32), cols).astype(np.float64)
        inner = da @ db.T
        absin = np.abs(da) @ np.abs(db).T
        outer = fa[:, None] * fb[None, :]
        return inner * outer, absin * np.abs(outer)
    if mode == "mx32":
        da = dequantize(qa_s, _select(sa, rows), "mx32", fmt_a)
        db = dequantize(qb_s, _select(sb, cols), "mx32", fmt_b)
        return da @ db.T, np.abs(da) @ np.abs(db).T
    raise ValueError(f"unknown scale mode {mode!r}")


def grouped_reference(qa, sa, offsets, qb, sb, mode: str, rows=None, cols=None,
                      fmt: str = "e4m3"):
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
            c, a = gemm_reference(qa[r], sa, qb[g], np.asarray(sb)[g], mode, cols=cols,
                                  fmt_a=fmt, fmt_b=fmt)
        else:
            c, a = gemm_reference(qa[r], np.asarray(sa)[r], qb[g], np.asarray(sb)[g], mode,
                                  cols=cols, fmt_a=fmt, fmt_b=fmt)
        C[sel] = c
        A[sel] = a
    return C, A


# ---- fused epilogue: bias and activation ------------------------------------
# The Cutlass-named Triton FP8 post fuses a Cutlass bias_add_relu epilogue into
# the GEMM to save a round trip of C through memory.  Read here as
#     C[m,n] = act(y[m,n] + bias[n]),  y the scaled GEMM above,
# with act one of ReLU (the post's), or the exact (erf) GELU and SiLU, the other
# activations a GEMM epilogue commonly fuses.

# Lipschitz bounds of the activations: sup |act'| (GELU: 1.1289 at y = sqrt(2);
# SiLU: 1.0998 at y = 2.3994)
ACT_LIPSCHITZ = {"none": 1.0, "relu": 1.0, "gelu": 1.129, "silu": 1.1}


def activation(y: np.ndarray, act: str) -> np.ndarray:
    """The activation in float64: identity, max(y, 0), y * (1 + erf(y / sqrt 2)) / 2
    or y / (1 + exp(-y))."""
    y = np.asarray(y, dtype=np.float64)
    if act == "none":
        return y
    if act == "relu":
        return np.maximum(y, 0.0)
    if act == "gelu":
        from scipy.special import erf
        return 0.5 * y * (1.0 + erf(y / np.sqrt(2.0)))
    if act == "silu":
        with np.errstate(over="ignore"):
            return y / (1.0 + np.exp(-y))
    raise ValueError(f"unknown activation {act!r}")


def epilogue_reference(C_ref, abs_ref, bias, act: str, cols=None):
    """(out_ref, y_ref) of the fused epilogue: y = C_ref + bias[n] (float64, bias
    float32 [N] or None), out = act(y).  ``cols`` selects the bias entries of the
    columns C_ref holds (default all)."""
    y = np.asarray(C_ref, dtype=np.float64)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float32).astype(np.float64)
        y = y + (b if cols is None else b[np.asarray(cols)])[None, :]
    return activation(y, act), y


def epilogue_tolerance(out_ref, y_ref, abs_ref, act: str, out: str) -> np.ndarray:
    """Bound for the fused epilogue, from the arithmetic: the GEMM part
    1e-3 * sum|a*b|, plus the fp32 rounding of the scaled value and of the bias
    add (2^-22 |y|), both through the activation's Lipschitz bound L; plus the
    activation's own fp32 evaluation (2^-20 (|act(y)| + |y|), covering the
    cancellation in 1 + erf for large negative y); plus one output ulp."""
    L = ACT_LIPSCHITZ[act]
    y = np.abs(np.asarray(y_ref, np.float64))
    o = np.abs(np.asarray(out_ref, np.float64))
    return (L * (1e-3 * np.asarray(abs_ref, np.float64) + 2.0 ** -22 * y)
            + 2.0 ** -20 * (o + y) + output_ulp(out_ref, out))


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
    """Round-to-nearest-even of float64 values onto the output format (the 16-bit
    layer output in references; diagnostics).

    Values whose rounding exceeds the largest finite number become +-inf.
    """
    p, emin, fmax = _OUT_FORMATS[out]
    x = np.asarray(x, dtype=np.float64)
    q = output_ulp(x, out)
    r = np.rint(x / q) * q                    # x / q is exact (power of two); rint is RNE
    return np.where(np.abs(r) > fmax, np.copysign(np.inf, x), r)


# ---- output quantised for the next layer (e4m3 + E8M0 per 32 columns) --------
# The fused epilogue may write its result as MX codes, the form the next FP8
# GEMM consumes (the Cutlass-named Triton FP8 post fuses epilogues to save a
# round trip of C).  Reading: y = act(C + bias) is quantised per row in blocks
# of 32 consecutive columns with the MX rule of ``quant.quantize_mx``.

def mx_output_reference(out_ref: np.ndarray):
    """(codes uint8 [M,N], E8M0 uint8 [M,N/32]): the MX e4m3 quantisation of the
    binary32 rounding of the exact epilogue output."""
    from .quant import quantize_mx
    return quantize_mx(np.asarray(out_ref, np.float64).astype(np.float32), "e4m3")


def _e4m3_half_spacing(x: np.ndarray) -> np.ndarray:
    """Half the e4m3 spacing at scaled magnitudes x (2^-10 in the subnormal range)."""
    x = np.abs(np.asarray(x, np.float64))
    _, ex = np.frexp(np.maximum(x, 2.0 ** -6))
    return np.ldexp(1.0, (ex.astype(np.int64) - 1) - 3 - 1)


def mx_output_within_bound(q, codes, out_ref, tol_y) -> np.ndarray:
    """Which outputs of an MX-quantised result (q [M,N] e4m3 codes, codes [M,N/32]
    E8M0) are acceptable against the exact output out_ref with tolerance tol_y.

    The dequantised value decode(q) * 2^e must lie within tol_y plus half an e4m3
    spacing (at the block exponent e and the magnitude |out_ref| + tol_y) of
    out_ref, or, for a block maximum in [448, 512) * 2^e, at most the saturation
    distance beyond 448 * 2^e; the block exponent may differ by one from that of
    the exact block maximum only where that maximum lies within its tolerance of
    a power of two."""
    from .formats import decode_e4m3
    from .quant import mx_scale_code
    y = np.asarray(out_ref, np.float64)
    t = np.asarray(tol_y, np.float64) * np.ones_like(y)
    M, N = y.shape
    e = np.repeat(np.asarray(codes, np.int64) - 127, 32, axis=1)          # [M, N]
    dq = decode_e4m3(q) * np.ldexp(1.0, e)
    scaled = (np.abs(y) + t) * np.ldexp(1.0, -e)
    allow = t + _e4m3_half_spacing(scaled) * np.ldexp(1.0, e)
    sat = np.maximum(np.abs(y) + t - 448.0 * np.ldexp(1.0, e), 0.0)
    ok = np.abs(dq - y) <= allow + sat
    # block exponents: exact unless the block maximum's band crosses a power of two
    blk = np.abs(y).reshape(M, N // 32, 32)
    tb = t.reshape(M, N // 32, 32)
    amax = blk.max(axis=2)
    lo = mx_scale_code(np.maximum(blk - tb, 0).max(axis=2).astype(np.float32)).astype(np.int64)
    hi = mx_scale_code((blk + tb).max(axis=2).astype(np.float32)).astype(np.int64)
    c = np.asarray(codes, np.int64)
    ok_code = (c >= np.minimum(lo, mx_scale_code(amax.astype(np.float32)))) & (c <= hi)
    return ok & np.repeat(ok_code, 32, axis=1)


# ---- output quantised for the next layer with a fresh per-tensor / per-row scale
# The same saving of a C round trip, with the output's scale chosen afresh from
# the layer's output itself: one for the whole output or one per row (the
# scale_a of a row-wise GEMM that takes the codes as its A operand).  Reading:
# the layer's output is the GEMM's bf16 result (the pages' kernels accumulate in
# fp32 and cast the tile to a 16-bit type on store), and the next layer's
# operand is that tensor quantised with the per-tensor or row-wise rule of
# ``quant.quantize_tensor`` / ``quant.quantize_rowwise``.

def scaled_output_reference(out_ref: np.ndarray, out_mode: str, fmt: str = "e4m3"):
    """(codes uint8 [M,N], scales float32 [M] or ()): the row-wise ("rowwise") or
    per-tensor ("tensor") quantisation of the bf16 rounding of the exact epilogue
    output (bf16 values are exact in binary32)."""
    from .quant import quantize_rowwise, quantize_tensor
    y16 = round_to_output(np.asarray(out_ref, np.float64), "bf16").astype(np.float32)
    if out_mode == "rowwise":
        return quantize_rowwise(y16, fmt)
    if out_mode == "tensor":
        return quantize_tensor(y16, fmt)
    raise ValueError(f"unknown output scale mode {out_mode!r}")


_SPACING = {"e4m3": (3, -6), "e5m2": (2, -14)}      # mantissa bits, smallest normal exponent


def _half_spacing(x: np.ndarray, fmt: str) -> np.ndarray:
    """Half the spacing of the format's values at magnitudes x (the subnormal
    spacing below the smallest normal)."""
    mbits, emin = _SPACING[fmt]
    x = np.abs(np.asarray(x, np.float64))
    _, ex = np.frexp(np.maximum(x, 2.0 ** emin))
    return np.ldexp(1.0, (ex.astype(np.int64) - 1) - mbits - 1)


def scaled_output_within_bound(q, scales, out_ref, tol_y, out_mode: str,
                               fmt: str = "e4m3") -> np.ndarray:
    """Which outputs of a result quantised with fresh scales (q [M,N] codes,
    scales float [M] for "rowwise" or one value for "tensor") are acceptable
    against the exact output out_ref, given the GEMM's tolerance tol_y.

    A computed output y' lies within tol_y of out_ref and its bf16 rounding y16
    within t = tol_y + half a bf16 ulp at |out_ref| + tol_y; the maximum of |y16|
    over the row (or the whole output) lies between those of |out_ref| - t and
    |out_ref| + t, so its scale fl32(amax / max) lies between the scales of those
    two bounds (binary32 rounding is monotone), or is 1 where the lower bound is
    0.  A code then dequantises (value times the scale s) to within t, half a
    spacing of the format at the scaled magnitude (|out_ref| + t) / s, the
    binary32 rounding of the quotient (2^-24 relative) and, for values beyond
    max * s, the saturation distance, of out_ref.  The mask is False for every
    output of a row (or of the output) whose scale is out of range."""
    from .formats import FORMATS
    y = np.asarray(out_ref, np.float64)
    a = np.abs(y)
    t0 = np.asarray(tol_y, np.float64) * np.ones_like(y)
    t = t0 + 0.5 * output_ulp(a + t0, "bf16")
    fmax = float(FORMATS[fmt]["max"])
    lo_v = np.maximum(a - t, 0.0)
    hi_v = a + t
    if out_mode == "rowwise":
        lo, hi = lo_v.max(axis=1), hi_v.max(axis=1)
        s = np.asarray(scales, np.float64).reshape(-1)
        sb = s[:, None] * np.ones_like(y)
    elif out_mode == "tensor":
        lo, hi = np.asarray(lo_v.max()), np.asarray(hi_v.max())
        s = np.asarray(scales, np.float64).reshape(())
        sb = s * np.ones_like(y)
    else:
        raise ValueError(f"unknown output scale mode {out_mode!r}")
    s_lo = (lo.astype(np.float32) / np.float32(fmax)).astype(np.float64)
    s_hi = (hi.astype(np.float32) / np.float32(fmax)).astype(np.float64)
    ok_s = ((s >= s_lo) & (s <= s_hi) & (s > 0)) | ((lo == 0) & (s == 1.0))
    dq = FORMATS[fmt]["decode"](np.asarray(q, np.uint8)) * sb
    allow = (t + _half_spacing(hi_v / sb, fmt) * sb + 2.0 ** -24 * hi_v
             + np.maximum(hi_v - fmax * sb, 0.0))
    ok = np.abs(dq - y) <= allow
    ok_s = ok_s[:, None] if out_mode == "rowwise" else ok_s
    return ok & ok_s
