"""fp32 -> e4m3fn / e5m2 quantisation with per-tensor, row-wise and 32-element MX scales.

TEST INFRASTRUCTURE (see the package docstring).

What is quantised and why.  The JAX/Triton Blackwell FP8 GEMM post (paragraph
on kernel parameters) prefers E4M3 with per-block scale factors, and its
monitoring paragraph recommends fine-grained quantisation against FP8
underflow; "Hopper/Blackwell architecture features" §12.3.4 measures an FP8
row-wise GEMM and §12.6.1 names MXFP8 micro-scaling.  The pages leave the
scale rule open; the readings taken here are:

* per-tensor / row-wise: ``s = fl32(amax / 448)`` with amax the largest
  magnitude over the tensor, or over each row of A / each column of B (the
  reduction runs over K); ``s = 1`` when amax is 0; each element becomes
  ``encode(fl32(x / s))`` using IEEE binary32 division.
* MX (32 contiguous K elements per block, OCP MX v1.0 conversion): with
  E = floor(log2 amax) read exactly from the binary32 exponent, the shared
  exponent is e = E - 8 (8 being the largest e4m3 exponent, 448 = 1.75*2^8),
  stored as the E8M0 code clamp(e + 127, 0, 254); amax = 0 gives code 127.
  Each element becomes ``encode(x * 2^-e)``; the product is a power-of-two
  scaling, exact in float64, and values in (448, 512) saturate.

The same rules quantise to e5m2 (the JAX/Triton Blackwell FP8 GEMM post's
second FP8 format) with its largest magnitude 57344 in place of 448 and its
largest exponent 15 in place of 8 (the OCP MX rule for MXFP8 E5M2 elements).

MXFP4 (the FP4 micro-scaled format "Hopper/Blackwell architecture features"
§12.6.1 lists) takes the MX rule with e2m1 elements: largest magnitude 6, whose
exponent is 2, so e = floor(log2 amax) - 2; values in (6, 8) saturate to 6.
Its codes are returned one per uint8 (``formats.pack_fp4`` gives the packed
two-per-byte layout); per-tensor and row-wise FP4 are not defined here.

MXFP6 likewise takes the MX rule with e2m3 elements (largest 7.5, exponent 2:
e = floor(log2 amax) - 2; values in (7.5, 8) saturate to 7.5) or e3m2 elements
(largest 28, exponent 4: e = floor(log2 amax) - 4; values in (28, 32)
saturate to 28).  Codes are returned one per uint8 (``formats.pack_fp6`` gives
the packed layout, four codes in three bytes).

Inputs are rows x K float32 arrays with K contiguous; a column-major B is
passed as its N x K transpose, so "row" always means the outer index.
"""
from __future__ import annotations

import numpy as np

from .formats import FORMATS

MX_BLOCK = 32
E4M3_EMAX = 8          # floor(log2(448))
E5M2_EMAX = 15         # floor(log2(57344))
E2M1_EMAX = 2          # floor(log2(6))
E2M3_EMAX = 2          # floor(log2(7.5))
E3M2_EMAX = 4          # floor(log2(28))
MX_ONLY = ("e2m1", "e2m3", "e3m2")     # element formats defined with MX scales only


def _scale_from_amax(amax: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """fl32(amax / fmax) elementwise (fmax = 448 or 57344), 1.0 where amax is zero
    (binary32 division)."""
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / np.float32(FORMATS[fmt]["max"])
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize_tensor(x: np.ndarray, fmt: str = "e4m3"):
    """Per-tensor scale: returns (q uint8 [R,K], s float32 scalar array shape ())."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x)) if x.size else np.float32(0)
    s = _scale_from_amax(amax, fmt)
    q = FORMATS[fmt]["encode"](x / s)          # float32 / float32: binary32 division
    return q, np.asarray(s, dtype=np.float32).reshape(())


def quantize_rowwise(x: np.ndarray, fmt: str = "e4m3"):
    """One scale per row (reduction over K): returns (q uint8 [R,K], s float32 [R])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = _scale_from_amax(amax, fmt)
    q = FORMATS[fmt]["encode"](x / s[:, None])
    return q, s


def mx_scale_code(amax: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """E8M0 code of the shared exponent for each block maximum (OCP MX v1.0 rule):
    clamp(floor(log2 amax) - emax + 127, 0, 254), 127 for an all-zero block."""
    amax = np.asarray(amax, dtype=np.float32).astype(np.float64)
    _, ex = np.frexp(amax)                  # amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex-1
    e = (ex.astype(np.int64) - 1) - FORMATS[fmt]["emax"]
    code = np.clip(e + 127, 0, 254)
    return np.where(amax == 0, 127, code).astype(np.uint8)


def quantize_mx(x: np.ndarray, fmt: str = "e4m3"):
    """32-element K blocks: returns (q uint8 [R,K], e8m0 codes uint8 [R, K/32])."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("MX quantisation needs K to be a multiple of 32")
    blocks = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2) if K else np.zeros((R, 0), np.float32)
    codes = mx_scale_code(amax, fmt)
    e = codes.astype(np.int64) - 127
    scaled = np.ldexp(blocks.astype(np.float64), -e[:, :, None])   # exact power-of-two scaling
    q = FORMATS[fmt]["encode"](scaled).reshape(R, K)
    return q, codes


def quantize(x: np.ndarray, mode: str, fmt: str = "e4m3"):
    """Dispatch on mode name: "tensor" | "rowwise" | "mx32"; fmt "e4m3" | "e5m2",
    or "e2m1" / "e2m3" / "e3m2" with "mx32" only."""
    if fmt in MX_ONLY and mode != "mx32":
        raise ValueError(f"{fmt} elements are defined with MX block scales only")
    if mode == "tensor":
        return quantize_tensor(x, fmt)
    if mode == "rowwise":
        return quantize_rowwise(x, fmt)
    if mode == "mx32":
        return quantize_mx(x, fmt)
    raise ValueError(f"unknown scale mode {mode!r}")
