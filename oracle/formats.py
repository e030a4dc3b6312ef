"""e4m3fn and E8M0 codes: decode tables and the round-to-nearest-even encoder.

TEST INFRASTRUCTURE (see the package docstring).

E4M3 is the operand format the JAX/Triton Blackwell FP8 GEMM post prefers
("E4M3 to balance precision and range"); the Cutlass-named Triton FP8 post
fixes the finite-only variant by naming ``torch.float8_e4m3fn``.  The field
layout below is the OCP OFP8 one: 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, subnormals when the exponent field is 0, and S.1111.111 as
the only NaN (no infinities), so the largest finite magnitude is
1.75 * 2^8 = 448.

E8M0 is the MX shared-scale format ("Hopper/Blackwell architecture features"
§12.6.1 names MXFP8): an 8-bit biased exponent, value 2^(code-127), with 0xFF
reserved for NaN.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F


def _e4m3_value(code: int) -> float:
    """Value of one e4m3fn code from its bit fields (OFP8 E4M3 definition)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = math.ldexp(m, -9)             # subnormal: 0.m * 2^(1-7) = m * 2^-9
    else:
        mag = math.ldexp(8 + m, e - 7 - 3)  # normal: 1.m * 2^(e-7) = (8+m) * 2^(e-10)
    return -mag if s else mag


def _e8m0_value(code: int) -> float:
    return math.nan if code == 0xFF else math.ldexp(1.0, code - 127)


E4M3_DECODE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_DECODE = np.array([_e8m0_value(c) for c in range(256)], dtype=np.float64)

# Non-negative finite magnitudes, indexed by code 0x00..0x7E (strictly increasing).
_POS_MAGS = E4M3_DECODE[:0x7F].copy()


def decode_e4m3(q: np.ndarray) -> np.ndarray:
    """float64 values of uint8 e4m3fn codes (exact)."""
    return E4M3_DECODE[np.asarray(q, dtype=np.uint8)]


def decode_e8m0(c: np.ndarray) -> np.ndarray:
    """float64 values 2^(c-127) of uint8 E8M0 codes (exact)."""
    return E8M0_DECODE[np.asarray(c, dtype=np.uint8)]


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code to each value, ties to the even code, saturating.

    Definition (no bit manipulation): for a = |v| in float64, take the two
    adjacent representable magnitudes lo <= a < hi from the table of the 127
    non-negative finite codes and return the nearer one; on an exact tie return
    the code whose least significant bit is 0 (round to nearest even, also
    across binades).  Magnitudes at or above 448 saturate to 448 (code 0x7E),
    the format having no infinity.  The sign bit is copied from v, so -0.0 and
    negative values that round to zero give 0x80.  NaN gives 0x7F | sign.
    """
    v = np.asarray(v)
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    lo = np.searchsorted(_POS_MAGS, a, side="right") - 1   # _POS_MAGS[lo] <= a
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _POS_MAGS[lo]
    d_hi = _POS_MAGS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(a >= E4M3_MAX, np.uint8(0x7E), code)
    code = np.where(np.isnan(a), np.uint8(E4M3_NAN_CODE), code)
    return (code | sign).astype(np.uint8)
