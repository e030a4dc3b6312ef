"""e4m3fn, e5m2, e2m1, e2m3, e3m2 and E8M0 codes: decode tables and the round-to-nearest-even encoders.

TEST INFRASTRUCTURE (see the package docstring).

E4M3 is the operand format the JAX/Triton Blackwell FP8 GEMM post prefers
("E4M3 to balance precision and range"); the Cutlass-named Triton FP8 post
fixes the finite-only variant by naming ``torch.float8_e4m3fn``.  The field
layout below is the OCP OFP8 one: 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, subnormals when the exponent field is 0, and S.1111.111 as
the only NaN (no infinities), so the largest finite magnitude is
1.75 * 2^8 = 448.

E5M2 is the second FP8 format the JAX/Triton Blackwell FP8 GEMM post names
(its second paragraph contrasts the two).  The OCP OFP8 layout: 1 sign bit,
5 exponent bits with bias 15, 2 mantissa bits, subnormals when the exponent
field is 0, and the IEEE-like specials S.11111.00 = infinity and S.11111.xx
(xx != 0) = NaN, so the largest finite magnitude is 1.75 * 2^15 = 57344.

E2M1 (FP4) is the 4-bit element format of MXFP4, one of the narrow formats
"Hopper/Blackwell architecture features" §12.6.1 lists for the new tensor
cores (FP4 / FP6 next to FP8, with micro-scaling); §12.6.4 lists FP4 GEMMs as
experimental.  The OCP MX v1.0 layout: 1 sign bit, 2 exponent bits with bias
1, 1 mantissa bit, a subnormal when the exponent field is 0, no infinity and
no NaN, so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  A code here is the
4-bit pattern S.EE.M in the low bits of a byte (sign = bit 3); two codes share
a byte when packed (see ``pack_fp4``).

E2M3 and E3M2 (FP6) are the 6-bit element formats of MXFP6, the other narrow
format §12.6.1 lists next to FP4.  The OCP MX v1.0 layouts: 1 sign bit (bit 5),
then 2 exponent bits with bias 1 and 3 mantissa bits (E2M3: subnormals m/8,
normals (1 + m/8) 2^(e-1), largest 7.5), or 3 exponent bits with bias 3 and 2
mantissa bits (E3M2: subnormals m/16, normals (1 + m/4) 2^(e-3), largest 28);
no infinity and no NaN.  Packed, a row of codes is a little-endian bit string,
element i in bits 6i .. 6i + 5 (four codes in three bytes, see ``pack_fp6``).

E8M0 is the MX shared-scale format ("Hopper/Blackwell architecture features"
§12.6.1 names MXFP8): an 8-bit biased exponent, value 2^(code-127), with 0xFF
reserved for NaN.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F
E5M2_MAX = 57344.0
E5M2_NAN_CODE = 0x7F


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


def _e5m2_value(code: int) -> float:
    """Value of one e5m2 code from its bit fields (OFP8 E5M2 definition)."""
    s = (code >> 7) & 1
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        mag = math.inf if m == 0 else math.nan
    elif e == 0:
        mag = math.ldexp(m, -16)            # subnormal: 0.m * 2^(1-15) = m * 2^-16
    else:
        mag = math.ldexp(4 + m, e - 15 - 2)  # normal: 1.m * 2^(e-15) = (4+m) * 2^(e-17)
    return -mag if s else mag


def _e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code from its bit fields (OCP MX FP4 definition)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = math.ldexp(m, -1)             # subnormal: 0.m * 2^(1-1) = m * 2^-1
    else:
        mag = math.ldexp(2 + m, e - 1 - 1)  # normal: 1.m * 2^(e-1) = (2+m) * 2^(e-2)
    return -mag if s else mag


def _e2m3_value(code: int) -> float:
    """Value of one 6-bit e2m3 code from its bit fields (OCP MX FP6 E2M3 definition)."""
    s = (code >> 5) & 1
    e = (code >> 3) & 0x3
    m = code & 0x7
    if e == 0:
        mag = math.ldexp(m, -3)             # subnormal: 0.m * 2^(1-1) = m * 2^-3
    else:
        mag = math.ldexp(8 + m, e - 1 - 3)  # normal: 1.m * 2^(e-1) = (8+m) * 2^(e-4)
    return -mag if s else mag


def _e3m2_value(code: int) -> float:
    """Value of one 6-bit e3m2 code from its bit fields (OCP MX FP6 E3M2 definition)."""
    s = (code >> 5) & 1
    e = (code >> 2) & 0x7
    m = code & 0x3
    if e == 0:
        mag = math.ldexp(m, -4)             # subnormal: 0.m * 2^(1-3) = m * 2^-4
    else:
        mag = math.ldexp(4 + m, e - 3 - 2)  # normal: 1.m * 2^(e-3) = (4+m) * 2^(e-5)
    return -mag if s else mag


def _e8m0_value(code: int) -> float:
    return math.nan if code == 0xFF else math.ldexp(1.0, code - 127)


E4M3_DECODE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E5M2_DECODE = np.array([_e5m2_value(c) for c in range(256)], dtype=np.float64)
E2M1_MAX = 6.0
E2M1_DECODE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
E2M3_MAX = 7.5
E2M3_DECODE = np.array([_e2m3_value(c) for c in range(64)], dtype=np.float64)
E3M2_MAX = 28.0
E3M2_DECODE = np.array([_e3m2_value(c) for c in range(64)], dtype=np.float64)
E8M0_DECODE = np.array([_e8m0_value(c) for c in range(256)], dtype=np.float64)

# Non-negative finite magnitudes, indexed by code (strictly increasing):
# e4m3fn 0x00..0x7E, e5m2 0x00..0x7B.
_POS_MAGS = E4M3_DECODE[:0x7F].copy()
_POS_MAGS_E5M2 = E5M2_DECODE[:0x7C].copy()
_POS_MAGS_E2M1 = E2M1_DECODE[:0x8].copy()          # e2m1 0x0..0x7
_POS_MAGS_E2M3 = E2M3_DECODE[:0x20].copy()         # e2m3 0x00..0x1F
_POS_MAGS_E3M2 = E3M2_DECODE[:0x20].copy()         # e3m2 0x00..0x1F


def decode_e4m3(q: np.ndarray) -> np.ndarray:
    """float64 values of uint8 e4m3fn codes (exact)."""
    return E4M3_DECODE[np.asarray(q, dtype=np.uint8)]


def decode_e5m2(q: np.ndarray) -> np.ndarray:
    """float64 values of uint8 e5m2 codes (exact)."""
    return E5M2_DECODE[np.asarray(q, dtype=np.uint8)]


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


def _encode_by_table(v: np.ndarray, mags: np.ndarray, fmax: float, nan_code: int,
                     sign_bit: int = 7) -> np.ndarray:
    """Nearest code among the non-negative finite magnitudes `mags` (code = index),
    ties to the even code, saturating at fmax, sign copied from v into bit
    `sign_bit`."""
    v = np.asarray(v)
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v).astype(np.uint8) << sign_bit
    top = len(mags) - 1
    lo = np.searchsorted(mags, a, side="right") - 1
    lo = np.clip(lo, 0, top)
    hi = np.minimum(lo + 1, top)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(a >= fmax, np.uint8(top), code)
    code = np.where(np.isnan(a), np.uint8(nan_code), code)
    return (code | sign).astype(np.uint8)


def encode_e5m2(v: np.ndarray) -> np.ndarray:
    """Nearest e5m2 code to each value, ties to the even code, saturating.

    The same definition as ``encode_e4m3`` over the 124 non-negative finite e5m2
    magnitudes: magnitudes at or above 57344 (infinity included) saturate to
    57344 (code 0x7B) -- the quantisers scale into range, and a saturating
    conversion never produces the format's infinity; NaN gives 0x7F | sign.
    """
    return _encode_by_table(v, _POS_MAGS_E5M2, E5M2_MAX, E5M2_NAN_CODE)


def decode_e2m1(q: np.ndarray) -> np.ndarray:
    """float64 values of 4-bit e2m1 codes held one per uint8 (exact)."""
    return E2M1_DECODE[np.asarray(q, dtype=np.uint8) & 0xF]


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code to each value (one 4-bit code per uint8), ties to the
    even code, saturating.

    The definition of ``encode_e4m3`` over the 8 non-negative e2m1 magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6: magnitudes at or above 6 saturate to 6 (code
    0x7), the sign goes to bit 3 (so -0.0 and small negatives give 0x8).  The
    format has no NaN; NaN inputs are out of contract (they give 0x7 | sign).
    """
    return _encode_by_table(v, _POS_MAGS_E2M1, E2M1_MAX, 0x7, sign_bit=3)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte along the last axis: element 2i in bits 0-3 and
    element 2i+1 in bits 4-7 (the first element in the low nibble)."""
    c = np.asarray(codes, dtype=np.uint8) & 0xF
    if c.shape[-1] % 2:
        raise ValueError("an even number of 4-bit codes per row is needed")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_fp4``: one 4-bit code per uint8, twice as many columns."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def decode_e2m3(q: np.ndarray) -> np.ndarray:
    """float64 values of 6-bit e2m3 codes held one per uint8 (exact)."""
    return E2M3_DECODE[np.asarray(q, dtype=np.uint8) & 0x3F]


def decode_e3m2(q: np.ndarray) -> np.ndarray:
    """float64 values of 6-bit e3m2 codes held one per uint8 (exact)."""
    return E3M2_DECODE[np.asarray(q, dtype=np.uint8) & 0x3F]


def encode_e2m3(v: np.ndarray) -> np.ndarray:
    """Nearest e2m3 code to each value (one 6-bit code per uint8), ties to the
    even code, saturating: the definition of ``encode_e4m3`` over the 32
    non-negative e2m3 magnitudes; magnitudes at or above 7.5 give 7.5 (code
    0x1F), the sign goes to bit 5.  No NaN exists (NaN inputs give 0x1F | sign)."""
    return _encode_by_table(v, _POS_MAGS_E2M3, E2M3_MAX, 0x1F, sign_bit=5)


def encode_e3m2(v: np.ndarray) -> np.ndarray:
    """Nearest e3m2 code to each value (one 6-bit code per uint8), ties to the
    even code, saturating at 28 (code 0x1F); sign in bit 5, as ``encode_e2m3``."""
    return _encode_by_table(v, _POS_MAGS_E3M2, E3M2_MAX, 0x1F, sign_bit=5)


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """6-bit codes packed along the last axis as a little-endian bit string:
    element i in bits 6i .. 6i + 5, so each group of four codes c0..c3 is the
    24-bit word c0 | c1 << 6 | c2 << 12 | c3 << 18 stored in three bytes, low
    byte first."""
    c = np.asarray(codes, dtype=np.uint32) & 0x3F
    if c.shape[-1] % 4:
        raise ValueError("a multiple of four 6-bit codes per row is needed")
    w = c[..., 0::4] | (c[..., 1::4] << 6) | (c[..., 2::4] << 12) | (c[..., 3::4] << 18)
    out = np.empty(c.shape[:-1] + (3 * w.shape[-1],), dtype=np.uint8)
    out[..., 0::3] = w & 0xFF
    out[..., 1::3] = (w >> 8) & 0xFF
    out[..., 2::3] = (w >> 16) & 0xFF
    return out


def unpack_fp6(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_fp6``: one 6-bit code per uint8, 4/3 as many columns."""
    p = np.asarray(packed, dtype=np.uint32)
    w = p[..., 0::3] | (p[..., 1::3] << 8) | (p[..., 2::3] << 16)
    out = np.empty(p.shape[:-1] + (4 * w.shape[-1],), dtype=np.uint8)
    for j in range(4):
        out[..., j::4] = (w >> (6 * j)) & 0x3F
    return out


# Element formats by name: decode, encode, largest finite magnitude and the
# exponent of that magnitude (emax, used by the MX scale rule).
FORMATS = {
    "e4m3": {"decode": decode_e4m3, "encode": encode_e4m3, "max": E4M3_MAX, "emax": 8},
    "e5m2": {"decode": decode_e5m2, "encode": encode_e5m2, "max": E5M2_MAX, "emax": 15},
    "e2m1": {"decode": decode_e2m1, "encode": encode_e2m1, "max": E2M1_MAX, "emax": 2},
    "e2m3": {"decode": decode_e2m3, "encode": encode_e2m3, "max": E2M3_MAX, "emax": 2},
    "e3m2": {"decode": decode_e3m2, "encode": encode_e3m2, "max": E3M2_MAX, "emax": 4},
}


def decode(q: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """float64 values of codes of element format `fmt`."""
    return FORMATS[fmt]["decode"](q)


def encode(v: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """Round-to-nearest-even saturating encoding onto element format `fmt`."""
    return FORMATS[fmt]["encode"](v)
