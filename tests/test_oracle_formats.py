"""Pins of the oracle's e4m3fn / e5m2 / E8M0 tables and its round-to-nearest-even encoders.

The encoder is checked against (a) the OCP specification's tabulated points,
(b) exhaustive enumeration of all 256 codes, (c) every midpoint between
adjacent representable magnitudes and the fp32 neighbours of each, (d) an
independent bit-level rounding of the binary32 representation written here,
and (e) PyTorch's CPU cast to ``float8_e4m3fn`` in its non-overflowing range.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_points(name):
    pts = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            pts.append((int(parts[0], 16), float(parts[1])))
    return pts


def test_e4m3_spec_points():
    for code, val in _read_points("ofp8_e4m3fn_points.txt"):
        got = F.E4M3_DECODE[code]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e8m0_spec_points():
    for code, val in _read_points("ocp_mx_e8m0_points.txt"):
        got = F.E8M0_DECODE[code]
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val, hex(code)
    # every finite code is an exact power of two 2^(c-127)
    for c in range(255):
        assert F.E8M0_DECODE[c] == math.ldexp(1.0, c - 127)


def test_e4m3_table_structure():
    t = F.E4M3_DECODE
    assert np.isnan(t).sum() == 2 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "127 non-negative finite magnitudes strictly increase"
    assert np.array_equal(t[0x80:0xFF], -pos), "sign bit mirrors magnitudes"
    assert pos[-1] == 448.0 and F.E4M3_MAX == 448.0
    # each binade holds 8 values with spacing 2^(e-10); subnormal spacing 2^-9
    assert np.all(np.diff(pos[:9]) == 2.0 ** -9)
    for e in range(1, 16):
        vals = pos[8 * e: 8 * e + 8]
        if e == 15:
            vals = vals[:7]
        assert np.all(vals == (8 + np.arange(len(vals))) * 2.0 ** (e - 10))


def test_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = F.E4M3_DECODE[codes]
    assert np.array_equal(F.encode_e4m3(vals), codes)
    assert np.array_equal(F.encode_e4m3(vals.astype(np.float32)), codes)


def test_encode_midpoints_ties_to_even():
    pos = F.E4M3_DECODE[:0x7F]
    for c in range(0x7E):
        lo, hi = pos[c], pos[c + 1]
        mid = (lo + hi) / 2                       # exact in fp32 and fp64
        even = c if c % 2 == 0 else c + 1
        for sgn in (1.0, -1.0):
            sb = 0x80 if sgn < 0 else 0
            assert F.encode_e4m3(np.float32(sgn * mid)) == even | sb
            assert F.encode_e4m3(np.float64(sgn * mid)) == even | sb
            up = np.nextafter(np.float32(mid), np.float32(np.inf))
            dn = np.nextafter(np.float32(mid), np.float32(0))
            assert F.encode_e4m3(np.float32(sgn) * up) == (c + 1) | sb
            assert F.encode_e4m3(np.float32(sgn) * dn) == c | sb


def test_encode_saturation_and_zero():
    sat = np.array([448, 449, 463.99, 464, 479, 480, 500, 511.9, 1e30,
                    np.finfo(np.float32).max], dtype=np.float32)
    assert np.all(F.encode_e4m3(sat) == 0x7E)
    assert np.all(F.encode_e4m3(-sat) == 0xFE)
    assert F.encode_e4m3(np.float32(0.0)) == 0x00
    assert F.encode_e4m3(np.float32(-0.0)) == 0x80
    assert F.encode_e4m3(np.float32(-1e-30)) == 0x80
    assert F.encode_e4m3(np.float32(2.0 ** -10)) == 0x00      # tie with 0x01 -> even
    assert F.encode_e4m3(np.float32(2.0 ** -10 * 1.0001)) == 0x01
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    assert F.encode_e4m3(tiny) == 0x00 and F.encode_e4m3(-tiny) == 0x80


def _bitlevel_rne_e4m3(x: np.ndarray) -> np.ndarray:
    """Independent reference: RNE on the binary32 bit pattern (no table)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.int64)
    sign = ((u >> 31) & 1).astype(np.uint8) << 7
    a = u & 0x7FFFFFFF
    exp = (a >> 23) - 127                      # unbiased binary32 exponent (normals)
    out = np.zeros(a.shape, dtype=np.int64)
    # target: e4m3 exponent field E = exp + 7 if >= 1 (normal) else subnormal (quantum 2^-9)
    for i in np.ndindex(a.shape):
        ai = int(a[i])
        if ai == 0:
            out[i] = 0
            continue
        if ai >= 0x7F800000:
            out[i] = 0x7F if ai > 0x7F800000 else 0x7E
            continue
        e = int(exp[i])
        mant = (ai & 0x7FFFFF) | (0x800000 if (ai >> 23) else 0)
        if (ai >> 23) == 0:
            e = -126
        # value = mant * 2^(e-23); quantum of the e4m3 slot holding it:
        q_exp = max(e, -6) - 3                 # ulp exponent: normal 2^(e-3), subnormal 2^-9
        shift = q_exp - (e - 23)               # bits of mant below the quantum
        if shift <= 0:
            n = mant << (-shift)
        else:
            n = mant >> shift
            rem = mant & ((1 << shift) - 1)
            half = 1 << (shift - 1)
            if rem > half or (rem == half and (n & 1)):
                n += 1
        # n * 2^q_exp is the rounded magnitude; rebuild the code
        mag = math.ldexp(n, q_exp)
        if mag >= 448.0:
            out[i] = 0x7E
            continue
        if mag < 2.0 ** -6:
            out[i] = int(round(mag / 2.0 ** -9))
        else:
            E = math.frexp(mag)[1] - 1
            out[i] = ((E + 7) << 3) | (int(mag / 2.0 ** (E - 3)) - 8)
    return (out.astype(np.uint8) | sign)


def _fp32_neighbourhood(center: np.ndarray, width: int) -> np.ndarray:
    c = np.asarray(center, dtype=np.float32).view(np.uint32).astype(np.int64)
    offs = np.arange(-width, width + 1, dtype=np.int64)
    u = (c[:, None] + offs[None, :]).ravel()
    u = u[(u >= 0) & (u < 0x7F800000)]
    return u.astype(np.uint32).view(np.float32)


def test_encode_matches_bitlevel_rounding_near_every_boundary():
    pos = F.E4M3_DECODE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([_fp32_neighbourhood(pos[1:], 3), _fp32_neighbourhood(mids, 3),
                          np.array([464.0, 470.0, 500.0], np.float32)])
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(F.encode_e4m3(pts), _bitlevel_rne_e4m3(pts))


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    pos = F.E4M3_DECODE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    dense = np.concatenate([_fp32_neighbourhood(pos[1:], 64), _fp32_neighbourhood(mids, 64)])
    # random binary32 patterns over [0, 464]: uniform in bit space covers all binades
    bits = rng.integers(0, np.float32(464.0).view(np.uint32) + 1, size=2_000_000, dtype=np.int64)
    rand = bits.astype(np.uint32).view(np.float32)
    x = np.concatenate([dense, rand])
    x = x[np.abs(x) <= 464.0]
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.encode_e4m3(x), ref)



# ---- e5m2 -------------------------------------------------------------------

def test_e5m2_spec_points():
    for code, val in _read_points("ofp8_e5m2_points.txt"):
        got = F.E5M2_DECODE[code]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e5m2_table_structure():
    t = F.E5M2_DECODE
    assert np.isnan(t).sum() == 6 and np.isinf(t).sum() == 2
    pos = t[:0x7C]
    assert np.all(np.diff(pos) > 0), "124 non-negative finite magnitudes strictly increase"
    assert np.array_equal(t[0x80:0xFC], -pos), "sign bit mirrors magnitudes"
    assert pos[-1] == 57344.0 and F.E5M2_MAX == 57344.0
    # subnormal spacing 2^-16; each binade e >= 1 holds 4 values (4+m) * 2^(e-17)
    assert np.all(np.diff(pos[:5]) == 2.0 ** -16)
    for e in range(1, 31):
        assert np.all(pos[4 * e: 4 * e + 4] == (4 + np.arange(4)) * 2.0 ** (e - 17))
    # e5m2 is e4m3's exponent range widened: the bit pattern is the top byte of an
    # IEEE binary16 number (1-5-10), so every code equals that half-precision value
    halves = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    fin = np.isfinite(t)
    assert np.array_equal(t[fin], halves[fin])
    assert np.array_equal(np.isnan(t), np.isnan(halves))


def test_e5m2_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if np.isfinite(F.E5M2_DECODE[c])], dtype=np.uint8)
    vals = F.E5M2_DECODE[codes]
    assert np.array_equal(F.encode_e5m2(vals), codes)
    assert np.array_equal(F.encode_e5m2(vals.astype(np.float32)), codes)
    assert np.array_equal(F.encode(vals, "e5m2"), codes)


def test_e5m2_midpoints_ties_to_even():
    pos = F.E5M2_DECODE[:0x7C]
    for c in range(0x7B):
        mid = (pos[c] + pos[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        for sgn in (1.0, -1.0):
            sb = 0x80 if sgn < 0 else 0
            assert F.encode_e5m2(np.float32(sgn * mid)) == even | sb
            up = np.nextafter(np.float32(mid), np.float32(np.inf))
            dn = np.nextafter(np.float32(mid), np.float32(0))
            assert F.encode_e5m2(np.float32(sgn) * up) == (c + 1) | sb
            assert F.encode_e5m2(np.float32(sgn) * dn) == c | sb


def test_e5m2_saturation_and_zero():
    sat = np.array([57344, 57345, 61439, 61440, 65536, 1e30, np.inf], dtype=np.float32)
    assert np.all(F.encode_e5m2(sat) == 0x7B)
    assert np.all(F.encode_e5m2(-sat) == 0xFB)
    assert F.encode_e5m2(np.float32(0.0)) == 0x00
    assert F.encode_e5m2(np.float32(-0.0)) == 0x80
    assert F.encode_e5m2(np.float32(2.0 ** -17)) == 0x00       # tie with 0x01 -> even
    assert F.encode_e5m2(np.float32(2.0 ** -17 * 1.0001)) == 0x01
    assert (F.encode_e5m2(np.float32(np.nan)) & 0x7F) == 0x7F


def _bitlevel_rne_small_float(x, mbits, emin, fmax):
    """Independent reference: RNE of binary32 values onto a small float format with
    `mbits` mantissa bits and minimum normal exponent `emin` (no table), returning
    the rounded magnitude with its sign, saturated at fmax."""
    out = np.empty(len(x), dtype=np.float64)
    for i, xi in enumerate(np.asarray(x, dtype=np.float32)):
        ai = int(np.float32(abs(xi)).view(np.uint32))
        if ai == 0:
            out[i] = math.copysign(0.0, xi)
            continue
        e = (ai >> 23) - 127 if (ai >> 23) else -126
        mant = (ai & 0x7FFFFF) | (0x800000 if (ai >> 23) else 0)
        q_exp = max(e, emin) - mbits
        shift = q_exp - (e - 23)
        if shift <= 0:
            n = mant << (-shift)
        else:
            n = mant >> shift
            rem = mant & ((1 << shift) - 1)
            half = 1 << (shift - 1)
            if rem > half or (rem == half and (n & 1)):
                n += 1
        mag = min(math.ldexp(n, q_exp), fmax)
        out[i] = math.copysign(mag, xi)
    return out


def test_e5m2_encode_matches_bitlevel_rounding_near_every_boundary():
    pos = F.E5M2_DECODE[:0x7C]
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([_fp32_neighbourhood(pos[1:], 3), _fp32_neighbourhood(mids, 3),
                          np.array([60000.0, 61440.0, 70000.0], np.float32)])
    pts = np.concatenate([pts, -pts])
    got = F.E5M2_DECODE[F.encode_e5m2(pts)]
    ref = _bitlevel_rne_small_float(pts, 2, -14, 57344.0)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_e5m2_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(11)
    pos = F.E5M2_DECODE[:0x7C]
    mids = (pos[:-1] + pos[1:]) / 2
    dense = np.concatenate([_fp32_neighbourhood(pos[1:], 64), _fp32_neighbourhood(mids, 64)])
    bits = rng.integers(0, np.float32(57344.0).view(np.uint32) + 1, size=2_000_000,
                        dtype=np.int64)
    x = np.concatenate([dense, bits.astype(np.uint32).view(np.float32)])
    x = x[np.abs(x) <= 57344.0]
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(F.encode_e5m2(x), ref)
