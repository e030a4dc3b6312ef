"""Pins of the oracle's FP6 (e2m3, e3m2) tables, encoders, 6-bit packing, MXFP6
quantiser and GEMM reference.

The tables are checked against the OCP MX specification's tabulated points, by
exhaustive round trip of all 64 codes of each format, at every midpoint between
adjacent magnitudes (ties to the even code) and their binary32 neighbours, and
against an independent rounding model (round to a multiple of the binade's
spacing with numpy's rint).  The packing is pinned by a hand-computed word; the
MXFP6 quantiser by a hand-derived worked example, block-maximum range and scale
linearity; the GEMM reference by exact rational arithmetic and closed forms.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from oracle import formats as F
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
# format -> (bias, mantissa bits, largest magnitude)
FMT = {"e2m3": (1, 3, 7.5), "e3m2": (3, 2, 28.0)}


def _mags(fmt):
    """The 32 non-negative magnitudes written out from the format definition."""
    bias, mb, _ = FMT[fmt]
    out = [m * 2.0 ** (1 - bias - mb) for m in range(2 ** mb)]           # subnormals
    for e in range(1, 2 ** (5 - mb)):
        out += [(1 + m / 2 ** mb) * 2.0 ** (e - bias) for m in range(2 ** mb)]
    return out


def _golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, *v = line.split()
                d[k] = v
    return d


def test_fp6_spec_points():
    n = 0
    with open(os.path.join(GOLDEN, "ocp_mx_fp6_points.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            fmt, code, val = line.split()
            got = F.decode(np.array([int(code, 16)], np.uint8), fmt)[0]
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))
            n += 1
    assert n == 14


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_table_structure(fmt):
    t = F.decode(np.arange(64, dtype=np.uint8), fmt)
    assert list(t[:32]) == _mags(fmt)
    assert np.all(np.diff(t[:32]) > 0), "32 strictly increasing magnitudes"
    assert np.array_equal(t[32:], -t[:32]), "bit 5 is the sign"
    assert F.FORMATS[fmt]["max"] == FMT[fmt][2] == t[31]
    assert F.FORMATS[fmt]["emax"] == math.floor(math.log2(FMT[fmt][2]))


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_exhaustive_round_trip(fmt):
    codes = np.arange(64, dtype=np.uint8)
    assert np.array_equal(F.encode(F.decode(codes, fmt), fmt), codes)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_midpoints_and_neighbours(fmt):
    mags = _mags(fmt)
    for lo in range(31):
        a, b = mags[lo], mags[lo + 1]
        mid = (a + b) / 2
        even = lo if lo % 2 == 0 else lo + 1
        for sgn, sbit in ((1.0, 0), (-1.0, 0x20)):
            assert F.encode(np.array([sgn * mid], np.float32), fmt)[0] == (even | sbit), (mid, sgn)
            below = np.nextafter(np.float32(mid), np.float32(0))
            above = np.nextafter(np.float32(mid), np.float32(1000))
            assert F.encode(np.array([sgn * below], np.float32), fmt)[0] == (lo | sbit)
            assert F.encode(np.array([sgn * above], np.float32), fmt)[0] == ((lo + 1) | sbit)


def test_fp6_saturation_and_signed_zero():
    v = np.array([7.5, 7.75, 7.9, 8.0, 1e30, -9.0, 0.0, -0.0, -1e-30], np.float32)
    assert list(F.encode_e2m3(v)) == [31, 31, 31, 31, 31, 63, 0, 32, 32]
    v = np.array([28.0, 29.9, 30.0, 32.0, 1e30, -40.0, 0.0, -0.0, -1e-30], np.float32)
    assert list(F.encode_e3m2(v)) == [31, 31, 31, 31, 31, 63, 0, 32, 32]


def _rint_model(v, fmt):
    """Independent RNE: round |v| to a multiple of its binade's spacing (the
    subnormal spacing below the smallest normal) with numpy's rint, saturate."""
    bias, mb, top = FMT[fmt]
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** (1 - bias))))
    ulp = 2.0 ** (e - mb)
    r = np.minimum(np.rint(a / ulp) * ulp, top)
    code = np.searchsorted(np.array(_mags(fmt)), r)
    return (code | (np.signbit(v).astype(np.int64) << 5)).astype(np.uint8)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_against_rint_model(fmt):
    rng = np.random.default_rng(7)
    top = FMT[fmt][2]
    grid = np.arange(-1.2 * top, 1.2 * top, top / 997, dtype=np.float32)
    rnd = (rng.standard_normal(20000) * top / 3).astype(np.float32)
    tiny = (rng.standard_normal(5000) * 0.2).astype(np.float32)
    for v in (grid, rnd, tiny):
        assert np.array_equal(F.encode(v, fmt), _rint_model(v, fmt))


def test_pack_fp6_word_and_round_trip():
    # 1 | 2 << 6 | 3 << 12 | 4 << 18 = 0x103081 -> 0x81 0x30 0x10
    assert list(F.pack_fp6(np.array([[1, 2, 3, 4]], np.uint8))[0]) == [0x81, 0x30, 0x10]
    assert list(F.pack_fp6(np.full((1, 4), 63, np.uint8))[0]) == [0xFF, 0xFF, 0xFF]
    codes = np.random.default_rng(3).integers(0, 64, (5, 64)).astype(np.uint8)
    p = F.pack_fp6(codes)
    assert p.shape == (5, 48)
    assert np.array_equal(F.unpack_fp6(p), codes)
    # element i sits in bits 6i .. 6i + 5 of the row's little-endian bit string
    bits = np.unpackbits(p[0], bitorder="little")
    for i in range(64):
        assert int(sum(int(b) << j for j, b in enumerate(bits[6 * i:6 * i + 6]))) == codes[0, i]


def _block(vals):
    x = np.zeros(32, np.float32)
    x[:len(vals)] = vals
    return x


def test_mxfp6_worked_example():
    g = _golden("mxfp6_worked_example.txt")
    b = [_block([float(v) for v in g[f"b{i}_x"]]) for i in (1, 2, 3, 4)]
    q, codes = Q.quantize_mx(np.concatenate(b[:2])[None], "e2m3")
    assert list(codes[0]) == [int(g["b1_code"][0]), int(g["b2_code"][0])]
    assert [int(c) for c in q[0, :4]] == [int(v, 16) for v in g["b1_q"]]
    assert np.all(q[0, 4:32] == 0)
    assert [int(c) for c in q[0, 32:35]] == [int(v, 16) for v in g["b2_q"]]
    assert [int(c) for c in F.pack_fp6(q)[0, :3]] == [int(v, 16) for v in g["b1_packed"]]
    q, codes = Q.quantize_mx(np.concatenate(b[2:])[None], "e3m2")
    assert list(codes[0]) == [int(g["b3_code"][0]), int(g["b4_code"][0])]
    assert [int(c) for c in q[0, :3]] == [int(v, 16) for v in g["b3_q"]]
    assert [int(c) for c in q[0, 32:33]] == [int(v, 16) for v in g["b4_q"]]


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_mxfp6_block_max_and_linearity(fmt):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((8, 256)) * rng.uniform(0.1, 10, (8, 8)).repeat(32, 1)).astype(np.float32)
    q, codes = Q.quantize_mx(x, fmt)
    blk = np.abs(x).reshape(8, 8, 32)
    j = np.argmax(blk, axis=2)
    top = np.take_along_axis(q.reshape(8, 8, 32), j[:, :, None], 2)[:, :, 0] & 0x1F
    lo = 24 if fmt == "e2m3" else 28            # amax * 2^-e lies in [2^emax, 2^(emax+1))
    assert np.all(top >= lo) and np.all(top <= 31)
    for sh in (-3, 5):
        q2, c2 = Q.quantize_mx(np.ldexp(x, sh).astype(np.float32), fmt)
        assert np.array_equal(q2, q) and np.array_equal(c2.astype(int), codes.astype(int) + sh)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_mxfp6_needs_mx_scales(fmt):
    with pytest.raises(ValueError):
        Q.quantize(np.zeros((1, 32), np.float32), "rowwise", fmt)


@pytest.mark.parametrize("fa,fb", [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2")])
def test_mxfp6_gemm_reference_exact_rational(fa, fb):
    rng = np.random.default_rng(5)
    xa = (rng.standard_normal((4, 64)) * 3).astype(np.float32)
    xb = (rng.standard_normal((4, 64)) * 0.01).astype(np.float32)
    qa, sa = Q.quantize_mx(xa, fa)
    qb, sb = Q.quantize_mx(xb, fb)
    C, A = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a=fa, fmt_b=fb)
    ma, mb = _mags(fa), _mags(fb)
    for m in range(4):
        for n in range(4):
            tot = Fraction(0)
            ab = Fraction(0)
            for k in range(64):
                da = (Fraction(ma[qa[m, k] & 31]) * (-1 if qa[m, k] & 32 else 1)
                      * Fraction(2) ** (int(sa[m, k // 32]) - 127))
                db = (Fraction(mb[qb[n, k] & 31]) * (-1 if qb[n, k] & 32 else 1)
                      * Fraction(2) ** (int(sb[n, k // 32]) - 127))
                tot += da * db
                ab += abs(da * db)
            assert C[m, n] == float(tot) and A[m, n] == float(ab)


def test_mxfp6_gemm_closed_forms():
    K = 96
    ones = np.ones((3, K), np.float32)
    q, s = Q.quantize_mx(ones, "e2m3")           # 1 = 4 * 2^-2: code 24, e = -2
    assert np.all(q == 24) and np.all(s == 125)
    C, _ = O.gemm_reference(q, s, q, s, "mx32", fmt_a="e2m3", fmt_b="e2m3")
    assert np.all(C == K)
    q3, s3 = Q.quantize_mx(ones, "e3m2")         # 1 = 16 * 2^-4: code 28, e = -4
    assert np.all(q3 == 28) and np.all(s3 == 123)
    C, _ = O.gemm_reference(q, s, q3, s3, "mx32", fmt_a="e2m3", fmt_b="e3m2")
    assert np.all(C == K)
    # A = 7.5 * I: C = 7.5 * dq(B) restricted to those columns
    eye = np.zeros((32, 32), np.float32)
    np.fill_diagonal(eye, 7.5)
    qi, si = Q.quantize_mx(eye, "e2m3")
    xb = np.random.default_rng(1).standard_normal((5, 32)).astype(np.float32)
    qb, sb = Q.quantize_mx(xb, "e3m2")
    C, _ = O.gemm_reference(qi, si, qb, sb, "mx32", fmt_a="e2m3", fmt_b="e3m2")
    assert np.array_equal(C, 7.5 * O.dequantize(qb, sb, "mx32", "e3m2").T)
