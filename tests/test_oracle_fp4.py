"""Pins of the oracle's FP4 (e2m1) table, encoder, nibble packing, MXFP4
quantiser and GEMM reference.

The e2m1 table is checked against the OCP MX specification's tabulated points,
by exhaustive round trip of all 16 codes, at every midpoint between adjacent
magnitudes (ties to the even code) and their binary32 neighbours, and against
an independent rounding model (round to a multiple of the binade's spacing
with numpy's rint).  The MXFP4 quantiser is pinned by a hand-derived worked
example, block-maximum range and scale linearity; the GEMM reference by exact
rational arithmetic and closed forms.
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
MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, *v = line.split()
                d[k] = v
    return d


def test_e2m1_spec_points():
    with open(os.path.join(GOLDEN, "ocp_mx_e2m1_points.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            code, val = int(line.split()[0], 16), float(line.split()[1])
            got = F.E2M1_DECODE[code]
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e2m1_table_structure():
    t = F.E2M1_DECODE
    assert t.shape == (16,) and not np.isnan(t).any()
    assert list(t[:8]) == MAGS, "the 8 magnitudes, strictly increasing"
    assert np.array_equal(t[8:], -t[:8]), "bit 3 is the sign"
    assert F.E2M1_MAX == 6.0 and F.FORMATS["e2m1"]["emax"] == 2 == Q.E2M1_EMAX


def test_e2m1_exhaustive_round_trip():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.encode_e2m1(F.decode_e2m1(codes)), codes)


def test_e2m1_midpoints_and_neighbours():
    for lo in range(7):
        a, b = MAGS[lo], MAGS[lo + 1]
        mid = (a + b) / 2
        even = lo if lo % 2 == 0 else lo + 1
        for sgn, sbit in ((1.0, 0), (-1.0, 8)):
            v = np.float32(sgn * mid)
            assert F.encode_e2m1(np.array([v]))[0] == (even | sbit), (mid, sgn)
            below = np.nextafter(np.float32(mid), np.float32(0))
            above = np.nextafter(np.float32(mid), np.float32(100))
            assert F.encode_e2m1(np.array([sgn * below], np.float32))[0] == (lo | sbit)
            assert F.encode_e2m1(np.array([sgn * above], np.float32))[0] == ((lo + 1) | sbit)


def test_e2m1_saturation_and_signed_zero():
    v = np.array([6.0, 6.5, 7.0, 8.0, 1e30, -7.0, -1e30, 0.0, -0.0, -1e-30], np.float32)
    assert list(F.encode_e2m1(v)) == [7, 7, 7, 7, 7, 15, 15, 0, 8, 8]


def _rint_model(v):
    """Independent RNE: round |v| to a multiple of its binade's e2m1 spacing
    (0.5 below 2, 1 below 4, 2 above) with numpy's rint, saturate at 6."""
    a = np.abs(v.astype(np.float64))
    ulp = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    r = np.minimum(np.rint(a / ulp) * ulp, 6.0)
    code = np.searchsorted(np.array(MAGS), r)
    return (code | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def test_e2m1_against_rint_model():
    rng = np.random.default_rng(7)
    grid = np.arange(-9.0, 9.0, 1.0 / 64, dtype=np.float32)
    rnd = (rng.standard_normal(20000) * 3).astype(np.float32)
    for v in (grid, rnd):
        assert np.array_equal(F.encode_e2m1(v), _rint_model(v))


def test_pack_unpack():
    codes = np.arange(32, dtype=np.uint8).reshape(2, 16) & 0xF
    p = F.pack_fp4(codes)
    assert p.shape == (2, 8) and p[0, 0] == 0x10 and p[0, 1] == 0x32
    assert np.array_equal(F.unpack_fp4(p), codes)


def _block(vals, rest):
    x = np.full(32, rest, np.float32)
    x[:len(vals)] = vals
    return x


def test_mxfp4_worked_example():
    g = _golden("mxfp4_worked_example.txt")
    b1 = _block([float(v) for v in g["b1_x"]], float(g["b1_rest"][0]))
    b2 = _block([float(v) for v in g["b2_x"]], 0.0)
    b3 = np.zeros(32, np.float32)
    x = np.stack([np.concatenate([b1, b2, b3])])          # one row, three blocks
    q, codes = Q.quantize_mx(x, "e2m1")
    assert list(codes[0]) == [int(g["b1_code"][0]), int(g["b2_code"][0]), int(g["b3_code"][0])]
    n1 = len(g["b1_q"])
    assert [int(c) for c in q[0, :n1]] == [int(v, 16) for v in g["b1_q"]]
    assert np.all(q[0, n1:32] == int(g["b1_qrest"][0], 16))
    assert [int(c) for c in q[0, 32:36]] == [int(v, 16) for v in g["b2_q"]]
    assert np.all(q[0, 36:] == 0)
    p = F.pack_fp4(q)
    assert [int(b) for b in p[0, :4]] == [int(v, 16) for v in g["b1_packed"]]
    assert np.all(p[0, 4:16] == int(g["b1_packed_rest"][0], 16))
    assert [int(b) for b in p[0, 16:18]] == [int(v, 16) for v in g["b2_packed"]]
    assert np.all(p[0, 18:] == 0)


def test_mxfp4_block_max_and_linearity():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((8, 256)) * rng.uniform(0.1, 10, (8, 8)).repeat(32, 1)).astype(np.float32)
    q, codes = Q.quantize_mx(x, "e2m1")
    blk = np.abs(x).reshape(8, 8, 32)
    j = np.argmax(blk, axis=2)
    qb = q.reshape(8, 8, 32)
    top = np.take_along_axis(qb, j[:, :, None], 2)[:, :, 0] & 7
    assert np.all(top >= 6), "amax * 2^-e lies in [4, 8): code of 4 or 6"
    for sh in (-3, 5):
        q2, c2 = Q.quantize_mx(np.ldexp(x, sh).astype(np.float32), "e2m1")
        assert np.array_equal(q2, q) and np.array_equal(c2.astype(int), codes.astype(int) + sh)


def test_mxfp4_needs_mx_scales():
    with pytest.raises(ValueError):
        Q.quantize(np.zeros((1, 32), np.float32), "tensor", "e2m1")


def test_mxfp4_gemm_reference_exact_rational():
    rng = np.random.default_rng(5)
    xa = (rng.standard_normal((4, 64)) * 3).astype(np.float32)
    xb = (rng.standard_normal((4, 64)) * 0.01).astype(np.float32)
    qa, sa = Q.quantize_mx(xa, "e2m1")
    qb, sb = Q.quantize_mx(xb, "e2m1")
    C, A = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a="e2m1", fmt_b="e2m1")
    for m in range(4):
        for n in range(4):
            tot = Fraction(0)
            ab = Fraction(0)
            for k in range(64):
                da = Fraction(MAGS[qa[m, k] & 7]) * (-1 if qa[m, k] & 8 else 1) * Fraction(2) ** (int(sa[m, k // 32]) - 127)
                db = Fraction(MAGS[qb[n, k] & 7]) * (-1 if qb[n, k] & 8 else 1) * Fraction(2) ** (int(sb[n, k // 32]) - 127)
                tot += da * db
                ab += abs(da * db)
            assert C[m, n] == float(tot) and A[m, n] == float(ab)


def test_mxfp4_gemm_closed_forms():
    K = 96
    ones = np.ones((3, K), np.float32)
    q, s = Q.quantize_mx(ones, "e2m1")           # 1 = 4 * 2^-2: code 6, e = -2
    assert np.all(q == 6) and np.all(s == 125)
    C, _ = O.gemm_reference(q, s, q, s, "mx32", fmt_a="e2m1", fmt_b="e2m1")
    assert np.all(C == K)
    # A = 6 * I (rows of 32-blocks): C = 6 * dq(B) restricted to those columns
    eye = np.zeros((32, 32), np.float32)
    np.fill_diagonal(eye, 6.0)
    qi, si = Q.quantize_mx(eye, "e2m1")
    xb = np.random.default_rng(1).standard_normal((5, 32)).astype(np.float32)
    qb, sb = Q.quantize_mx(xb, "e2m1")
    C, _ = O.gemm_reference(qi, si, qb, sb, "mx32", fmt_a="e2m1", fmt_b="e2m1")
    dqb = O.dequantize(qb, sb, "mx32", "e2m1")
    assert np.array_equal(C, 6.0 * dqb.T)
