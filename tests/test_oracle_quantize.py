"""Pins of the oracle's quantisation (per-tensor, row-wise, MX).

Closed forms: a hand-derived worked example (tests/golden), the largest element
of a tensor / row maps to +-448, an MX block maximum lands in [256, 448];
scale linearity (x -> 2^j x leaves codes unchanged, scales the per-tensor and
row-wise scale by exactly 2^j and adds j to every E8M0 code); degenerate inputs
(all zero); and special cases that reduce to one another (a row-wise quantise
of one row is a per-tensor quantise; MX blocks whose maxima are 448*2^e equal
per-tensor quantisation with s = 2^e).
"""
import os

import numpy as np
import pytest

from oracle import quant as Q
from oracle import formats as F
from oracle.formats import decode_e4m3
from workloads import block_scaled_normal, normal, with_outliers

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_worked_example.txt")


def _golden():
    d = {}
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, *v = line.split()
                d[k] = v
    return d


def test_worked_example_tensor():
    g = _golden()
    x = np.array([float(v) for v in g["x"]], np.float32)[None, :]
    q, s = Q.quantize_tensor(x)
    assert [int(c) for c in q[0]] == [int(v, 16) for v in g["q"]]
    assert float(s) == float(g["s"][0])


def test_worked_example_mx():
    g = _golden()
    x = np.full((1, 32), float(g["mx_rest"][0]), np.float32)
    x[0, 0] = float(g["mx_x0"][0])
    q, codes = Q.quantize_mx(x)
    assert codes.shape == (1, 1) and codes[0, 0] == int(g["mx_code"][0])
    assert q[0, 0] == int(g["mx_q0"][0], 16)
    assert np.all(q[0, 1:] == int(g["mx_qrest"][0], 16))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_max_element_maps_to_448(seed):
    rng = np.random.default_rng(seed)
    x = with_outliers(rng, 64, 96)
    q, s = Q.quantize_tensor(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[i] == (0xFE if x[i] < 0 else 0x7E)
    qr, sr = Q.quantize_rowwise(x)
    j = np.argmax(np.abs(x), axis=1)
    for r in range(x.shape[0]):
        assert qr[r, j[r]] == (0xFE if x[r, j[r]] < 0 else 0x7E)
    assert np.all(np.abs(decode_e4m3(qr)) <= 448)


def test_mx_block_max_range_and_code():
    rng = np.random.default_rng(3)
    x = block_scaled_normal(rng, 16, 256)
    q, codes = Q.quantize_mx(x)
    blocks = np.abs(x).reshape(16, 8, 32)
    amax = blocks.max(axis=2)
    # shared exponent e satisfies 2^(e+8) <= amax < 2^(e+9)
    e = codes.astype(np.int64) - 127
    assert np.all(np.ldexp(1.0, e + 8) <= amax) and np.all(amax < np.ldexp(1.0, e + 9))
    arg = blocks.argmax(axis=2)
    qmax = np.abs(decode_e4m3(q.reshape(16, 8, 32)))[np.arange(16)[:, None], np.arange(8)[None, :], arg]
    assert np.all((qmax >= 256) & (qmax <= 448))


@pytest.mark.parametrize("j", [-20, -3, 1, 7, 30])
def test_scale_linearity(j):
    rng = np.random.default_rng(11)
    x = block_scaled_normal(rng, 8, 128)
    y = np.ldexp(x, j).astype(np.float32)
    assert np.array_equal(np.ldexp(y, -j), x), "power-of-two scaling is exact here"
    q1, s1 = Q.quantize_tensor(x)
    q2, s2 = Q.quantize_tensor(y)
    assert np.array_equal(q1, q2) and float(s2) == float(np.ldexp(s1, j))
    q1, s1 = Q.quantize_rowwise(x)
    q2, s2 = Q.quantize_rowwise(y)
    assert np.array_equal(q1, q2) and np.array_equal(s2, np.ldexp(s1, j).astype(np.float32))
    q1, c1 = Q.quantize_mx(x)
    q2, c2 = Q.quantize_mx(y)
    assert np.array_equal(q1, q2) and np.array_equal(c2.astype(int), c1.astype(int) + j)


def test_all_zero_inputs():
    x = np.zeros((3, 64), np.float32)
    x[1] = -0.0
    q, s = Q.quantize_tensor(x)
    assert float(s) == 1.0 and np.all(q[0] == 0) and np.all(q[1] == 0x80)
    qr, sr = Q.quantize_rowwise(x)
    assert np.all(sr == 1.0)
    qm, cm = Q.quantize_mx(x)
    assert np.all(cm == 127) and np.array_equal(qm, q)


def test_rowwise_single_row_is_tensor():
    rng = np.random.default_rng(5)
    x = with_outliers(rng, 6, 200)
    qr, sr = Q.quantize_rowwise(x)
    for r in range(6):
        qt, st = Q.quantize_tensor(x[r:r + 1])
        assert np.array_equal(qt[0], qr[r]) and float(st) == float(sr[r])


def test_mx_equals_tensor_when_block_max_is_448_times_power_of_two():
    rng = np.random.default_rng(9)
    e = 3
    x = (rng.uniform(-1, 1, size=(4, 96)) * 448 * 2.0 ** e).astype(np.float32)
    x.reshape(4, 3, 32)[:, :, 5] = np.float32(448 * 2.0 ** e)    # every block's max = 448*2^e
    qm, cm = Q.quantize_mx(x)
    assert np.all(cm == 127 + e)
    qt, st = Q.quantize_tensor(x)
    assert float(st) == 2.0 ** e
    assert np.array_equal(qm, qt)


def test_mx_subnormal_and_extreme_exponents():
    x = np.zeros((1, 96), np.float32)
    x[0, :32] = np.float32(1e-40)                # subnormal block maximum -> code 0
    x[0, 32:64] = np.float32(3e38)               # floor(log2) = 127 -> code 127+119 = 246
    x[0, 64] = np.float32(2.0 ** -126)           # min normal -> e = -134 -> clamped code 0
    q, c = Q.quantize_mx(x)
    assert c[0, 0] == 0 and c[0, 1] == 127 + 127 - 8 and c[0, 2] == 0
    # 1e-40 * 2^127 ~ 0.017 -> nearest e4m3 code
    assert q[0, 0] == F.encode_e4m3(np.ldexp(np.float64(np.float32(1e-40)), 127))


def test_quantize_rejects_bad_mx_k():
    with pytest.raises(ValueError):
        Q.quantize_mx(np.zeros((2, 48), np.float32))


def test_division_is_binary32():
    # fl32(x / s) differs from the float64 quotient for some x: the oracle must use the former.
    rng = np.random.default_rng(2)
    x = normal(rng, 1, 4096)
    q, s = Q.quantize_tensor(x)
    fl32 = (x / s).astype(np.float32)
    assert np.array_equal(q, F.encode_e4m3(fl32))


# ---- e5m2 elements ------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_e5m2_max_element_maps_to_57344(seed):
    rng = np.random.default_rng(seed)
    x = with_outliers(rng, 64, 96)
    q, s = Q.quantize_tensor(x, "e5m2")
    assert float(s) == float(np.float32(np.max(np.abs(x))) / np.float32(57344.0))
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[i] == (0xFB if x[i] < 0 else 0x7B)
    qr, sr = Q.quantize_rowwise(x, "e5m2")
    j = np.argmax(np.abs(x), axis=1)
    for r in range(x.shape[0]):
        assert qr[r, j[r]] == (0xFB if x[r, j[r]] < 0 else 0x7B)
    assert np.all(np.abs(F.decode_e5m2(qr)) <= 57344)
    assert np.all(np.isfinite(F.decode_e5m2(qr)))


def test_e5m2_mx_block_max_range_and_code():
    rng = np.random.default_rng(4)
    x = block_scaled_normal(rng, 16, 256)
    q, codes = Q.quantize_mx(x, "e5m2")
    blocks = np.abs(x).reshape(16, 8, 32)
    amax = blocks.max(axis=2)
    # shared exponent e = floor(log2 amax) - 15: 2^(e+15) <= amax < 2^(e+16)
    e = codes.astype(np.int64) - 127
    assert np.all(np.ldexp(1.0, e + 15) <= amax) and np.all(amax < np.ldexp(1.0, e + 16))
    arg = blocks.argmax(axis=2)
    qmax = np.abs(F.decode_e5m2(q.reshape(16, 8, 32)))[np.arange(16)[:, None],
                                                       np.arange(8)[None, :], arg]
    assert np.all((qmax >= 32768) & (qmax <= 57344))
    # the e5m2 code is the e4m3 code lowered by the difference of the largest exponents
    _, c4 = Q.quantize_mx(x, "e4m3")
    assert np.array_equal(codes.astype(int), c4.astype(int) - 7)


@pytest.mark.parametrize("j", [-9, 2, 13])
def test_e5m2_scale_linearity(j):
    rng = np.random.default_rng(12)
    x = block_scaled_normal(rng, 8, 128)
    y = np.ldexp(x, j).astype(np.float32)
    for mode in ("tensor", "rowwise"):
        q1, s1 = Q.quantize(x, mode, "e5m2")
        q2, s2 = Q.quantize(y, mode, "e5m2")
        assert np.array_equal(q1, q2)
        assert np.array_equal(np.asarray(s2), np.ldexp(np.asarray(s1), j).astype(np.float32))
    q1, c1 = Q.quantize_mx(x, "e5m2")
    q2, c2 = Q.quantize_mx(y, "e5m2")
    assert np.array_equal(q1, q2) and np.array_equal(c2.astype(int), c1.astype(int) + j)


def test_e5m2_encoding_is_coarser_rounding_of_the_same_value():
    # e5m2 keeps 2 mantissa bits: its code for a value equals the e4m3 code's value
    # rounded again only where no double-rounding tie occurs; check the simple
    # consequence that both lie within half an e5m2 ulp of the scaled input
    rng = np.random.default_rng(13)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    q, s = Q.quantize_tensor(x, "e5m2")
    v = x.astype(np.float64) / float(s)
    got = F.decode_e5m2(q)
    _, ex = np.frexp(np.maximum(np.abs(v), 2.0 ** -14))
    half_ulp = np.ldexp(1.0, ex - 1 - 2 - 1)          # 2^(floor(log2|v|) - 2) / 2
    assert np.all(np.abs(got - v) <= half_ulp * (1 + 1e-12))
