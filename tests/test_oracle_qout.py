"""Pins of the oracle's check for outputs quantised for the next layer with a fresh
per-tensor or per-row scale.  Its reference is the per-tensor / row-wise
quantiser (pinned in test_oracle_quantize and test_oracle_formats) applied to
the layer's bf16 output (round_to_output, pinned against torch's cast in
test_oracle_gemm); here the reference and the acceptance check are pinned by
hand-worked examples, closed forms, special cases and planted mistakes the
check must reject."""
import numpy as np
import pytest

import oracle as O
from oracle import quant as Q


def _y(seed, M=8, N=96):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, N)) * rng.uniform(0.01, 100, (M, 1))


def _bf16(y):
    return O.round_to_output(y, "bf16")


def test_worked_example_by_hand():
    """Row [3, -1.5, 0.1]: bf16(0.1) = 0.10009765625; amax 3, s = fl32(3 / 448);
    3 / s rounds to 448 (code 0x7E), -1.5 / s to -224 = -1.75 * 2^7 (sign,
    exponent field 14, mantissa 6: 0xF6), 0.10009765625 / s = 14.948... to 15 =
    1.875 * 2^3 (exponent field 10, mantissa 7: 0x57).  The all-zero second row
    takes scale 1 and zero codes."""
    y = np.array([[3.0, -1.5, 0.1], [0.0, 0.0, 0.0]])
    q, s = O.scaled_output_reference(y, "rowwise")
    assert s[0] == np.float32(3.0) / np.float32(448.0) and s[1] == 1.0
    assert list(q[0]) == [0x7E, 0xF6, 0x57] and list(q[1]) == [0, 0, 0]
    qt, st = O.scaled_output_reference(y, "tensor")
    assert st == s[0] and np.array_equal(qt[0], q[0]) and not qt[1].any()


def test_the_bf16_output_is_what_is_quantised():
    """With row maximum 448 (s = 1), 9.4990234375 sits just below the e4m3
    midpoint 9.5 (between 9 = 0x51 and 10 = 0x52): quantised in binary32 it
    gives 9, but its bf16 rounding is 9.5 exactly (bf16 spacing 1/16 there),
    a tie that goes to the even code 10."""
    y = np.array([[448.0, 9.4990234375]])
    q, s = O.scaled_output_reference(y, "rowwise")
    assert s[0] == 1.0 and q[0, 0] == 0x7E and q[0, 1] == 0x52
    q32, _ = Q.quantize_rowwise(y.astype(np.float32))
    assert q32[0, 1] == 0x51


@pytest.mark.parametrize("mode", ["rowwise", "tensor"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_exact_quantisation_passes_with_zero_tolerance(mode, fmt):
    for seed in range(4):
        y = _bf16(_y(seed))
        q, s = O.scaled_output_reference(y, mode, fmt)
        assert O.scaled_output_within_bound(q, s, y, 0.0, mode, fmt).all()


def test_reference_is_the_quantiser_of_the_bf16_output():
    y = _y(7)
    q, s = O.scaled_output_reference(y, "rowwise")
    q2, s2 = Q.quantize_rowwise(_bf16(y).astype(np.float32), "e4m3")
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    q, s = O.scaled_output_reference(y, "tensor", "e5m2")
    q2, s2 = Q.quantize_tensor(_bf16(y).astype(np.float32), "e5m2")
    assert np.array_equal(q, q2) and s == s2


def test_closed_form_representable_outputs():
    """y = decode(code) * 2^j with every row's maximum code 448 (e4m3 values have
    4 significant bits, so y is exact in bf16): the row scale is 2^j exactly and
    the codes are the constructed ones; with one j for every row, the per-tensor
    scale is that 2^j and the codes again the constructed ones."""
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7F, (6, 64)).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    codes[:, 5] = 0x7E
    j = rng.integers(-20, 20, 6)
    y = O.decode_e4m3(codes) * np.ldexp(1.0, j)[:, None]
    q, s = O.scaled_output_reference(y, "rowwise")
    assert np.array_equal(s, np.ldexp(1.0, j).astype(np.float32))
    assert np.array_equal(q, codes)
    assert O.scaled_output_within_bound(q, s, y, 0.0, "rowwise").all()
    yt = O.decode_e4m3(codes) * 2.0 ** 5
    qt, st = O.scaled_output_reference(yt, "tensor")
    assert st == 2.0 ** 5 and np.array_equal(qt, codes)


def test_planted_mistakes_are_rejected():
    y = _bf16(_y(11))
    q, s = O.scaled_output_reference(y, "rowwise")
    i = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    bad = q.copy()
    bad[i] ^= 0x02                                   # wrong mantissa of the row maximum
    assert not O.scaled_output_within_bound(bad, s, y, 0.0, "rowwise")[i]
    bad = q.copy()
    bad[i] ^= 0x80                                   # wrong sign
    assert not O.scaled_output_within_bound(bad, s, y, 0.0, "rowwise")[i]
    ss = s.copy()
    ss[2] *= 2                                       # a scale twice too large
    ok = O.scaled_output_within_bound(q, ss, y, 0.0, "rowwise")
    assert not ok[2].any() and ok[3].all()
    ss = s.copy()
    ss[[0, 1]] = ss[[1, 0]]                          # scales of two rows swapped
    assert not O.scaled_output_within_bound(q, ss, y, 0.0, "rowwise")[:2].any()
    qt, st = O.scaled_output_reference(y, "tensor")
    assert not O.scaled_output_within_bound(qt, st * np.float32(1.01), y, 0.0, "tensor").any()
    r = (int(np.argmax(np.abs(y).max(axis=1))) + 1) % y.shape[0]
    assert not O.scaled_output_within_bound(q, s[r], y, 0.0, "tensor").any()  # a row's scale


def test_tolerance_widens_the_scale_band():
    """A computed maximum within the tolerance of the exact one moves the scale
    by at most that much: accepted with the tolerance, rejected without."""
    y = _bf16(_y(5))
    q, s = O.scaled_output_reference(y, "rowwise")
    amax = np.abs(y).max(axis=1)
    y2 = y.copy()
    r = np.argmax(np.abs(y[0]))
    y2[0, r] += np.sign(y[0, r]) * 1e-2 * amax[0]    # the GPU's maximum larger
    q2, s2 = O.scaled_output_reference(y2, "rowwise")
    assert s2[0] > s[0]
    assert not O.scaled_output_within_bound(q2, s2, y, 0.0, "rowwise")[0].all()
    assert O.scaled_output_within_bound(q2, s2, y, 1.1e-2 * amax[0], "rowwise")[0].all()


def test_e5m2_saturation_and_zero_output():
    y = np.zeros((2, 16))
    q, s = O.scaled_output_reference(y, "tensor", "e5m2")
    assert s == 1.0 and not q.any()
    assert O.scaled_output_within_bound(q, s, y, 0.0, "tensor", "e5m2").all()
    y = np.array([[57344.0 * 3, -2.0, 1e-3] + [0.0] * 13])
    q, s = O.scaled_output_reference(y, "rowwise", "e5m2")
    assert s[0] == np.float32(3.0) and q[0, 0] == 0x7B          # 57344: largest finite e5m2
    assert O.scaled_output_within_bound(q, s, y, 0.0, "rowwise", "e5m2").all()
