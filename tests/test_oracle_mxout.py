"""Pins of the oracle's check for outputs quantised for the next layer (e4m3 with
an E8M0 scale per 32 columns): its reference is the MX quantiser (pinned in
test_oracle_quantize / test_oracle_formats) applied to the binary32 output, and
the acceptance check is pinned here by exact cases, closed forms and planted
mistakes it must reject."""
import numpy as np

import oracle as O
from oracle import quant as Q


def _y(seed, M=8, N=256):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, N)) * rng.uniform(0.01, 100, (M, N // 32)).repeat(32, 1)


def test_exact_quantisation_passes_with_zero_tolerance():
    for seed in range(4):
        y = _y(seed).astype(np.float32).astype(np.float64)
        q, c = O.mx_output_reference(y)
        assert O.mx_output_within_bound(q, c, y, 0.0).all()


def test_reference_is_the_mx_quantiser():
    y = _y(7)
    q, c = O.mx_output_reference(y)
    q2, c2 = Q.quantize_mx(y.astype(np.float32), "e4m3")
    assert np.array_equal(q, q2) and np.array_equal(c, c2)


def test_closed_form_representable_outputs():
    """y = decode(code) * 2^j with each block's maximum 448 * 2^j: the MX codes are
    the constructed codes and dequantise to y exactly."""
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7F, (4, 128)).astype(np.uint8)      # finite e4m3 magnitudes
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    codes[:, ::32] = 0x7E                                          # block maximum 448
    j = rng.integers(-20, 20, (4, 4))
    y = O.decode_e4m3(codes) * np.ldexp(1.0, np.repeat(j, 32, axis=1))
    q, c = O.mx_output_reference(y)
    assert np.array_equal(c.astype(np.int64), j + 127)
    assert np.array_equal(q, codes)
    assert O.mx_output_within_bound(q, c, y, 0.0).all()


def test_planted_mistakes_are_rejected():
    y = _y(11).astype(np.float32).astype(np.float64)
    q, c = O.mx_output_reference(y)
    i = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    bad = q.copy()
    bad[i] ^= 0x02                                  # wrong mantissa of the block maximum
    assert not O.mx_output_within_bound(bad, c, y, 0.0)[i]
    bad = q.copy()
    bad[i] ^= 0x80                                  # wrong sign
    assert not O.mx_output_within_bound(bad, c, y, 0.0)[i]
    cc = c.copy()
    cc[0, 0] += 2                                   # block exponent off by two
    assert not O.mx_output_within_bound(q, cc, y, 0.0)[0, :32].any()
    cc = c.copy()
    cc[0, 0] += 1                                   # off by one, far from a power of two
    amax = np.abs(y[0, :32]).max()
    if abs(np.log2(amax) - np.round(np.log2(amax))) > 0.01:
        assert not O.mx_output_within_bound(q, cc, y, 0.0)[0, :32].all()


def test_saturation_and_exponent_band():
    y = np.zeros((1, 32))
    y[0, 0] = 500.0                                 # block maximum in [448, 512)
    y[0, 1] = 3.0
    q, c = O.mx_output_reference(y)
    assert c[0, 0] == 127 and q[0, 0] == 0x7E
    assert O.mx_output_within_bound(q, c, y, 0.0).all()
    # a block maximum just below 256: exponent -1 exactly, 0 allowed within a tolerance
    y = np.zeros((1, 32))
    y[0, 0] = 256.0 * (1 - 2.0 ** -20)
    q, c = O.mx_output_reference(y)
    assert c[0, 0] == 126
    q0, c0 = O.mx_output_reference(np.array([[256.0] + [0.0] * 31]))
    assert c0[0, 0] == 127
    assert O.mx_output_within_bound(q0, c0, y, 1e-3).all()
    assert not O.mx_output_within_bound(q0, c0, y, 0.0).all()
