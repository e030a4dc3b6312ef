"""Pins of the oracle's GEMM reference, error bound and grouped form.

* brute force with exact rationals (``fractions.Fraction``) on 4x4x32 (one MX
  block) and 3x5x64 problems, all three scale modes;
* an integer-exact route: 512*decode(q) are integers, so the inner sums of the
  per-tensor / row-wise GEMM are checked against int64 matrix products;
* closed forms: all-ones operands give K*sa*sb, a 448*identity A returns the
  scaled B;
* reductions: MX with uniform block codes equals per-tensor with s = 2^e,
  row-wise with uniform scales equals per-tensor, a grouped GEMM with one
  expert equals the dense GEMM, and a grouped GEMM equals the concatenation of
  per-expert dense GEMMs (empty experts included);
* the output-format ulp and round-to-nearest-even against numpy's float16 and
  PyTorch's bfloat16 casts;
* scale linearity end to end (x -> 2^j x gives C -> 2^j C exactly).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from oracle import quant as Q
from workloads import block_scaled_normal, normal, with_outliers


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01           # no NaN codes
    return c


def _exact_value(code, fmt="e4m3"):
    table = O.E4M3_DECODE if fmt == "e4m3" else O.E5M2_DECODE
    return Fraction(table[int(code)])  # table values are exact dyadic rationals


def _rand_codes_fmt(rng, shape, fmt):
    if fmt == "e4m3":
        return _rand_codes(rng, shape)
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    bad = (c & 0x7C) == 0x7C                 # e5m2 infinities and NaNs
    c[bad] &= 0xF3
    return c


def _exact_gemm(qa, sa, qb, sb, mode, fmt_a="e4m3", fmt_b="e4m3"):
    M, K = qa.shape
    N = qb.shape[0]
    C = np.empty((M, N), dtype=object)
    A = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            aab = Fraction(0)
            for k in range(K):
                if mode == "tensor":
                    fa, fb = Fraction(float(sa)), Fraction(float(sb))
                elif mode == "rowwise":
                    fa, fb = Fraction(float(sa[m])), Fraction(float(sb[n]))
                else:
                    fa = Fraction(2) ** (int(sa[m, k // 32]) - 127)
                    fb = Fraction(2) ** (int(sb[n, k // 32]) - 127)
                t = fa * _exact_value(qa[m, k], fmt_a) * fb * _exact_value(qb[n, k], fmt_b)
                acc += t
                aab += abs(t)
            C[m, n] = acc
            A[m, n] = aab
    return C, A


@pytest.mark.parametrize("mode", ["tensor", "rowwise", "mx32"])
@pytest.mark.parametrize("shape", [(4, 4, 32), (3, 5, 64)])
def test_bruteforce_exact_rationals(mode, shape):
    M, N, K = shape
    rng = np.random.default_rng([["tensor", "rowwise", "mx32"].index(mode), M, N, K])
    qa, qb = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    if mode == "tensor":
        sa, sb = np.float32(0.37), np.float32(1.9e-3)
    elif mode == "rowwise":
        sa = rng.uniform(0.01, 3, M).astype(np.float32)
        sb = rng.uniform(0.01, 3, N).astype(np.float32)
    else:
        sa = rng.integers(100, 150, size=(M, K // 32)).astype(np.uint8)
        sb = rng.integers(100, 150, size=(N, K // 32)).astype(np.uint8)
    C, A = O.gemm_reference(qa, sa, qb, sb, mode)
    Ce, Ae = _exact_gemm(qa, sa, qb, sb, mode)
    for m in range(M):
        for n in range(N):
            # float64 results: at most a few roundings of the exact value
            assert abs(Fraction(C[m, n]) - Ce[m, n]) <= Fraction(2) ** -50 * Ae[m, n]
            assert abs(Fraction(A[m, n]) - Ae[m, n]) <= Fraction(2) ** -50 * Ae[m, n]


def test_integer_exact_inner_sums():
    rng = np.random.default_rng(21)
    M, N, K = 24, 40, 4096
    qa, qb = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    qa[0, :] = 0x7E                         # extremes: +-448 everywhere in one row / column
    qb[0, :] = 0xFE
    ia = np.rint(O.decode_e4m3(qa) * 512).astype(np.int64)
    ib = np.rint(O.decode_e4m3(qb) * 512).astype(np.int64)
    assert np.array_equal(ia / 512.0, O.decode_e4m3(qa)), "512*value is an integer"
    exact = ia @ ib.T                       # int64 product: exact (|sum| < 2^63)
    C, _ = O.gemm_reference(qa, np.float32(1), qb, np.float32(1), "tensor")
    assert np.array_equal(C * 2.0 ** 18, exact.astype(np.float64))
    assert np.all(np.abs(exact) < 2 ** 53)
    Cr, _ = O.gemm_reference(qa, np.ones(M, np.float32), qb, np.ones(N, np.float32), "rowwise")
    assert np.array_equal(Cr * 2.0 ** 18, exact.astype(np.float64))


def test_closed_form_all_ones():
    M, N, K = 8, 12, 256
    qa = np.full((M, K), 0x38, np.uint8)      # decode 1.0
    qb = np.full((N, K), 0x38, np.uint8)
    sa, sb = np.float32(0.125), np.float32(3.0)
    C, A = O.gemm_reference(qa, sa, qb, sb, "tensor")
    assert np.all(C == K * 0.125 * 3.0) and np.all(A == C)
    qx, sx = Q.quantize_tensor(np.full((M, K), 5.0, np.float32))   # end to end
    qy, sy = Q.quantize_tensor(np.full((N, K), 0.5, np.float32))
    assert np.all(qx == 0x7E) and np.all(qy == 0x7E)
    C2, _ = O.gemm_reference(qx, sx, qy, sy, "tensor")
    assert np.all(C2 == K * (448 * float(sx)) * (448 * float(sy)))


def test_closed_form_identity():
    rng = np.random.default_rng(4)
    K = N = 64
    qa = np.zeros((K, K), np.uint8)
    np.fill_diagonal(qa, 0x7E)                # 448 * I
    qb = _rand_codes(rng, (N, K))
    sb = rng.uniform(0.1, 2, N).astype(np.float32)
    sa = np.full(K, 0.25, np.float32)
    C, _ = O.gemm_reference(qa, sa, qb, sb, "rowwise")
    expect = 448 * 0.25 * O.dequantize(qb, sb, "rowwise").T
    assert np.array_equal(C, expect)


def test_mx_uniform_codes_equal_tensor():
    rng = np.random.default_rng(8)
    M, N, K = 16, 20, 128
    qa, qb = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    ca = np.full((M, K // 32), 130, np.uint8)
    cb = np.full((N, K // 32), 120, np.uint8)
    Cm, Am = O.gemm_reference(qa, ca, qb, cb, "mx32")
    Ct, At = O.gemm_reference(qa, np.float32(2.0 ** 3), qb, np.float32(2.0 ** -7), "tensor")
    assert np.array_equal(Cm, Ct) and np.array_equal(Am, At)


def test_rowwise_uniform_equals_tensor():
    rng = np.random.default_rng(10)
    M, N, K = 9, 7, 96
    qa, qb = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    Cr, Ar = O.gemm_reference(qa, np.full(M, 0.3, np.float32), qb, np.full(N, 0.7, np.float32),
                              "rowwise")
    Ct, At = O.gemm_reference(qa, np.float32(0.3), qb, np.float32(0.7), "tensor")
    assert np.array_equal(Cr, Ct) and np.array_equal(Ar, At)


def test_sampling_selects_subblock():
    rng = np.random.default_rng(12)
    x, y = block_scaled_normal(rng, 64, 128), block_scaled_normal(rng, 48, 128)
    qa, ca = Q.quantize_mx(x)
    qb, cb = Q.quantize_mx(y)
    C, A = O.gemm_reference(qa, ca, qb, cb, "mx32")
    rows, cols = np.array([0, 5, 63]), np.array([47, 1])
    Cs, As = O.gemm_reference(qa, ca, qb, cb, "mx32", rows=rows, cols=cols)
    assert np.allclose(Cs, C[np.ix_(rows, cols)], rtol=1e-14, atol=0)
    assert np.allclose(As, A[np.ix_(rows, cols)], rtol=1e-14, atol=0)


@pytest.mark.parametrize("mode", ["tensor", "rowwise", "mx32"])
def test_grouped_matches_per_expert_dense(mode):
    rng = np.random.default_rng(13)
    G, N, K = 4, 24, 64
    counts = np.array([5, 0, 9, 3])
    off = np.concatenate([[0], np.cumsum(counts)])
    x = normal(rng, int(off[-1]), K)
    w = np.stack([normal(rng, N, K, 0.02) for _ in range(G)])
    if mode == "tensor":
        qa, sa = Q.quantize_tensor(x)
        qw, sw = zip(*[Q.quantize_tensor(w[g]) for g in range(G)])
        sw = np.array([float(s) for s in sw], np.float32)
    elif mode == "rowwise":
        qa, sa = Q.quantize_rowwise(x)
        qw, sw = zip(*[Q.quantize_rowwise(w[g]) for g in range(G)])
        sw = np.stack(sw)
    else:
        qa, sa = Q.quantize_mx(x)
        qw, sw = zip(*[Q.quantize_mx(w[g]) for g in range(G)])
        sw = np.stack(sw)
    qw = np.stack(qw)
    C, A = O.grouped_reference(qa, sa, off, qw, sw, mode)
    for g in range(G):
        r = slice(off[g], off[g + 1])
        if counts[g] == 0:
            continue
        a_s = sa if mode == "tensor" else sa[r]
        Cg, Ag = O.gemm_reference(qa[r], a_s, qw[g], sw[g], mode)
        assert np.array_equal(C[r], Cg) and np.array_equal(A[r], Ag)
    # one expert == dense
    C1, _ = O.grouped_reference(qa, sa, [0, qa.shape[0]], qw[:1], sw[:1], mode)
    Cd, _ = O.gemm_reference(qa, sa, qw[0], sw[0], mode)
    assert np.array_equal(C1, Cd)
    # row sampling
    rows = np.array([0, 4, 5, 13, 16])
    Cs, _ = O.grouped_reference(qa, sa, off, qw, sw, mode, rows=rows)
    assert np.array_equal(Cs, C[rows])


def test_output_ulp_values():
    assert O.output_ulp(np.array(1.0), "bf16") == 2.0 ** -7
    assert O.output_ulp(np.array(1.0), "f16") == 2.0 ** -10
    assert O.output_ulp(np.array(1.99), "f16") == 2.0 ** -10
    assert O.output_ulp(np.array(-1024.0), "f16") == 1.0
    assert O.output_ulp(np.array(0.0), "f16") == 2.0 ** -24
    assert O.output_ulp(np.array(1e-9), "f16") == 2.0 ** -24
    assert O.output_ulp(np.array(0.0), "bf16") == 2.0 ** -133


def test_round_to_output_matches_library_casts():
    rng = np.random.default_rng(14)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-8, 5, 200000),
                        [0.0, 65504.0, 65519.0, 65520.0, 1e6, 2.0 ** -25, 3 * 2.0 ** -26]])
    with np.errstate(over="ignore"):
        ref16 = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(O.round_to_output(x, "f16"), ref16)
    x32 = x.astype(np.float32)               # torch's bf16 cast rounds binary32 once
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to_output(x32.astype(np.float64), "bf16"), ref)
    # RNE result is within half an ulp, so the bound accepts it
    C = x32.astype(np.float64)
    assert np.all(O.within_bound(O.round_to_output(C, "bf16"), C, np.abs(C), "bf16"))


@pytest.mark.parametrize("mode", ["tensor", "rowwise", "mx32"])
def test_end_to_end_scale_linearity(mode):
    rng = np.random.default_rng(15)
    x, y = with_outliers(rng, 16, 128), with_outliers(rng, 12, 128)
    qa, sa = Q.quantize(x, mode)
    qb, sb = Q.quantize(y, mode)
    qa2, sa2 = Q.quantize(np.ldexp(x, 5).astype(np.float32), mode)
    C1, _ = O.gemm_reference(qa, sa, qb, sb, mode)
    C2, _ = O.gemm_reference(qa2, sa2, qb, sb, mode)
    assert np.array_equal(C2, np.ldexp(C1, 5))


def test_tolerance_rejects_planted_errors():
    rng = np.random.default_rng(16)
    x, y = normal(rng, 32, 256), normal(rng, 32, 256)
    qa, sa = Q.quantize_rowwise(x)
    qb, sb = Q.quantize_rowwise(y)
    C, A = O.gemm_reference(qa, sa, qb, sb, "rowwise")
    good = O.round_to_output(C, "bf16")
    assert np.all(O.within_bound(good, C, A, "bf16"))
    # a dropped k term, a transposed operand and a sign flip are all caught
    Cdrop, _ = O.gemm_reference(qa[:, 1:], sa, qb[:, 1:], sb, "rowwise")
    assert not np.all(O.within_bound(Cdrop, C, A, "bf16"))
    assert not np.all(O.within_bound(C.T, C, A, "bf16"))
    assert not np.all(O.within_bound(-C, C, A, "bf16"))



@pytest.mark.parametrize("mode", ["tensor", "rowwise", "mx32"])
@pytest.mark.parametrize("fmts", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_bruteforce_exact_rationals_e5m2(mode, fmts):
    """e5m2 and mixed-format operands against exact rationals (4x4x64)."""
    M, N, K = 4, 4, 64
    fa_, fb_ = fmts
    rng = np.random.default_rng([7, ["tensor", "rowwise", "mx32"].index(mode), len(fa_ + fb_),
                                 fa_ == "e4m3"])
    qa, qb = _rand_codes_fmt(rng, (M, K), fa_), _rand_codes_fmt(rng, (N, K), fb_)
    if mode == "tensor":
        sa, sb = np.float32(0.37), np.float32(1.9e-3)
    elif mode == "rowwise":
        sa = rng.uniform(0.01, 3, M).astype(np.float32)
        sb = rng.uniform(0.01, 3, N).astype(np.float32)
    else:
        sa = rng.integers(100, 150, size=(M, K // 32)).astype(np.uint8)
        sb = rng.integers(100, 150, size=(N, K // 32)).astype(np.uint8)
    C, A = O.gemm_reference(qa, sa, qb, sb, mode, fmt_a=fa_, fmt_b=fb_)
    Ce, Ae = _exact_gemm(qa, sa, qb, sb, mode, fa_, fb_)
    for m in range(M):
        for n in range(N):
            # float64 sums of terms spanning ~75 binades: K roundings at most
            assert abs(Fraction(C[m, n]) - Ce[m, n]) <= Fraction(2) ** -46 * Ae[m, n]
            assert abs(Fraction(A[m, n]) - Ae[m, n]) <= Fraction(2) ** -46 * Ae[m, n]


def test_e5m2_operand_swaps_formats_consistently():
    """Transposition symmetry: C(A:e4m3, B:e5m2) = C(B:e5m2, A:e4m3)^T."""
    rng = np.random.default_rng(31)
    qa, qb = _rand_codes_fmt(rng, (6, 96), "e4m3"), _rand_codes_fmt(rng, (5, 96), "e5m2")
    sa = rng.uniform(0.1, 2, 6).astype(np.float32)
    sb = rng.uniform(0.1, 2, 5).astype(np.float32)
    C1, A1 = O.gemm_reference(qa, sa, qb, sb, "rowwise", fmt_a="e4m3", fmt_b="e5m2")
    C2, A2 = O.gemm_reference(qb, sb, qa, sa, "rowwise", fmt_a="e5m2", fmt_b="e4m3")
    assert np.allclose(C1, C2.T, rtol=1e-14, atol=0) and np.allclose(A1, A2.T, rtol=1e-14)
    # and the wrong format assignment gives a different answer (the pin can see it)
    C3, _ = O.gemm_reference(qa, sa, qb, sb, "rowwise", fmt_a="e4m3", fmt_b="e4m3")
    assert not np.allclose(C1, C3)


# ---- fused epilogue -----------------------------------------------------------

def test_activation_closed_forms():
    y = np.array([-2.0, -1.0, 0.0, 1.0, 2.0])
    assert np.array_equal(O.activation(y, "none"), y)
    assert np.array_equal(O.activation(y, "relu"), [0, 0, 0, 1, 2])
    # GELU(y) = y * Phi(y): Phi(1) = 0.8413447460685429, Phi(2) = 0.9772498680518208
    g = O.activation(y, "gelu")
    assert abs(g[3] - 0.8413447460685429) < 1e-15 and abs(g[4] - 2 * 0.9772498680518208) < 1e-15
    assert abs(g[1] + 0.15865525393145707) < 1e-15 and g[2] == 0
    # SiLU(1) = 1 / (1 + e^-1)
    s = O.activation(y, "silu")
    assert abs(s[3] - 1 / (1 + np.exp(-1.0))) < 1e-15 and s[2] == 0
    # odd-part identities: act(y) - act(-y) = y for GELU and SiLU
    x = np.linspace(-30, 30, 2001)
    for act in ("gelu", "silu", "relu"):
        assert np.allclose(O.activation(x, act) - O.activation(-x, act), x, rtol=0, atol=1e-12)
    # large negative inputs go to (signed) zero, large positive ones to y
    assert O.activation(np.array([-800.0]), "silu")[0] == 0.0
    assert O.activation(np.array([-40.0]), "gelu")[0] == 0.0
    assert O.activation(np.array([40.0]), "gelu")[0] == 40.0


def test_activation_lipschitz_bounds():
    x = np.linspace(-20, 20, 400001)
    for act, L in O.ACT_LIPSCHITZ.items():
        d = np.abs(np.diff(O.activation(x, act)) / np.diff(x))
        assert d.max() <= L, (act, d.max())
        if act in ("gelu", "silu"):
            assert d.max() > L - 0.002, (act, d.max())       # and the bound is tight


def test_epilogue_reference_bias_and_identity():
    rng = np.random.default_rng(41)
    qa, qb = _rand_codes(rng, (8, 64)), _rand_codes(rng, (12, 64))
    sa = rng.uniform(0.1, 1, 8).astype(np.float32)
    sb = rng.uniform(0.1, 1, 12).astype(np.float32)
    C, A = O.gemm_reference(qa, sa, qb, sb, "rowwise")
    out, y = O.epilogue_reference(C, A, None, "none")
    assert np.array_equal(out, C) and np.array_equal(y, C)
    bias = rng.standard_normal(12).astype(np.float32)
    out, y = O.epilogue_reference(C, A, bias, "none")
    assert np.array_equal(out, C + bias.astype(np.float64)[None, :])
    out, y = O.epilogue_reference(C, A, bias, "relu")
    assert np.array_equal(out, np.maximum(C + bias.astype(np.float64)[None, :], 0))
    # a column selection picks the matching bias entries
    cols = np.array([3, 7, 11])
    Cs, As = O.gemm_reference(qa, sa, qb, sb, "rowwise", cols=cols)
    outs, _ = O.epilogue_reference(Cs, As, bias, "gelu", cols=cols)
    full, _ = O.epilogue_reference(C, A, bias, "gelu")
    assert np.array_equal(outs, full[:, cols])


@pytest.mark.parametrize("act", ["relu", "gelu", "silu"])
def test_epilogue_tolerance_rejects_planted_mistakes(act):
    """The bound accepts the correctly rounded result and rejects a dropped bias,
    a wrong activation and a bias applied to the wrong column."""
    rng = np.random.default_rng(["relu", "gelu", "silu"].index(act) + 50)
    qa, qb = _rand_codes(rng, (16, 128)), _rand_codes(rng, (24, 128))
    sa, sb = np.float32(0.02), np.float32(0.03)
    C, A = O.gemm_reference(qa, sa, qb, sb, "tensor")
    bias = (rng.standard_normal(24) * np.abs(C).mean()).astype(np.float32)
    out, y = O.epilogue_reference(C, A, bias, act)
    tol = O.epilogue_tolerance(out, y, A, act, "bf16")
    good = O.round_to_output(out, "bf16")
    assert np.all(np.abs(good - out) <= tol)
    for bad in (O.activation(C, act),                                   # bias dropped
                O.activation(y, "none" if act != "relu" else "silu"),   # wrong activation
                O.activation(C + bias[::-1].astype(np.float64), act)):   # bias columns reversed
        assert np.any(np.abs(O.round_to_output(bad, "bf16") - out) > tol)
