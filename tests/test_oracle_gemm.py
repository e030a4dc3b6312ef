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


def _exact_value(code):
    return Fraction(O.E4M3_DECODE[int(code)])  # table values are exact dyadic rationals


def _exact_gemm(qa, sa, qb, sb, mode):
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
                t = fa * _exact_value(qa[m, k]) * fb * _exact_value(qb[n, k])
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
