"""GPU parity of MXFP6 (e2m3 / e3m2 elements with E8M0 block scales).

* Quantisation: packed FP6 codes (four in three bytes) and E8M0 codes bit-exact
  against the oracle on ragged shapes, on the block-scaled workload distribution
  and on adversarial values (every midpoint of the format's grid and its binary32
  neighbours at several block exponents, saturation, all-zero blocks, signed
  zeros).
* GEMM, FP6 x FP6 in every pairing of e2m3 and e3m2: ragged M and N (edge rows),
  several tiles, both output types, the fused bias + activation epilogue and the
  output quantised for the next layer, against the oracle's bound.
"""
import numpy as np
import pytest
import torch

import block_scaled_gemm_fp8gemm_amd as F
import oracle as O
from oracle import quant as Q
from workloads import random_inputs

from gpu_support import DEV, announce, scale_to_dev, to_dev, to_host

pytestmark = pytest.mark.gpu

FP6 = ["e2m3", "e3m2"]
TOP = {"e2m3": 7.5, "e3m2": 28.0}


def _check_quant(x, fmt, what):
    announce("quantize", fmt, what, x.shape)
    q, s = F.quantize(to_dev(x, pad_cols_to=16), "mx32", fmt=fmt)
    torch.cuda.synchronize()
    qr, sr = Q.quantize_mx(x, fmt)
    pr = O.pack_fp6(qr)
    qg = to_host(q)
    assert qg.shape == pr.shape
    mism = np.argwhere(qg != pr)
    if mism.size:
        r, b = mism[0]
        raise AssertionError(f"{what}: {len(mism)} byte mismatches, first at row {r} byte {b}: "
                             f"x={x[r, b // 3 * 4:b // 3 * 4 + 4]!r} gpu={qg[r, b]:#04x} "
                             f"ref={pr[r, b]:#04x}")
    assert np.array_equal(to_host(s), sr), f"{what}: E8M0 codes differ"


@pytest.mark.parametrize("fmt", FP6)
@pytest.mark.parametrize("shape", [(1, 32), (3, 64), (257, 4128), (5, 14336), (64, 96)])
def test_quantize_fp6_random(fmt, shape):
    rows, k = shape
    x, _ = random_inputs(rows, 1, k, seed=rows * 7 + k, dist="mx_block")
    _check_quant(x, fmt, f"random{shape}")


def _adversarial_block_rows(fmt, k):
    """Rows of 32-blocks whose maximum is the format's largest value times 2^j:
    the other 31 values are grid points, midpoints, their fp32 neighbours,
    saturating values and zeros of both signs."""
    pos = O.FORMATS[fmt]["decode"](np.arange(32, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    vals = [pos, mids]
    for c in (pos[1:], mids):
        u = c.astype(np.float32).view(np.uint32).astype(np.int64)
        vals += [(u + 1).astype(np.uint32).view(np.float32), (u - 1).astype(np.uint32).view(np.float32)]
    top = TOP[fmt]
    v = np.concatenate([np.asarray(a, np.float64) for a in vals] +
                       [[top * 1.01, top * 1.06, 0.0, top / 1000]])
    v = np.concatenate([v, -v, [-0.0]])
    rows = []
    rng = np.random.default_rng(3)
    for j in (-3, 0, 5):
        row = np.resize(rng.permutation(v), k).astype(np.float32).reshape(-1, 32)
        row[:, 0] = top                       # block maximum: shared exponent 0
        row = row * np.float32(2.0 ** j)      # shifted binades: exponent j
        row[1] = 0.0                          # an all-zero block
        row[2, 1:] = -0.0
        rows.append(row.reshape(-1))
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("fmt", FP6)
def test_quantize_fp6_adversarial(fmt):
    _check_quant(_adversarial_block_rows(fmt, 4096), fmt, "adversarial")


def _operands(M, N, K, fa, fb, seed, dist="mx_block"):
    A, B = random_inputs(M, N, K, seed, dist)
    qa, sa = Q.quantize_mx(A, fa)
    qb, sb = Q.quantize_mx(B, fb)
    return qa, sa, qb, sb


def _run(qa, sa, qb, sb, fa, fb, out="bf16", bias=None, act="none"):
    bd = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(DEV)
    return F.gemm(to_dev(O.pack_fp6(qa), 16), scale_to_dev(sa, "mx32"),
                  to_dev(O.pack_fp6(qb), 16), scale_to_dev(sb, "mx32"), "mx32", out,
                  fmt_a=fa, fmt_b=fb, bias=bd, activation=act)


def _assert(C, Cr, Ar, out, what, bias=None, act="none", cols=None):
    o_ref, y_ref = O.epilogue_reference(Cr, Ar, bias, act, cols=cols)
    tol = O.epilogue_tolerance(o_ref, y_ref, Ar, act, out)
    bad = np.argwhere(np.abs(C - o_ref) > tol)
    assert bad.size == 0, f"{what}: {len(bad)} of {C.size} outside the bound, first " \
                          f"{tuple(bad[0])}: gpu={C[tuple(bad[0])]!r} ref={o_ref[tuple(bad[0])]!r}"
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"


@pytest.mark.parametrize("fa,fb", [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2"),
                                   ("e3m2", "e2m3")])
@pytest.mark.parametrize("out,shape", [("bf16", (1, 1, 128)), ("f16", (33, 70, 128)),
                                       ("bf16", (128, 128, 256)), ("bf16", (257, 263, 640)),
                                       ("f16", (300, 520, 1024)), ("bf16", (64, 300, 1152))])
def test_gemm_fp6(fa, fb, out, shape):
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, fa, fb, seed=M + 5 * N + K)
    assert F.fp8gemm_run_path(M, N, K, K * 3 // 4, K * 3 // 4, F.FORMATS[fa], F.FORMATS[fb],
                              2, 0) == "tile128"
    announce("gemm fp6", fa, fb, out, shape)
    C = to_host(_run(qa, sa, qb, sb, fa, fb, out))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a=fa, fmt_b=fb)
    _assert(C, Cr, Ar, out, f"{fa}x{fb} {out} {shape}")


@pytest.mark.parametrize("fmt", FP6)
def test_gemm_fp6_many_tiles_sampled(fmt):
    """64 tiles and a K of 4096 (32 code groups): sampled 128 x 128 blocks."""
    M, N, K = 1024, 1024, 4096
    qa, sa, qb, sb = _operands(M, N, K, fmt, fmt, seed=77)
    announce("gemm fp6 sampled", fmt, (M, N, K))
    C = _run(qa, sa, qb, sb, fmt, fmt)
    torch.cuda.synchronize()
    for r0, c0 in ((0, 0), (896, 896), (384, 640), (512, 128)):
        ri, ci = np.arange(r0, r0 + 128), np.arange(c0, c0 + 128)
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", rows=ri, cols=ci, fmt_a=fmt, fmt_b=fmt)
        _assert(to_host(C[r0:r0 + 128, c0:c0 + 128]), Cr, Ar, "bf16",
                f"{fmt} {(M, N, K)} block {(r0, c0)}")


@pytest.mark.parametrize("act", ["relu", "gelu", "silu"])
def test_gemm_fp6_fused_epilogue(act):
    M, N, K = 257, 263, 640
    qa, sa, qb, sb = _operands(M, N, K, "e2m3", "e3m2", seed=9)
    bias = np.random.default_rng(N).standard_normal(N).astype(np.float32) * 4
    announce("gemm fp6 epilogue", act)
    C = to_host(_run(qa, sa, qb, sb, "e2m3", "e3m2", "bf16", bias=bias, act=act))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a="e2m3", fmt_b="e3m2")
    _assert(C, Cr, Ar, "bf16", f"fp6 {act}", bias=bias, act=act)


def test_gemm_fp6_quantised_output():
    M, N, K = 200, 256, 512
    qa, sa, qb, sb = _operands(M, N, K, "e3m2", "e3m2", seed=12)
    announce("gemm fp6 mxout")
    q, c = F.gemm_mxout(to_dev(O.pack_fp6(qa), 16), scale_to_dev(sa, "mx32"),
                        to_dev(O.pack_fp6(qb), 16), scale_to_dev(sb, "mx32"), "mx32",
                        fmt_a="e3m2", fmt_b="e3m2")
    torch.cuda.synchronize()
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a="e3m2", fmt_b="e3m2")
    tol = O.tolerance(Cr, Ar, "bf16") - O.output_ulp(Cr, "bf16")
    ok = O.mx_output_within_bound(to_host(q), to_host(c), Cr, tol)
    assert ok.all(), f"{int((~ok).sum())} quantised outputs outside the bound"


@pytest.mark.parametrize("fa,fb", [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2")])
@pytest.mark.parametrize("shape", [(4096, 4096, 1024), (4100, 4160, 512)])
def test_gemm_fp6_large_tile_sampled(fa, fb, shape):
    """256 x 256 tiles (a tile per CU and more): full grid, and a grid cut by M
    and N; sampled 128 x 128 blocks, first, last, inner and edge ones."""
    M, N, K = shape
    assert F.fp8gemm_run_path(M, N, K, K * 3 // 4, K * 3 // 4, F.FORMATS[fa], F.FORMATS[fb],
                              2, 0) == "tile256"
    qa, sa, qb, sb = _operands(M, N, K, fa, fb, seed=M + N + K)
    announce("gemm fp6 256", fa, fb, shape)
    C = _run(qa, sa, qb, sb, fa, fb)
    torch.cuda.synchronize()
    for r0, c0 in ((0, 0), (M - 128, N - 128), (1920, 2176), (256 * 15, N - 80), (M - 20, 384)):
        ri = np.arange(r0, min(r0 + 128, M))
        ci = np.arange(c0, min(c0 + 128, N))
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", rows=ri, cols=ci, fmt_a=fa, fmt_b=fb)
        _assert(to_host(C[ri[0]:ri[-1] + 1, ci[0]:ci[-1] + 1]), Cr, Ar, "bf16",
                f"{fa}x{fb} {shape} block {(r0, c0)}")


@pytest.mark.parametrize("act", ["none", "gelu"])
def test_gemm_fp6_large_tile_fused(act):
    """The fused epilogue (bias, activation) and f16 output on 256 x 256 tiles,
    over a whole output with cut tiles."""
    M, N, K = 4128, 4096, 256
    qa, sa, qb, sb = _operands(M, N, K, "e2m3", "e3m2", seed=21)
    assert F.fp8gemm_run_path(M, N, K, K * 3 // 4, K * 3 // 4, F.FORMATS["e2m3"],
                              F.FORMATS["e3m2"], 2, 1) == "tile256"
    bias = np.random.default_rng(22).standard_normal(N).astype(np.float32)
    announce("gemm fp6 256 fused", act)
    C = to_host(_run(qa, sa, qb, sb, "e2m3", "e3m2", "f16", bias=bias, act=act))
    rows = np.concatenate([np.arange(0, 64), np.arange(M - 96, M)])
    cols = np.concatenate([np.arange(0, 64), np.arange(N - 64, N)])
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", rows=rows, cols=cols, fmt_a="e2m3",
                              fmt_b="e3m2")
    _assert(C[np.ix_(rows, cols)], Cr, Ar, "f16", f"fp6 256 {act}", bias=bias, act=act, cols=cols)
