"""GPU parity of the e5m2 operand format and the fused epilogue.

* e5m2 quantisation, every mode: codes and scales bit-exact against the oracle on
  ragged shapes and on adversarial values (every e5m2 midpoint and its binary32
  neighbours, the saturation range, zeros).
* GEMMs with e5m2 x e5m2 and mixed e4m3 x e5m2 operands, every mode, on ragged
  small shapes (edge path), full-tile shapes (interior path, sampled blocks) and a
  split-K shape, against the oracle's bound.
* The fused bias + activation epilogue on the same paths (staged and direct
  epilogues, split-K reduction), against the oracle's epilogue bound.
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

MODES = ["tensor", "rowwise", "mx32"]


def _check_quant(x, mode, what, pad=16):
    announce("quantize e5m2", what, mode, x.shape)
    q, s = F.quantize(to_dev(x, pad_cols_to=pad), mode, fmt="e5m2")
    torch.cuda.synchronize()
    qr, sr = Q.quantize(x, mode, "e5m2")
    qg = to_host(q)
    mism = np.argwhere(qg != qr)
    assert mism.size == 0, f"{what} {mode}: {len(mism)} code mismatches, first {tuple(mism[0])} " \
                           f"x={x[tuple(mism[0])]!r} gpu={qg[tuple(mism[0])]:#x} ref={qr[tuple(mism[0])]:#x}"
    sg = to_host(s)
    if mode == "mx32":
        assert np.array_equal(sg, sr)
    else:
        assert np.array_equal(sg.reshape(-1).view(np.uint32),
                              np.asarray(sr, np.float32).reshape(-1).view(np.uint32))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(1, 32), (3, 64), (257, 4128), (5, 14336)])
def test_quantize_e5m2_random(mode, shape):
    rows, k = shape
    x, _ = random_inputs(rows, 1, k, seed=rows * 11 + k, dist="outlier")
    _check_quant(x, mode, f"random{shape}")


def _adversarial_row_e5m2(k):
    pos = O.E5M2_DECODE[:0x7C]
    mids = (pos[:-1] + pos[1:]) / 2
    vals = [pos, mids]
    for w in (1, 2):
        for c in (pos[1:], mids):
            u = c.astype(np.float32).view(np.uint32).astype(np.int64)
            vals.append((u + w).astype(np.uint32).view(np.float32).astype(np.float64))
            vals.append((u - w).astype(np.uint32).view(np.float32).astype(np.float64))
    v = np.concatenate(vals)
    v = v[(v > 0) & (v <= 57344)]
    v = np.concatenate([v, -v, [0.0, -0.0, 2.0 ** -17, -(2.0 ** -17), 1e-30]])
    v = np.resize(v, k).astype(np.float32)
    v[0] = 57344.0                    # amax = 57344 -> s = 1, so x/s = x exactly
    return v


def test_quantize_e5m2_adversarial():
    k = 2048
    x = np.stack([_adversarial_row_e5m2(k), -np.roll(_adversarial_row_e5m2(k), 5)])
    for mode in ("tensor", "rowwise"):
        _check_quant(x, mode, "adversarial")
    # MX: blocks whose maximum is 2^15 * 1.75 keep their values (scale 2^0 after
    # the -15 shift of a block maximum in [2^15, 2^16))
    _check_quant(x, "mx32", "adversarial")


def _operands(M, N, K, mode, fa, fb, seed, dist="mx_block"):
    A, B = random_inputs(M, N, K, seed, dist)
    qa, sa = Q.quantize(A, mode, fa)
    qb, sb = Q.quantize(B, mode, fb)
    return qa, sa, qb, sb


def _run(qa, sa, qb, sb, mode, out, fa, fb, bias=None, act="none"):
    bd = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(DEV)
    return F.gemm(to_dev(qa, 16), scale_to_dev(sa, mode), to_dev(qb, 16), scale_to_dev(sb, mode),
                  mode, out, fmt_a=fa, fmt_b=fb, bias=bd, activation=act)


def _assert_epilogue(C, Cr, Ar, bias, act, out, what, cols=None):
    o_ref, y_ref = O.epilogue_reference(Cr, Ar, bias, act, cols=cols)
    tol = O.epilogue_tolerance(o_ref, y_ref, Ar, act, out)
    err = np.abs(C - o_ref)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{what}: {len(bad)} outside the bound, first {tuple(bad[0])}: " \
                          f"gpu={C[tuple(bad[0])]!r} ref={o_ref[tuple(bad[0])]!r} " \
                          f"tol={tol[tuple(bad[0])]!r}"


FMTS = [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmts", FMTS)
@pytest.mark.parametrize("shape", [(33, 70, 64), (257, 263, 4160), (129, 1000, 96)])
def test_gemm_formats_small(mode, fmts, shape):
    M, N, K = shape
    fa, fb = fmts
    qa, sa, qb, sb = _operands(M, N, K, mode, fa, fb, seed=M + 3 * N + K)
    announce("gemm formats", fa, fb, mode, shape)
    C = to_host(_run(qa, sa, qb, sb, mode, "bf16", fa, fb))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode, fmt_a=fa, fmt_b=fb)
    _assert_epilogue(C, Cr, Ar, None, "none", "bf16", f"{fa}x{fb} {mode} {shape}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fmts", FMTS)
def test_gemm_formats_interior_and_splitk(mode, fmts):
    fa, fb = fmts
    for M, N, K in ((2048, 4096, 512), (128, 4096, 4096)):     # interior tiles; split-K
        qa, sa, qb, sb = _operands(M, N, K, mode, fa, fb, seed=N + K + len(fa + fb))
        announce("gemm formats", fa, fb, mode, (M, N, K))
        C = _run(qa, sa, qb, sb, mode, "bf16", fa, fb)
        torch.cuda.synchronize()
        rng = np.random.default_rng(K)
        blocks = [(0, 0), (M - 128, N - 128)] + [
            (int(r) * 128, int(c) * 128) for r, c in rng.integers(0, [M // 128, N // 128], (3, 2))]
        for r0, c0 in blocks:
            ri, ci = np.arange(r0, r0 + 128), np.arange(c0, c0 + 128)
            Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode, rows=ri, cols=ci, fmt_a=fa,
                                      fmt_b=fb)
            _assert_epilogue(to_host(C[r0:r0 + 128, c0:c0 + 128]), Cr, Ar, None, "none", "bf16",
                             f"{fa}x{fb} {mode} {(M, N, K)} block {(r0, c0)}")


@pytest.mark.parametrize("act", ["none", "relu", "gelu", "silu"])
@pytest.mark.parametrize("mode,out,shape", [
    ("rowwise", "bf16", (257, 263, 4160)),    # edge tiles: staged epilogue
    ("tensor", "f16", (1024, 1024, 512)),     # full 128 x 128 tiles: direct epilogue
    ("mx32", "bf16", (4096, 4096, 512)),      # 256 x 256 tiles: direct epilogue
    ("tensor", "bf16", (128, 4096, 4096)),    # split-K reduction epilogue
])
def test_gemm_fused_epilogue(act, mode, out, shape):
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, mode, "e4m3", "e4m3", seed=M * 5 + N + K)
    rng = np.random.default_rng(N + K)
    # a bias of the size of the outputs (well above the bound, so a dropped or
    # misplaced bias fails), and the activation sees both signs
    c0, _ = O.gemm_reference(qa, sa, qb, sb, mode, rows=np.arange(min(M, 64)),
                             cols=np.arange(min(N, 64)))
    bias = (rng.standard_normal(N) * float(np.std(c0))).astype(np.float32)
    announce("gemm epilogue", act, mode, out, shape)
    C = _run(qa, sa, qb, sb, mode, out, "e4m3", "e4m3", bias=bias, act=act)
    torch.cuda.synchronize()
    if M * N <= 300 * 300:
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
        _assert_epilogue(to_host(C), Cr, Ar, bias, act, out, f"{act} {mode} {shape}")
        return
    for r0, c0 in ((0, 0), (M - 128, N - 128), (M // 2 - 64, N // 3)):
        r0 = max(0, min(r0, M - 128))
        ri, ci = np.arange(r0, r0 + 128), np.arange(c0, c0 + 128)
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode, rows=ri, cols=ci)
        _assert_epilogue(to_host(C[r0:r0 + 128, c0:c0 + 128]), Cr, Ar, bias, act, out,
                         f"{act} {mode} {shape} block {(r0, c0)}", cols=ci)


def test_gemm_fused_epilogue_e5m2_mixed():
    """Formats and epilogue together (the gradient-GEMM pairing with a bias)."""
    M, N, K = 300, 520, 384
    qa, sa, qb, sb = _operands(M, N, K, "rowwise", "e4m3", "e5m2", seed=77)
    bias = np.random.default_rng(78).standard_normal(N).astype(np.float32)
    announce("gemm epilogue mixed formats")
    C = to_host(_run(qa, sa, qb, sb, "rowwise", "bf16", "e4m3", "e5m2", bias=bias, act="silu"))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "rowwise", fmt_a="e4m3", fmt_b="e5m2")
    _assert_epilogue(C, Cr, Ar, bias, "silu", "bf16", "mixed silu")
