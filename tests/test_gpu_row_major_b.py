"""GPU parity of the dense GEMM with B in row-major [K, N] layout (N contiguous).

The oracle's B is [N, K]; the GPU gets its transpose (and, for MX, the transposed
codes [K/32, N]) through fp8gemm_run_kn, on ragged shapes (edge path), full
tiles (interior path, sampled blocks), a split-K shape and with e5m2 codes and a
fused epilogue.
"""
import numpy as np
import pytest
import torch

import block_scaled_gemm_fp8gemm_amd as F
import oracle as O
from oracle import quant as Q
from workloads import random_inputs

from gpu_support import DEV, announce, assert_within_bound, scale_to_dev, to_dev, to_host

pytestmark = pytest.mark.gpu

MODES = ["tensor", "rowwise", "mx32"]


def _operands(M, N, K, mode, seed, fb="e4m3"):
    A, B = random_inputs(M, N, K, seed, "mx_block")
    qa, sa = Q.quantize(A, mode)
    qb, sb = Q.quantize(B, mode, fb)
    return qa, sa, qb, sb


def _run_kn(qa, sa, qb, sb, mode, out="bf16", fb="e4m3", bias=None, act="none"):
    qb_kn = to_dev(np.ascontiguousarray(qb.T), 16)               # [K, N], padded row pitch
    if mode == "mx32":
        sb_d = torch.from_numpy(np.ascontiguousarray(np.asarray(sb, np.uint8).T)).to(DEV)
    else:
        sb_d = scale_to_dev(sb, mode)
    bd = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(DEV)
    return F.gemm(to_dev(qa, 16), scale_to_dev(sa, mode), qb_kn, sb_d, mode, out, fmt_b=fb,
                  bias=bd, activation=act, b_layout="kn")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out,shape", [("f16", (33, 70, 64)), ("bf16", (257, 263, 4160)),
                                       ("bf16", (129, 1000, 96)), ("bf16", (128, 4096, 4096))])
def test_gemm_row_major_b(mode, out, shape):
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, mode, seed=M + 5 * N + 3 * K)
    announce("gemm row-major B", mode, out, shape)
    C = to_host(_run_kn(qa, sa, qb, sb, mode, out))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
    assert_within_bound(C, Cr, Ar, out, f"row-major B {mode}/{out}/{shape}")


@pytest.mark.parametrize("mode", MODES)
def test_gemm_row_major_b_interior(mode):
    M, N, K = 2048, 4096, 1024
    qa, sa, qb, sb = _operands(M, N, K, mode, seed=91)
    announce("gemm row-major B interior", mode, (M, N, K))
    C = _run_kn(qa, sa, qb, sb, mode)
    torch.cuda.synchronize()
    for r0, c0 in ((0, 0), (M - 128, N - 128), (1024, 2048)):
        ri, ci = np.arange(r0, r0 + 128), np.arange(c0, c0 + 128)
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode, rows=ri, cols=ci)
        assert_within_bound(to_host(C[r0:r0 + 128, c0:c0 + 128]), Cr, Ar, "bf16",
                            f"row-major B interior {mode} block {(r0, c0)}")


def test_gemm_row_major_b_e5m2_fused():
    M, N, K = 300, 520, 384
    qa, sa, qb, sb = _operands(M, N, K, "rowwise", seed=93, fb="e5m2")
    bias = np.random.default_rng(94).standard_normal(N).astype(np.float32)
    announce("gemm row-major B e5m2 + bias + relu")
    C = to_host(_run_kn(qa, sa, qb, sb, "rowwise", fb="e5m2", bias=bias, act="relu"))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "rowwise", fmt_b="e5m2")
    o_ref, y_ref = O.epilogue_reference(Cr, Ar, bias, "relu")
    tol = O.epilogue_tolerance(o_ref, y_ref, Ar, "relu", "bf16")
    assert np.all(np.abs(C - o_ref) <= tol)


def test_row_major_b_shares_the_workspace_with_split_k():
    """Row-major-B calls and K-contiguous split-K calls of different shapes share the
    binding's one workspace: the copies of B never land on the split-K counters."""
    seq = [("nk", (128, 4096, 4096)), ("kn", (128, 8192, 2048)), ("nk", (128, 8192, 2048)),
           ("kn", (300, 260, 512)), ("nk", (64, 2048, 4096)), ("kn", (128, 4096, 4096))]
    for i, (layout, (M, N, K)) in enumerate(seq):
        qa, sa, qb, sb = _operands(M, N, K, "rowwise", seed=60 + i)
        announce("gemm shared workspace", layout, (M, N, K))
        if layout == "kn":
            C = to_host(_run_kn(qa, sa, qb, sb, "rowwise"))
        else:
            C = to_host(F.gemm(to_dev(qa, 16), scale_to_dev(sa, "rowwise"), to_dev(qb, 16),
                               scale_to_dev(sb, "rowwise"), "rowwise", "bf16"))
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "rowwise")
        assert_within_bound(C, Cr, Ar, "bf16", f"shared workspace {layout} {(M, N, K)}")
