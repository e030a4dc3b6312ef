"""GPU parity of the GEMM whose output is quantised for the next layer
(fp8gemm_run_mxout): e4m3 codes with one E8M0 scale per 32 columns, produced by
the fused epilogue on the edge, interior (both tile sizes) and split-K paths, in
every scale mode, with and without bias + activation, and with FP4 operands.
Checked against the oracle's MX-output bound (the GEMM bound plus the e4m3
rounding at the block exponent)."""
import numpy as np
import pytest
import torch

import block_scaled_gemm_fp8gemm_amd as F
import oracle as O
from oracle import quant as Q
from workloads import random_inputs

from gpu_support import DEV, announce, scale_to_dev, to_dev, to_host

pytestmark = pytest.mark.gpu


def _check(qa, sa, qb, sb, mode, fmt, rows=None, cols=None, q=None, c=None, bias=None,
           act="none", what=""):
    ri = np.arange(qa.shape[0]) if rows is None else rows
    ci = np.arange(qb.shape[0]) if cols is None else cols
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode, rows=ri, cols=ci, fmt_a=fmt, fmt_b=fmt)
    o_ref, y_ref = O.epilogue_reference(Cr, Ar, bias, act, cols=ci)
    tol = O.epilogue_tolerance(o_ref, y_ref, Ar, act, "bf16") - O.output_ulp(o_ref, "bf16")
    qg = q[np.ix_(ri, ci)]
    cg = c[np.ix_(ri, ci[::32] // 32)]
    ok = O.mx_output_within_bound(qg, cg, o_ref, tol)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outputs outside the bound; "
                             f"first {i}: code {qg[i]:#04x} block code {cg[i[0], i[1] // 32]} "
                             f"ref {o_ref[i]!r}")


def _operands(M, N, K, mode, fmt, seed):
    A, B = random_inputs(M, N, K, seed, "mx_block")
    qa, sa = Q.quantize(A, mode, fmt)
    qb, sb = Q.quantize(B, mode, fmt)
    return qa, sa, qb, sb


def _run(qa, sa, qb, sb, mode, fmt, bias=None, act="none"):
    pack = O.pack_fp4 if fmt == "e2m1" else (lambda a: a)
    bd = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(DEV)
    q, c = F.gemm_mxout(to_dev(pack(qa), 16), scale_to_dev(sa, mode), to_dev(pack(qb), 16),
                        scale_to_dev(sb, mode), mode, fmt_a=fmt, fmt_b=fmt, bias=bd,
                        activation=act)
    torch.cuda.synchronize()
    return to_host(q), to_host(c)


@pytest.mark.parametrize("mode", ["tensor", "rowwise", "mx32"])
@pytest.mark.parametrize("shape", [(33, 64, 64), (257, 288, 4160), (300, 256, 512)])
def test_mxout_small(mode, shape):
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, mode, "e4m3", seed=M + N + K)
    announce("gemm mxout", mode, shape)
    q, c = _run(qa, sa, qb, sb, mode, "e4m3")
    assert q.shape == (M, N) and c.shape == (M, N // 32)
    _check(qa, sa, qb, sb, mode, "e4m3", q=q, c=c, what=f"mxout {mode} {shape}")


@pytest.mark.parametrize("mode", ["rowwise", "mx32"])
@pytest.mark.parametrize("shape", [(2048, 4096, 512), (512, 512, 1024), (128, 4096, 4096)])
def test_mxout_interior_and_splitk(mode, shape):
    """256 x 256 tiles, 128 x 128 tiles and the split-K reduction (sampled blocks)."""
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, mode, "e4m3", seed=N + K)
    announce("gemm mxout", mode, shape)
    q, c = _run(qa, sa, qb, sb, mode, "e4m3")
    rng = np.random.default_rng(K)
    for r0, c0 in [(0, 0), (M - 128, N - 128)] + [
            (int(r) * 128, int(cc) * 128) for r, cc in rng.integers(0, [M // 128, N // 128], (3, 2))]:
        _check(qa, sa, qb, sb, mode, "e4m3", rows=np.arange(r0, r0 + 128),
               cols=np.arange(c0, c0 + 128), q=q, c=c, what=f"mxout {mode} {shape} {(r0, c0)}")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_mxout_bias_activation_and_fp4(fmt):
    M, N, K = 257, 288, 4160
    qa, sa, qb, sb = _operands(M, N, K, "mx32", fmt, seed=5)
    bias = np.random.default_rng(9).standard_normal(N).astype(np.float32) * 8
    announce("gemm mxout fused", fmt, (M, N, K))
    q, c = _run(qa, sa, qb, sb, "mx32", fmt, bias, "gelu")
    _check(qa, sa, qb, sb, "mx32", fmt, q=q, c=c, bias=bias, act="gelu",
           what=f"mxout {fmt} bias+gelu")


def test_mxout_feeds_the_next_gemm():
    """The quantised output is the next GEMM's A operand (MX blocks along its K)."""
    M, N, K, N2 = 256, 512, 1024, 384
    qa, sa, qb, sb = _operands(M, N, K, "mx32", "e4m3", seed=21)
    announce("gemm mxout chain", (M, N, K, N2))
    q, c = _run(qa, sa, qb, sb, "mx32", "e4m3")
    W2 = random_inputs(1, N2, N, 22, "normal")[1]
    q2, s2 = Q.quantize(W2, "mx32")
    C2 = F.gemm(to_dev(q, 16), scale_to_dev(c, "mx32"), to_dev(q2, 16), scale_to_dev(s2, "mx32"),
                "mx32", "bf16")
    Cr, Ar = O.gemm_reference(q, c, q2, s2, "mx32")          # from the GPU's own layer-1 codes
    ok = O.within_bound(to_host(C2), Cr, Ar, "bf16")
    assert ok.all(), f"{int((~ok).sum())} outputs of the second GEMM outside the bound"


@pytest.mark.parametrize("shape,fmt", [((1, 32, 64), "e4m3"), ((2, 64, 32), "e5m2"),
                                       ((130, 96, 160), "e5m2")])
def test_mxout_degenerate_and_e5m2(shape, fmt):
    """One 32-column block, a single row, the smallest K, and e5m2 operands."""
    M, N, K = shape
    mode = "mx32"
    qa, sa, qb, sb = _operands(M, N, K, mode, fmt, seed=M + 7 * N + K)
    announce("gemm mxout degenerate", fmt, shape)
    q, c = _run(qa, sa, qb, sb, mode, fmt)
    _check(qa, sa, qb, sb, mode, fmt, q=q, c=c, what=f"mxout {fmt} {shape}")
