"""GPU parity of the GEMM whose output is quantised for the next layer with a fresh
per-tensor or per-row scale (fp8gemm_run_qout): the GEMM kernels store the bf16
output exactly as fp8gemm_run_ex does and fold the stored values' magnitudes into
atomic maxima in their epilogue (registers on full tiles, the staged loops on
edge tiles and after the split-K reduction), a second kernel derives the scales
and encodes.  Every case is checked twice: bit for bit against the library's own
two-step path (the bf16 GEMM, then the quantiser on its output), and against the
oracle's bound (the GEMM bound plus the bf16 and format roundings at the scale;
the scale itself within the band the bound allows).  Covered: every input scale
mode, both output scale modes, e4m3 and e5m2 codes, ragged M, 256- and 128-wide
tiles, split-K, the persistent grid, bias + activation, FP4 and FP6 operands,
all-zero rows, workspace reuse across shapes, and the codes feeding a row-wise
GEMM as its A operand."""
import numpy as np
import pytest
import torch

import block_scaled_gemm_fp8gemm_amd as F
import oracle as O
from oracle import quant as Q
from workloads import random_inputs

from gpu_support import DEV, announce, scale_to_dev, to_dev, to_host

pytestmark = pytest.mark.gpu


def _operands(M, N, K, mode, fmt, seed, dist="mx_block"):
    A, B = random_inputs(M, N, K, seed, dist)
    qa, sa = Q.quantize(A, mode, fmt)
    qb, sb = Q.quantize(B, mode, fmt)
    return qa, sa, qb, sb


def _pack(fmt):
    if fmt == "e2m1":
        return O.pack_fp4
    if fmt in ("e2m3", "e3m2"):
        return O.pack_fp6
    return lambda a: a


def _run(qa, sa, qb, sb, mode, fmt, out_mode, cfmt="e4m3", bias=None, act="none",
         workspace=None, two_step=True):
    bd = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(DEV)
    ops = (to_dev(_pack(fmt)(qa), 16), scale_to_dev(sa, mode), to_dev(_pack(fmt)(qb), 16),
           scale_to_dev(sb, mode))
    q, s = F.gemm_qout(*ops, mode, out_mode, cfmt, fmt_a=fmt, fmt_b=fmt, bias=bd,
                       activation=act, workspace=workspace)
    torch.cuda.synchronize()
    q, s = to_host(q), to_host(s)
    if two_step:
        # the library's own path in two calls: bf16 GEMM, then the quantiser on C
        C = F.gemm(*ops, mode, "bf16", fmt_a=fmt, fmt_b=fmt, bias=bd, activation=act)
        q2, s2 = F.quantize(C.float().contiguous(), out_mode, fmt=cfmt)
        q2, s2 = to_host(q2), to_host(s2).reshape(s.shape)
        bad = np.argwhere(q != q2)
        assert bad.size == 0, f"{len(bad)} codes differ from quantize(gemm); first {tuple(bad[0])}"
        assert np.array_equal(s, s2), "scales differ from quantize(gemm)"
    return q, s


def _check(qa, sa, qb, sb, mode, fmt, out_mode, q, s, cfmt="e4m3", rows=None, bias=None,
           act="none", what=""):
    """Whole rows (``rows``, default all): a row's scale depends on all of it."""
    ri = np.arange(qa.shape[0]) if rows is None else np.asarray(rows)
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode, rows=ri, fmt_a=fmt, fmt_b=fmt)
    o_ref, y_ref = O.epilogue_reference(Cr, Ar, bias, act)
    tol = O.epilogue_tolerance(o_ref, y_ref, Ar, act, "bf16") - O.output_ulp(o_ref, "bf16")
    sg = s[ri] if out_mode == "rowwise" else s.reshape(())
    ok = O.scaled_output_within_bound(q[ri], sg, o_ref, tol, out_mode, cfmt)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        si = sg[i[0]] if out_mode == "rowwise" else sg
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outputs outside the bound;"
                             f" first {i}: code {q[ri][i]:#04x} scale {float(si)!r}"
                             f" ref {o_ref[i]!r} row max {np.abs(o_ref[i[0]]).max()!r}")
    assert np.all(np.isfinite(s)) and np.all(s > 0), f"{what}: scales not positive"


@pytest.mark.parametrize("mode", ["tensor", "rowwise", "mx32"])
@pytest.mark.parametrize("out_mode", ["rowwise", "tensor"])
@pytest.mark.parametrize("shape", [(33, 64, 64), (257, 288, 4160), (300, 256, 512)])
def test_qout_small(mode, out_mode, shape):
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, mode, "e4m3", seed=M + N + K)
    announce("gemm qout", mode, out_mode, shape)
    q, s = _run(qa, sa, qb, sb, mode, "e4m3", out_mode)
    assert q.shape == (M, N) and s.shape == ((M,) if out_mode == "rowwise" else (1,))
    _check(qa, sa, qb, sb, mode, "e4m3", out_mode, q, s, what=f"qout {mode} {out_mode} {shape}")


@pytest.mark.parametrize("mode", ["rowwise", "mx32"])
@pytest.mark.parametrize("out_mode", ["rowwise", "tensor"])
@pytest.mark.parametrize("shape", [(2048, 4096, 512), (512, 512, 1024), (128, 4096, 4096)])
def test_qout_interior_and_splitk(mode, out_mode, shape):
    """256 x 256 tiles, 128 x 128 tiles and the split-K reduction: whole sampled
    rows for row scales, the whole output for the one scale."""
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, mode, "e4m3", seed=N + K)
    announce("gemm qout", mode, out_mode, shape)
    q, s = _run(qa, sa, qb, sb, mode, "e4m3", out_mode)
    rows = None
    if out_mode == "rowwise":
        rng = np.random.default_rng(K)
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 30)]))
    _check(qa, sa, qb, sb, mode, "e4m3", out_mode, q, s, rows=rows,
           what=f"qout {mode} {out_mode} {shape}")


@pytest.mark.parametrize("fmt,act", [("e4m3", "gelu"), ("e2m1", "silu"), ("e2m3", "relu")])
@pytest.mark.parametrize("out_mode", ["rowwise", "tensor"])
def test_qout_bias_activation_fp4_fp6(fmt, act, out_mode):
    M, N, K = 257, 288, (4160 if fmt != "e2m3" else 4096)
    mode = "mx32"
    qa, sa, qb, sb = _operands(M, N, K, mode, fmt, seed=5)
    bias = np.random.default_rng(9).standard_normal(N).astype(np.float32) * 8
    announce("gemm qout fused", fmt, act, out_mode, (M, N, K))
    q, s = _run(qa, sa, qb, sb, mode, fmt, out_mode, bias=bias, act=act)
    _check(qa, sa, qb, sb, mode, fmt, out_mode, q, s, bias=bias, act=act,
           what=f"qout {fmt} bias+{act} {out_mode}")


@pytest.mark.parametrize("shape,fmt,out_mode",
                         [((1, 16, 64), "e4m3", "rowwise"), ((2, 32, 32), "e5m2", "tensor"),
                          ((130, 96, 160), "e5m2", "rowwise")])
def test_qout_e5m2_codes_and_degenerate(shape, fmt, out_mode):
    """e5m2 output codes (and e5m2 operands), a single row, the smallest N."""
    M, N, K = shape
    mode = "rowwise"
    qa, sa, qb, sb = _operands(M, N, K, mode, fmt, seed=M + 7 * N + K)
    announce("gemm qout e5m2", fmt, out_mode, shape)
    q, s = _run(qa, sa, qb, sb, mode, fmt, out_mode, cfmt="e5m2")
    _check(qa, sa, qb, sb, mode, fmt, out_mode, q, s, cfmt="e5m2",
           what=f"qout e5m2 {fmt} {out_mode} {shape}")


def test_qout_zero_rows_take_scale_one():
    """Rows of A that are all zero give zero rows of y: scale 1 and zero codes."""
    M, N, K = 200, 256, 512
    qa, sa, qb, sb = _operands(M, N, K, "rowwise", "e4m3", seed=3)
    qa[[0, 17, 199]] = 0
    announce("gemm qout zero rows", (M, N, K))
    q, s = _run(qa, sa, qb, sb, "rowwise", "e4m3", "rowwise")
    assert np.all(s[[0, 17, 199]] == 1.0) and not q[[0, 17, 199]].any()
    _check(qa, sa, qb, sb, "rowwise", "e4m3", "rowwise", q, s, what="qout zero rows")


def test_qout_workspace_reused_across_shapes():
    """One workspace for a split-K shape, a tiled shape and the split-K shape again:
    each result equals that of a call on a fresh zero-filled workspace."""
    shapes = [(128, 2048, 4096), (520, 1024, 512), (128, 2048, 4096)]
    need = max(F.fp8gemm_qout_workspace_size(M, N, K, 1) for M, N, K in shapes)
    shared = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, (M, N, K) in enumerate(shapes):
        qa, sa, qb, sb = _operands(M, N, K, "rowwise", "e4m3", seed=40 + i)
        for out_mode in ("rowwise", "tensor"):
            announce("gemm qout reuse", i, out_mode, (M, N, K))
            q1, s1 = _run(qa, sa, qb, sb, "rowwise", "e4m3", out_mode, workspace=shared)
            fresh = torch.zeros(F.fp8gemm_qout_workspace_size(M, N, K, 1), dtype=torch.uint8,
                                device=DEV)
            q2, s2 = _run(qa, sa, qb, sb, "rowwise", "e4m3", out_mode, workspace=fresh)
            assert np.array_equal(s1, s2) and np.array_equal(q1, q2), (i, out_mode)


def test_qout_feeds_a_rowwise_gemm():
    """The codes and their row scales are the A operand of a row-wise GEMM."""
    M, N, K, N2 = 256, 512, 1024, 384
    qa, sa, qb, sb = _operands(M, N, K, "mx32", "e4m3", seed=21)
    announce("gemm qout chain", (M, N, K, N2))
    q, s = _run(qa, sa, qb, sb, "mx32", "e4m3", "rowwise")
    W2 = random_inputs(1, N2, N, 22, "normal")[1]
    q2, s2 = Q.quantize(W2, "rowwise")
    C2 = F.gemm(to_dev(q, 16), scale_to_dev(s, "rowwise"), to_dev(q2, 16),
                scale_to_dev(s2, "rowwise"), "rowwise", "bf16")
    Cr, Ar = O.gemm_reference(q, s, q2, s2, "rowwise")      # from the GPU's own layer-1 codes
    ok = O.within_bound(to_host(C2), Cr, Ar, "bf16")
    assert ok.all(), f"{int((~ok).sum())} outputs of the second GEMM outside the bound"


@pytest.mark.parametrize("mode,out_mode", [("tensor", "tensor"), ("mx32", "rowwise")])
def test_qout_persistent_grid(mode, out_mode):
    """A shape with 2048 tiles of 256 x 256 takes the persistent copy-stream grid,
    whose register epilogue folds the maxima too (sampled rows against the
    oracle; every code against the two-step path)."""
    M, N, K = 16384, 8192, 512
    assert F.fp8gemm_run_path(M, N, K, K, K, 0, 0, F.SCALE_MODES[mode], 0) == "persistent"
    qa, sa, qb, sb = _operands(M, N, K, mode, "e4m3", seed=61)
    announce("gemm qout persistent", mode, out_mode, (M, N, K))
    q, s = _run(qa, sa, qb, sb, mode, "e4m3", out_mode)
    if out_mode == "rowwise":
        rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(1).integers(0, M, 24)]))
        _check(qa, sa, qb, sb, mode, "e4m3", out_mode, q, s, rows=rows,
               what=f"qout persistent {mode} {out_mode}")
