"""GPU parity of the dense GEMM with B in row-major [K, N] layout (N contiguous).

The oracle's B is [N, K]; the GPU gets its transpose (and, for MX, the transposed
codes [K/32, N]) through fp8gemm_run_kn.  Two forms: shapes with K % 128 == 0
(MX: K % 512 == 0, N % 16 == 0) are read row-major by the GEMM kernels
themselves (transposing LDS reads), the others are made K-contiguous first.
Both are checked against the oracle on ragged shapes, full tiles (sampled
blocks), split-K shapes, every e4m3 / e5m2 pairing and fused epilogues; the
in-kernel form must also equal the K-contiguous GEMM bit for bit where the two
run the same tile path (same products, same order).
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


def _run_nk(qa, sa, qb, sb, mode, out="bf16", fb="e4m3", bias=None, act="none"):
    bd = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(DEV)
    return F.gemm(to_dev(qa, 16), scale_to_dev(sa, mode), to_dev(qb, 16), scale_to_dev(sb, mode),
                  mode, out, fmt_b=fb, bias=bd, activation=act)


def _kn_path(M, N, K, mode, fb="e4m3"):
    return F.fp8gemm_run_kn_path(M, N, K, (K + 15) // 16 * 16, (N + 15) // 16 * 16,
                                 F.FORMATS["e4m3"], F.FORMATS[fb], F.SCALE_MODES[mode])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out,shape,path", [
    ("bf16", (300, 528, 512), "tile128"),         # edge tiles in M and N
    ("f16", (128, 256, 512), "tile128"),          # one row of full tiles
    ("bf16", (300, 528, 1024), "splitk"),         # ragged split tiles
    ("bf16", (100, 2000, 4096), "splitk"),
    ("f16", (64, 1024, 8192), "splitk"),
])
def test_gemm_row_major_b_in_kernel(mode, out, shape, path):
    M, N, K = shape
    assert _kn_path(M, N, K, mode) == path
    qa, sa, qb, sb = _operands(M, N, K, mode, seed=7 * M + N + K)
    announce("gemm row-major B in-kernel", mode, out, shape, path)
    C = to_host(_run_kn(qa, sa, qb, sb, mode, out))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
    assert_within_bound(C, Cr, Ar, out, f"row-major B in-kernel {mode}/{out}/{shape}")
    Cn = to_host(_run_nk(qa, sa, qb, sb, mode, out))
    assert F.fp8gemm_run_path(M, N, K, (K + 15) // 16 * 16, (K + 15) // 16 * 16, 0, 0,
                              F.SCALE_MODES[mode], 0) == path
    diff = np.argwhere(C != Cn)
    assert diff.size == 0, (f"in-kernel row-major B differs from the K-contiguous GEMM "
                            f"({mode}, {shape}) at {len(diff)} outputs, first {tuple(diff[0])}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(4096, 4096, 512), (4352, 4160, 512)])
def test_gemm_row_major_b_in_kernel_large_tile(mode, shape):
    """256 x 256 tiles read row-major: all full tiles, and a grid cut by N (and
    full in M); sampled 128 x 128 blocks, first, last and edge ones."""
    M, N, K = shape
    assert _kn_path(M, N, K, mode) == "tile256"
    qa, sa, qb, sb = _operands(M, N, K, mode, seed=M + N)
    announce("gemm row-major B in-kernel 256", mode, shape)
    C = _run_kn(qa, sa, qb, sb, mode)
    torch.cuda.synchronize()
    for r0, c0 in ((0, 0), (M - 128, N - 128), (2048, 1024), (256 * 7, N - 64)):
        ri = np.arange(r0, min(r0 + 128, M))
        ci = np.arange(c0, min(c0 + 128, N))
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode, rows=ri, cols=ci)
        assert_within_bound(to_host(C[ri[0]:ri[-1] + 1, ci[0]:ci[-1] + 1]), Cr, Ar, "bf16",
                            f"row-major B in-kernel 256 {mode} block {(r0, c0)}")


@pytest.mark.parametrize("fa,fb", [("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("mode", MODES)
def test_gemm_row_major_b_in_kernel_formats(fa, fb, mode):
    M, N, K = 192, 400, 512
    A, B = random_inputs(M, N, K, 31, "mx_block")
    qa, sa = Q.quantize(A, mode, fa)
    qb, sb = Q.quantize(B, mode, fb)
    assert F.fp8gemm_run_kn_path(M, N, K, K, (N + 15) // 16 * 16, F.FORMATS[fa], F.FORMATS[fb],
                                 F.SCALE_MODES[mode]) == "tile128"
    announce("gemm row-major B in-kernel formats", fa, fb, mode)
    qb_kn = to_dev(np.ascontiguousarray(qb.T), 16)
    sb_d = (torch.from_numpy(np.ascontiguousarray(np.asarray(sb, np.uint8).T)).to(DEV)
            if mode == "mx32" else scale_to_dev(sb, mode))
    C = to_host(F.gemm(to_dev(qa, 16), scale_to_dev(sa, mode), qb_kn, sb_d, mode, "bf16",
                       fmt_a=fa, fmt_b=fb, b_layout="kn"))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode, fmt_a=fa, fmt_b=fb)
    assert_within_bound(C, Cr, Ar, "bf16", f"row-major B in-kernel {fa}x{fb} {mode}")


@pytest.mark.parametrize("act", ["relu", "gelu", "silu"])
def test_gemm_row_major_b_in_kernel_fused(act):
    M, N, K = 300, 528, 512
    qa, sa, qb, sb = _operands(M, N, K, "mx32", seed=17)
    bias = np.random.default_rng(18).standard_normal(N).astype(np.float32) * 2
    assert _kn_path(M, N, K, "mx32") == "tile128"
    announce("gemm row-major B in-kernel fused", act)
    C = to_host(_run_kn(qa, sa, qb, sb, "mx32", bias=bias, act=act))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32")
    o_ref, y_ref = O.epilogue_reference(Cr, Ar, bias, act)
    tol = O.epilogue_tolerance(o_ref, y_ref, Ar, act, "bf16")
    bad = np.argwhere(np.abs(C - o_ref) > tol)
    assert bad.size == 0, f"{act}: {len(bad)} outside the bound, first {tuple(bad[0])}"


def test_gemm_row_major_b_in_kernel_wide_pitch():
    """B rows (K-rows) with a pitch well past N, and codes of MX rows of N."""
    M, N, K = 256, 384, 512
    for mode in MODES:
        qa, sa, qb, sb = _operands(M, N, K, mode, seed=44)
        buf = torch.zeros((K, N + 208), dtype=torch.uint8, device=DEV)
        buf[:, :N] = torch.from_numpy(np.ascontiguousarray(qb.T)).to(DEV)
        qb_kn = buf[:, :N]
        assert F.fp8gemm_run_kn_path(M, N, K, K, N + 208, 0, 0, F.SCALE_MODES[mode]) == "tile128"
        sb_d = (torch.from_numpy(np.ascontiguousarray(np.asarray(sb, np.uint8).T)).to(DEV)
                if mode == "mx32" else scale_to_dev(sb, mode))
        announce("gemm row-major B in-kernel wide pitch", mode)
        C = to_host(F.gemm(to_dev(qa, 16), scale_to_dev(sa, mode), qb_kn, sb_d, mode, "bf16",
                           b_layout="kn"))
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
        assert_within_bound(C, Cr, Ar, "bf16", f"row-major B wide pitch {mode}")


def _fp4_operands(M, N, K, seed):
    A, B = random_inputs(M, N, K, seed, "mx_block")
    qa, sa = Q.quantize(A, "mx32", "e2m1")
    qb, sb = Q.quantize(B, "mx32", "e2m1")
    return qa, sa, qb, sb


@pytest.mark.parametrize("shape,path", [((33, 70, 64), "none"), ((257, 262, 4160), "none"),
                                        ((128, 4096, 4096), "splitk"),
                                        ((512, 1024, 2048), "splitk"),
                                        ((2048, 1024, 2048), "tile128"),
                                        ((300, 528, 1024), "tile128"),
                                        ((100, 2000, 4096), "splitk")])
def test_gemm_row_major_b_fp4(shape, path):
    """MXFP4 with B row-major: the oracle's [N, K] codes transposed to [K, N] and
    packed two per byte along N (low nibble first).  With K % 512 == 0 and N % 16
    == 0 the GEMM kernels read them as they are (ds_read_b64_tr_b4), else the
    library nibble-transposes them into K-contiguous FP4 rows first; either way
    the products and their order are those of the K-contiguous FP4 GEMM."""
    M, N, K = shape
    qa, sa, qb, sb = _fp4_operands(M, N, K, seed=M + 3 * N + K)
    announce("gemm row-major B fp4", shape, path)
    qb_kn = O.pack_fp4(np.ascontiguousarray(qb.T))                 # [K, N/2]
    ldb = (N // 2 + 15) // 16 * 16
    assert F.fp8gemm_run_kn_path(M, N, K, (K // 2 + 15) // 16 * 16, ldb, F.FORMATS["e2m1"],
                                 F.FORMATS["e2m1"], F.SCALE_MODES["mx32"]) == path
    C = F.gemm(to_dev(O.pack_fp4(qa), 16), scale_to_dev(sa, "mx32"), to_dev(qb_kn, 16),
               torch.from_numpy(np.ascontiguousarray(np.asarray(sb, np.uint8).T)).to(DEV),
               "mx32", "bf16", fmt_a="e2m1", fmt_b="e2m1", b_layout="kn")
    torch.cuda.synchronize()
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a="e2m1", fmt_b="e2m1")
    assert_within_bound(to_host(C), Cr, Ar, "bf16", f"row-major B fp4 {shape}")
    # the same products as the K-contiguous FP4 GEMM, in the same order: equal bits
    Cnk = F.gemm(to_dev(O.pack_fp4(qa), 16), scale_to_dev(sa, "mx32"), to_dev(O.pack_fp4(qb), 16),
                 scale_to_dev(sb, "mx32"), "mx32", "bf16", fmt_a="e2m1", fmt_b="e2m1")
    assert torch.equal(C, Cnk)


@pytest.mark.parametrize("shape", [(4096, 4096, 512), (4352, 4160, 1024)])
def test_gemm_row_major_b_fp4_large_tile(shape):
    """MXFP4 row-major B on 256 x 256 tiles, full and cut by M and N (sampled
    128 x 128 blocks, and bit-equality with the K-contiguous FP4 GEMM where that
    takes the same tile path: it keeps cut shapes on 128 x 128 tiles)."""
    M, N, K = shape
    qa, sa, qb, sb = _fp4_operands(M, N, K, seed=K + 7)
    announce("gemm row-major B fp4 large tile", shape)
    assert F.fp8gemm_run_kn_path(M, N, K, K // 2, N // 2, F.FORMATS["e2m1"], F.FORMATS["e2m1"],
                                 F.SCALE_MODES["mx32"]) == "tile256"
    qad, sad = to_dev(O.pack_fp4(qa), 16), scale_to_dev(sa, "mx32")
    C = F.gemm(qad, sad, to_dev(O.pack_fp4(np.ascontiguousarray(qb.T)), 16),
               torch.from_numpy(np.ascontiguousarray(np.asarray(sb, np.uint8).T)).to(DEV),
               "mx32", "bf16", fmt_a="e2m1", fmt_b="e2m1", b_layout="kn")
    Cnk = F.gemm(qad, sad, to_dev(O.pack_fp4(qb), 16), scale_to_dev(sb, "mx32"), "mx32", "bf16",
                 fmt_a="e2m1", fmt_b="e2m1")
    torch.cuda.synchronize()
    for r0, c0 in ((0, 0), (M - 128, N - 128), (2048, 1024)):
        ri, ci = np.arange(r0, r0 + 128), np.arange(c0, c0 + 128)
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", rows=ri, cols=ci, fmt_a="e2m1",
                                  fmt_b="e2m1")
        assert_within_bound(to_host(C[r0:r0 + 128, c0:c0 + 128]), Cr, Ar, "bf16",
                            f"row-major B fp4 {shape} block {(r0, c0)}")
    if F.fp8gemm_run_path(M, N, K, K // 2, K // 2, F.FORMATS["e2m1"], F.FORMATS["e2m1"],
                          F.SCALE_MODES["mx32"], 0) == "tile256":
        assert torch.equal(C, Cnk)
