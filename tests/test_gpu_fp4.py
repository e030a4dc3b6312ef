"""GPU parity of MXFP4 (e2m1 elements with E8M0 block scales).

* Quantisation: packed e2m1 codes and E8M0 codes bit-exact against the oracle on
  ragged shapes, on the block-scaled workload distribution and on adversarial
  values (every e2m1 midpoint and its binary32 neighbours at several block
  exponents, saturation between 6 and 8, all-zero blocks, signed zeros).
* GEMM, MXFP4 x MXFP4: ragged shapes (edge tiles, K tails), full-tile shapes on
  both tile sizes (interior path, sampled 128 x 128 blocks), both output types and
  the fused bias + activation epilogue, against the oracle's bound.
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


def _check_quant(x, what):
    announce("quantize e2m1", what, x.shape)
    q, s = F.quantize(to_dev(x, pad_cols_to=16), "mx32", fmt="e2m1")
    torch.cuda.synchronize()
    qr, sr = Q.quantize_mx(x, "e2m1")
    pr = O.pack_fp4(qr)
    qg = to_host(q)
    assert qg.shape == pr.shape
    mism = np.argwhere(qg != pr)
    if mism.size:
        r, b = mism[0]
        raise AssertionError(f"{what}: {len(mism)} byte mismatches, first at row {r} byte {b}: "
                             f"x={x[r, 2 * b:2 * b + 2]!r} gpu={qg[r, b]:#04x} ref={pr[r, b]:#04x}")
    assert np.array_equal(to_host(s), sr), f"{what}: E8M0 codes differ"


@pytest.mark.parametrize("shape", [(1, 32), (3, 64), (257, 4128), (5, 14336), (64, 96)])
def test_quantize_fp4_random(shape):
    rows, k = shape
    x, _ = random_inputs(rows, 1, k, seed=rows * 7 + k, dist="mx_block")
    _check_quant(x, f"random{shape}")


def _adversarial_block_rows(k):
    """Rows of 32-blocks whose maximum is 6 * 2^j (so x * 2^-e lands on the e2m1 grid
    scaled by 2^j): the other 31 values are midpoints, their fp32 neighbours,
    grid points, saturating values in (6, 8) and zeros of both signs."""
    pos = O.E2M1_DECODE[:8]
    mids = (pos[:-1] + pos[1:]) / 2
    vals = [pos, mids]
    for c in (pos[1:], mids):
        u = c.astype(np.float32).view(np.uint32).astype(np.int64)
        vals += [(u + 1).astype(np.uint32).view(np.float32), (u - 1).astype(np.uint32).view(np.float32)]
    v = np.concatenate([np.asarray(a, np.float64) for a in vals] + [[6.5, 7.0, 7.99, 0.0, 0.1]])
    v = np.concatenate([v, -v, [-0.0]])
    rows = []
    rng = np.random.default_rng(3)
    for j in (-3, 0, 5):
        row = np.resize(rng.permutation(v), k).astype(np.float32).reshape(-1, 32)
        row[:, 0] = 6.0                       # block maximum 6: shared exponent 0
        row = row * np.float32(2.0 ** j)      # shifted binades: exponent j
        row[1] = 0.0                          # an all-zero block
        row[2, 1:] = -0.0
        rows.append(row.reshape(-1))
    return np.stack(rows).astype(np.float32)


def test_quantize_fp4_adversarial():
    _check_quant(_adversarial_block_rows(2048), "adversarial")


def _operands(M, N, K, seed, dist="mx_block"):
    A, B = random_inputs(M, N, K, seed, dist)
    qa, sa = Q.quantize_mx(A, "e2m1")
    qb, sb = Q.quantize_mx(B, "e2m1")
    return qa, sa, qb, sb


def _run(qa, sa, qb, sb, out="bf16", bias=None, act="none"):
    bd = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(DEV)
    return F.gemm(to_dev(O.pack_fp4(qa), 16), scale_to_dev(sa, "mx32"),
                  to_dev(O.pack_fp4(qb), 16), scale_to_dev(sb, "mx32"), "mx32", out,
                  fmt_a="e2m1", fmt_b="e2m1", bias=bd, activation=act)


def _assert(C, Cr, Ar, out, what, bias=None, act="none", cols=None):
    o_ref, y_ref = O.epilogue_reference(Cr, Ar, bias, act, cols=cols)
    tol = O.epilogue_tolerance(o_ref, y_ref, Ar, act, out)
    bad = np.argwhere(np.abs(C - o_ref) > tol)
    assert bad.size == 0, f"{what}: {len(bad)} of {C.size} outside the bound, first " \
                          f"{tuple(bad[0])}: gpu={C[tuple(bad[0])]!r} ref={o_ref[tuple(bad[0])]!r}"
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(33, 70, 64), (100, 72, 96), (257, 263, 4160),
                                   (129, 1000, 2080), (300, 260, 640), (300, 260, 512)])
def test_gemm_fp4_small(out, shape):
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, seed=M + 5 * N + K)
    announce("gemm e2m1", out, shape)
    C = to_host(_run(qa, sa, qb, sb, out))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a="e2m1", fmt_b="e2m1")
    _assert(C, Cr, Ar, out, f"e2m1 {out} {shape}")


@pytest.mark.parametrize("shape", [(512, 512, 1024), (4096, 4096, 1024), (4096, 4096, 1536),
                                   (4000, 4100, 1024), (128, 4096, 4096), (96, 1000, 6144)])
def test_gemm_fp4_interior(shape):
    """Full tiles: 128 x 128 tiles (16 tiles) and 256 x 256 tiles (256 tiles), K a
    whole number of code groups, in two and in three groups; 256 x 256 tiles cut by
    M and N (272 tiles, the last tile row 160 rows, the last column 4, on the
    interior mainloop); and split-K shapes with few output tiles (decode-like
    M = 128, and ragged M and N with three code groups per K slice)."""
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, seed=N + K)
    announce("gemm e2m1 interior", shape)
    if shape == (4000, 4100, 1024):
        assert F.fp8gemm_run_path(M, N, K, K // 2, K // 2, F.FORMATS["e2m1"], F.FORMATS["e2m1"],
                                  F.SCALE_MODES["mx32"], 0) == "tile256"
    C = _run(qa, sa, qb, sb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    bm, bn = min(128, M), 128
    blocks = [(0, 0), (M - bm, N - bn)] + [
        (int(r) * bm, int(c) * bn) for r, c in rng.integers(0, [M // bm, N // bn], (3, 2))]
    for r0, c0 in blocks:
        ri, ci = np.arange(r0, r0 + bm), np.arange(c0, c0 + bn)
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", rows=ri, cols=ci, fmt_a="e2m1",
                                  fmt_b="e2m1")
        _assert(to_host(C[r0:r0 + bm, c0:c0 + bn]), Cr, Ar, "bf16",
                f"e2m1 {shape} block {(r0, c0)}")


@pytest.mark.parametrize("act", ["relu", "gelu"])
@pytest.mark.parametrize("shape", [(257, 263, 4160), (512, 512, 1024)])
def test_gemm_fp4_fused_epilogue(act, shape):
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, seed=3 * M + N)
    bias = np.random.default_rng(N).standard_normal(N).astype(np.float32) * 4
    announce("gemm e2m1 fused", act, shape)
    C = to_host(_run(qa, sa, qb, sb, "bf16", bias, act))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a="e2m1", fmt_b="e2m1")
    _assert(C, Cr, Ar, "bf16", f"e2m1 fused {act} {shape}", bias, act)


def test_quantize_then_gemm_fp4():
    """The library's own quantiser feeds its GEMM (workload-like MX inputs)."""
    M, N, K = 256, 384, 1024
    A, B = random_inputs(M, N, K, seed=91, dist="mx_block")
    announce("quantize + gemm e2m1", (M, N, K))
    qa, sa = F.quantize(torch.from_numpy(A).to(DEV), "mx32", fmt="e2m1")
    qb, sb = F.quantize(torch.from_numpy(B).to(DEV), "mx32", fmt="e2m1")
    C = to_host(F.gemm(qa, sa, qb, sb, "mx32", "bf16", fmt_a="e2m1", fmt_b="e2m1"))
    qar, sar = Q.quantize_mx(A, "e2m1")
    qbr, sbr = Q.quantize_mx(B, "e2m1")
    Cr, Ar = O.gemm_reference(qar, sar, qbr, sbr, "mx32", fmt_a="e2m1", fmt_b="e2m1")
    _assert(C, Cr, Ar, "bf16", "quantize + gemm e2m1")


@pytest.mark.parametrize("shape", [(1, 1, 32), (1, 33, 64), (65, 1, 96), (2, 64, 32)])
def test_gemm_fp4_degenerate(shape):
    """Single rows / columns and the smallest K (one 32-element block, 16 bytes)."""
    M, N, K = shape
    qa, sa, qb, sb = _operands(M, N, K, seed=M * 31 + N + K)
    announce("gemm e2m1 degenerate", shape)
    C = to_host(_run(qa, sa, qb, sb))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a="e2m1", fmt_b="e2m1")
    _assert(C, Cr, Ar, "bf16", f"e2m1 degenerate {shape}")


def test_quantize_fp4_block_maxima_at_binade_edges():
    """Block maxima at 4 * 2^j, 6 * 2^j and just below 8 * 2^j (the top of the binade
    the shared exponent maps to [4, 8)), and just below 4 * 2^j (one exponent less)."""
    rows = []
    for j in (-10, -1, 0, 3, 20):
        for top in (4.0, 6.0, np.nextafter(np.float32(8.0), np.float32(0)),
                    np.nextafter(np.float32(4.0), np.float32(0))):
            row = np.linspace(-top, top, 32).astype(np.float32) * np.float32(2.0 ** j)
            rows.append(row)
    x = np.stack(rows).astype(np.float32)
    _check_quant(x, "binade edges")


@pytest.mark.parametrize("shape,path,lda", [((300, 256, 512), "tile128", (1 << 25) + 64),
                                            ((4096, 4096, 512), "tile128", (1 << 23) + 64)])
def test_gemm_fp4_spans_past_32_bit_offsets(shape, path, lda):
    """MXFP4 A with a row pitch whose tile rows span more than 2^31 bytes: the
    large tile is not planned (its interior mainloop needs 32-bit spans) and the
    128-row tiles take the general mainloop with 64-bit row addresses."""
    M, N, K = shape
    assert F.fp8gemm_run_path(M, N, K, lda, K // 2, 4, 4, F.SCALE_MODES["mx32"], 0) == path
    qa, sa, qb, sb = _operands(M, N, K, seed=M + N + K)
    announce("fp4 32-bit spans", shape, lda)
    pa = O.pack_fp4(qa)
    a_buf = torch.zeros((M, lda), dtype=torch.uint8, device=DEV)   # 9.4 or 32 GiB
    a_buf[:, :K // 2] = torch.from_numpy(pa).to(DEV)
    C = F.gemm(a_buf[:, :K // 2], scale_to_dev(sa, "mx32"), to_dev(O.pack_fp4(qb), 16),
               scale_to_dev(sb, "mx32"), "mx32", "bf16", fmt_a="e2m1", fmt_b="e2m1")
    torch.cuda.synchronize()
    del a_buf
    torch.cuda.empty_cache()
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "mx32", fmt_a="e2m1", fmt_b="e2m1")
    _assert(to_host(C), Cr, Ar, "bf16", f"fp4 spans {shape}")
