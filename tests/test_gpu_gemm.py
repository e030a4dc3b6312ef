"""GPU GEMM parity: |C - C_ref| <= 1e-3 * sum|a*b| + 1 output ulp against the oracle.

Operands are quantised by the oracle (so the GEMM is checked on its own) and,
in the end-to-end cases, by the GPU (checked bit-exact against the oracle
first).  Shapes span several tiles, ragged M / N / K edges, the single-element
case, both tile configurations, all scale modes and both output types; the
dense workloads run at full size (the 8192^3 MX case on sampled 128 x 128
tiles).  Determinism and out-of-bounds stores (guard canaries) are checked too.
"""
import numpy as np
import pytest
import torch

import block_scaled_gemm_fp8gemm_amd as F
import oracle as O
from oracle import quant as Q
from workloads import WORKLOADS, dense_inputs, random_inputs

from gpu_support import DEV, announce, assert_within_bound, scale_to_dev, to_dev, to_host

pytestmark = pytest.mark.gpu

MODES = ["tensor", "rowwise", "mx32"]


def _oracle_operands(M, N, K, mode, seed, dist="outlier"):
    A, B = random_inputs(M, N, K, seed, dist)
    qa, sa = Q.quantize(A, mode)
    qb, sb = Q.quantize(B, mode)
    return qa, sa, qb, sb


def _run_gpu(qa, sa, qb, sb, mode, out):
    return F.gemm(to_dev(qa, 16), scale_to_dev(sa, mode), to_dev(qb, 16), scale_to_dev(sb, mode),
                  mode, out)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 32), (33, 70, 64), (256, 256, 256), (300, 520, 384),
                                   (257, 263, 4160), (129, 1000, 96)])
def test_gemm_small_shapes(mode, out, shape):
    M, N, K = shape
    qa, sa, qb, sb = _oracle_operands(M, N, K, mode, seed=M + 3 * N + 7 * K)
    announce("gemm", mode, out, shape)
    C = to_host(_run_gpu(qa, sa, qb, sb, mode, out))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
    assert_within_bound(C, Cr, Ar, out, f"{mode}/{out}/{shape}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(4096, 4096, 256), (4000, 4100, 192), (4352, 4096, 256),
                                   (4300, 4000, 128)])
def test_gemm_big_tiles(mode, shape):
    """Shapes with >= 256 tiles of 256 x 256 take the large-tile kernel (ragged edges
    too); with 17 tile rows the last one joins the last group of four in the tile
    order.  Every output element is checked."""
    M, N, K = shape
    qa, sa, qb, sb = _oracle_operands(M, N, K, mode, seed=11, dist="mx_block")
    announce("gemm big", mode, shape)
    C = to_host(_run_gpu(qa, sa, qb, sb, mode, "bf16"))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
    assert_within_bound(C, Cr, Ar, "bf16", f"big {mode} {shape}")


def _slice_scales(s, idx, mode):
    return s if mode == "tensor" else s[idx]


@pytest.mark.parametrize("mode,shape", [
    ("mx32", (4096, 4096, 512)),      # large tiles, one 512-K group of MX codes
    ("mx32", (4096, 4096, 1536)),     # three code groups, loop over 4 K tiles at a time
    ("tensor", (4096, 4352, 384)),    # odd number of 128-K tiles: loop tail
    ("rowwise", (4096, 4096, 640)),
    ("mx32", (1024, 1024, 512)),      # small-tile kernel
    ("rowwise", (1024, 768, 384)),
    # 512 - 1024 tiles of 256 x 256: one tile per workgroup, several waves of workgroups
    ("tensor", (8192, 4096, 1024)),
    ("rowwise", (8192, 8192, 512)),
    ("mx32", (6144, 8192, 1024)),
])
def test_gemm_interior_sampled(mode, shape):
    """Full-tile shapes on the interior mainloop; the oracle checks sampled 128 x 128 blocks."""
    M, N, K = shape
    qa, sa, qb, sb = _oracle_operands(M, N, K, mode, seed=M + N + K, dist="mx_block")
    announce("gemm interior", mode, shape)
    C = _run_gpu(qa, sa, qb, sb, mode, "bf16")
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    blocks = [(0, 0), (M - 128, N - 128)] + [
        (int(r) * 128, int(c) * 128) for r, c in rng.integers(0, [M // 128, N // 128], size=(6, 2))]
    for r0, c0 in blocks:
        ri, ci = np.arange(r0, r0 + 128), np.arange(c0, c0 + 128)
        Cr, Ar = O.gemm_reference(qa[ri], _slice_scales(sa, ri, mode), qb[ci],
                                  _slice_scales(sb, ci, mode), mode)
        assert_within_bound(to_host(C[r0:r0 + 128, c0:c0 + 128]), Cr, Ar, "bf16",
                            f"interior {mode} {shape} block {(r0, c0)}")


def _grouped_tile(linear, tiles_m, tiles_n, group_m=4):
    """Position in the grouped tile order -> (tile row, tile column): groups of
    group_m tile rows, column-major inside a group (the order the kernels use)."""
    per_group = group_m * tiles_n
    gid = linear // per_group
    first_m = gid * group_m
    rows = min(tiles_m - first_m, group_m)
    in_group = linear - gid * per_group
    return first_m + in_group % rows, in_group // rows


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(16384, 8192, 512), (8192, 16384, 1024)])
def test_gemm_persistent_sampled(mode, out, shape):
    """Shapes with >= 2048 tiles of 256 x 256, all interior, take the persistent
    kernel: one workgroup per CU walks tiles slot, slot + 256, ... of the grouped
    order as one copy stream.  The oracle checks 128 x 128 blocks of the first and
    the last tile of several workgroups' lists (both diagonal quadrants of each),
    the first and the last tile of the matrix."""
    M, N, K = shape
    assert F.fp8gemm_run_path(M, N, K, K, K, 0, 0, F.SCALE_MODES[mode], 0) == "persistent"
    qa, sa, qb, sb = _oracle_operands(M, N, K, mode, seed=M // 7 + N + K, dist="mx_block")
    announce("gemm persistent", mode, out, shape)
    C = _run_gpu(qa, sa, qb, sb, mode, out)
    torch.cuda.synchronize()
    tiles_m, tiles_n = M // 256, N // 256
    total, grid = tiles_m * tiles_n, 256            # one workgroup per CU of an MI355X
    positions = {0, total - 1}
    for slot in (0, 37, 128, 200, 255):
        count = (total - slot + grid - 1) // grid
        positions |= {slot, slot + (count - 1) * grid}
    blocks = set()
    for pos in sorted(positions):
        tm, tn = _grouped_tile(pos, tiles_m, tiles_n)
        blocks |= {(tm * 256, tn * 256), (tm * 256 + 128, tn * 256 + 128)}
    for r0, c0 in sorted(blocks):
        ri, ci = np.arange(r0, r0 + 128), np.arange(c0, c0 + 128)
        Cr, Ar = O.gemm_reference(qa[ri], _slice_scales(sa, ri, mode), qb[ci],
                                  _slice_scales(sb, ci, mode), mode)
        assert_within_bound(to_host(C[r0:r0 + 128, c0:c0 + 128]), Cr, Ar, out,
                            f"persistent {mode}/{out} {shape} block {(r0, c0)}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(128, 4096, 4096), (100, 1000, 2048), (256, 640, 4096),
                                   (128, 4096, 1024), (200, 1024, 1024)])
def test_gemm_splitk(mode, shape):
    """Shapes with few output tiles run split along K (ragged M / N included)."""
    M, N, K = shape
    assert F.fp8gemm_workspace_size(M, N, K, F.SCALE_MODES[mode]) > 0, "shape is not split"
    qa, sa, qb, sb = _oracle_operands(M, N, K, mode, seed=M + 5 * N + K, dist="mx_block")
    announce("gemm split-K", mode, shape)
    C = to_host(_run_gpu(qa, sa, qb, sb, mode, "bf16"))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
    assert_within_bound(C, Cr, Ar, "bf16", f"split-K {mode} {shape}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out,shape", [
    ("f16", (1, 2048, 1024)),         # one row of A
    ("bf16", (17, 2056, 4160)),       # ragged M, N % 16 = 8, K % 128 = 64
    ("f16", (64, 8200, 1056)),        # K % 128 = 32
    ("bf16", (100, 2048, 384)),       # three 128-K tiles
])
def test_gemm_few_rows(mode, out, shape):
    """Few rows of A against many columns (decode-like), ragged in every dimension."""
    M, N, K = shape
    qa, sa, qb, sb = _oracle_operands(M, N, K, mode, seed=7 * M + N + K, dist="mx_block")
    announce("gemm few rows", mode, out, shape)
    C = to_host(_run_gpu(qa, sa, qb, sb, mode, out))
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
    assert_within_bound(C, Cr, Ar, out, f"few rows {mode}/{out}/{shape}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out,shape", [
    ("bf16", (128, 4096, 4096)),   # the decode-like shape
    ("f16", (1, 2048, 1024)),      # one row; 512-K slices
    ("bf16", (33, 1000, 2048)),    # ragged M and N
    ("f16", (100, 12000, 1024)),   # N ragged
    ("bf16", (64, 4100, 8192)),    # last tile 4 columns, K = 8192
    ("bf16", (128, 4096, 8192)),
    ("bf16", (128, 256, 1024)),    # few tiles
])
def test_gemm_decode_shapes(mode, out, shape):
    """Few rows of A (M <= 128) against many columns of B, split along K where the
    output tiles alone do not fill the GPU; the whole output, or all rows x
    sampled 128-column blocks for the large shapes, against the oracle."""
    M, N, K = shape
    qa, sa, qb, sb = _oracle_operands(M, N, K, mode, seed=M + 3 * N + K, dist="mx_block")
    path = F.fp8gemm_run_path(M, N, K, K, K, 0, 0, F.SCALE_MODES[mode], 0)
    announce("gemm decode shape", mode, out, shape, path)
    C = _run_gpu(qa, sa, qb, sb, mode, out)
    torch.cuda.synchronize()
    if N * K <= 4096 * 4096:
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
        assert_within_bound(to_host(C), Cr, Ar, out, f"decode {mode}/{out} {shape}")
        return
    for c0 in (0, N - 128, (N // 3) // 32 * 32):
        ci = np.arange(c0, c0 + 128)
        Cr, Ar = O.gemm_reference(qa, sa, qb[ci], _slice_scales(sb, ci, mode), mode)
        assert_within_bound(to_host(C[:, c0:c0 + 128]), Cr, Ar, out,
                            f"decode {mode}/{out} {shape} columns {c0}..")


def test_gemm_splitk_repeat_and_interleave():
    """The per-tile counters reset themselves: repeated and interleaved calls on one
    workspace give bit-identical results (the partials are summed in slice order)."""
    ops1 = _oracle_operands(128, 4096, 4096, "tensor", seed=21)
    ops2 = _oracle_operands(100, 1000, 2048, "rowwise", seed=22)
    announce("gemm split-K repeat")
    d1 = [to_dev(ops1[0], 16), scale_to_dev(ops1[1], "tensor"), to_dev(ops1[2], 16),
          scale_to_dev(ops1[3], "tensor")]
    d2 = [to_dev(ops2[0], 16), scale_to_dev(ops2[1], "rowwise"), to_dev(ops2[2], 16),
          scale_to_dev(ops2[3], "rowwise")]
    first1 = F.gemm(*d1, "tensor", "bf16")
    first2 = F.gemm(*d2, "rowwise", "bf16")
    for _ in range(3):
        again1 = F.gemm(*d1, "tensor", "bf16")
        again2 = F.gemm(*d2, "rowwise", "bf16")
        torch.cuda.synchronize()
        assert torch.equal(first1, again1)
        assert torch.equal(first2, again2)
    Cr, Ar = O.gemm_reference(*ops1, "tensor")
    assert_within_bound(to_host(first1), Cr, Ar, "bf16", "split-K repeat")


def test_gemm_splitk_two_streams():
    """Split-K GEMMs queued on two streams at once: the binding gives each stream
    its own workspace (counters and partial tiles), so neither corrupts the other."""
    ops1 = _oracle_operands(128, 4096, 4096, "tensor", seed=31)
    ops2 = _oracle_operands(128, 2048, 4096, "rowwise", seed=32)
    announce("gemm split-K on two streams")
    d1 = [to_dev(ops1[0], 16), scale_to_dev(ops1[1], "tensor"), to_dev(ops1[2], 16),
          scale_to_dev(ops1[3], "tensor")]
    d2 = [to_dev(ops2[0], 16), scale_to_dev(ops2[1], "rowwise"), to_dev(ops2[2], 16),
          scale_to_dev(ops2[3], "rowwise")]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()        # default priority
    outs1, outs2 = [], []
    for _ in range(6):
        with torch.cuda.stream(s1):
            outs1.append(F.gemm(*d1, "tensor", "bf16"))
        with torch.cuda.stream(s2):
            outs2.append(F.gemm(*d2, "rowwise", "bf16"))
    torch.cuda.synchronize()
    for c in outs1[1:]:
        assert torch.equal(c, outs1[0])
    for c in outs2[1:]:
        assert torch.equal(c, outs2[0])
    Cr, Ar = O.gemm_reference(*ops1, "tensor")
    assert_within_bound(to_host(outs1[0]), Cr, Ar, "bf16", "split-K stream 1")
    Cr, Ar = O.gemm_reference(*ops2, "rowwise")
    assert_within_bound(to_host(outs2[-1]), Cr, Ar, "bf16", "split-K stream 2")


def test_gemm_k16_tail_with_canaries():
    """K = 16 (one partial chunk pair) and guard bands around C must stay untouched."""
    M, N, K = 70, 90, 16
    qa, sa, qb, sb = _oracle_operands(M, N, K, "rowwise", seed=5)
    announce("gemm canary", (M, N, K))
    ldc = 128
    sentinel = 12352.0                       # exactly representable in bfloat16
    buf = torch.full((M + 2, ldc), sentinel, dtype=torch.bfloat16, device=DEV)
    out = buf[1:M + 1, :N]
    F.gemm(to_dev(qa, 16), scale_to_dev(sa, "rowwise"), to_dev(qb, 16),
           scale_to_dev(sb, "rowwise"), "rowwise", "bf16", out=out)
    torch.cuda.synchronize()
    host = to_host(buf)
    assert np.all(host[0] == sentinel) and np.all(host[-1] == sentinel)
    assert np.all(host[1:M + 1, N:] == sentinel)
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "rowwise")
    assert_within_bound(host[1:M + 1, :N], Cr, Ar, "bf16", "canary")


def test_gemm_deterministic():
    qa, sa, qb, sb = _oracle_operands(1024, 1024, 1024, "mx32", seed=9, dist="mx_block")
    announce("gemm determinism")
    c1 = _run_gpu(qa, sa, qb, sb, "mx32", "bf16")
    c2 = _run_gpu(qa, sa, qb, sb, "mx32", "bf16")
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


def _end_to_end(name, rows=None, cols=None, tiles=None):
    """GPU quantize + GEMM on a workload; oracle on the same (sampled) rows/columns."""
    w = WORKLOADS[name]
    A, B = dense_inputs(w)
    announce("end-to-end", name, w.mode, (w.M, w.N, w.K))
    qa_d, sa_d = F.quantize(to_dev(A), w.mode)
    qb_d, sb_d = F.quantize(to_dev(B), w.mode)
    C_d = F.gemm(qa_d, sa_d, qb_d, sb_d, w.mode, w.out)
    torch.cuda.synchronize()
    qa_g, qb_g = to_host(qa_d), to_host(qb_d)
    if tiles is None:
        qa, sa = Q.quantize(A, w.mode)
        qb, sb = Q.quantize(B, w.mode)
        assert np.array_equal(qa_g, qa) and np.array_equal(qb_g, qb)
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, w.mode)
        assert_within_bound(to_host(C_d), Cr, Ar, w.out, name)
        return
    # sampled tiles: row-local (MX / row-wise) quantisation lets the oracle work on
    # just the rows of A and B a tile needs
    assert w.mode in ("mx32", "rowwise")
    C_full = C_d
    for (r0, c0) in tiles:
        rows_i = np.arange(r0, min(r0 + 128, w.M))
        cols_i = np.arange(c0, min(c0 + 128, w.N))
        qa, sa = Q.quantize(A[rows_i], w.mode)
        qb, sb = Q.quantize(B[cols_i], w.mode)
        assert np.array_equal(qa_g[rows_i], qa) and np.array_equal(qb_g[cols_i], qb)
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, w.mode)
        Cg = to_host(C_full[r0:r0 + 128, c0:c0 + 128])
        assert_within_bound(Cg, Cr, Ar, w.out, f"{name} tile {(r0, c0)}")


def test_workload_pertensor256():
    _end_to_end("pertensor256")


def test_workload_skinny128():
    _end_to_end("skinny128")


def test_workload_rowwise4096():
    _end_to_end("rowwise4096")


def test_workload_mx8192_sampled_tiles():
    w = WORKLOADS["mx8192"]
    rng = np.random.default_rng(404)
    corners = [(0, 0), (0, w.N - 128), (w.M - 128, 0), (w.M - 128, w.N - 128)]
    rand = [(int(r) * 128, int(c) * 128) for r, c in rng.integers(0, w.M // 128, size=(12, 2))]
    _end_to_end("mx8192", tiles=corners + rand)


def test_gemm_splitk_growing_tile_count():
    """Split shapes with more output tiles after fewer, on the one workspace the
    binding keeps: a later call's tile counters never lie where an earlier call
    left partial tiles (the counters have a fixed place)."""
    shapes = [(128, 2048, 4096), (128, 8192, 4096), (64, 8192, 2048), (128, 2048, 4096)]
    for i, (M, N, K) in enumerate(shapes):
        assert F.fp8gemm_workspace_size(M, N, K, F.SCALE_MODES["rowwise"]) > 0, "not split"
        qa, sa, qb, sb = _oracle_operands(M, N, K, "rowwise", seed=40 + i, dist="mx_block")
        announce("gemm split-K growing", (M, N, K))
        C = to_host(_run_gpu(qa, sa, qb, sb, "rowwise", "bf16"))
        Cr, Ar = O.gemm_reference(qa, sa, qb, sb, "rowwise")
        assert_within_bound(C, Cr, Ar, "bf16", f"split-K after other shapes {(M, N, K)}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape,path,lda", [((300, 256, 256), "tile128", (1 << 25) + 64),
                                            ((128, 4096, 1024), "splitk", (1 << 25) + 64),
                                            ((4096, 4096, 128), "tile256", (1 << 23) + 64)])
def test_gemm_spans_past_32_bit_offsets(mode, shape, path, lda):
    """Row pitches of 32 MiB + 64 bytes (8 MiB + 64 for the 256-row tiles): the
    rows of one tile of A span more than 2^31 bytes, past the 32-bit offsets of
    the interior mainloop's buffer descriptors, so the tiles take the general
    mainloop (64-bit row addresses).  Every output element is checked against
    the oracle."""
    M, N, K = shape
    assert F.fp8gemm_run_path(M, N, K, lda, K, 0, 0, F.SCALE_MODES[mode], 0) == path
    qa, sa, qb, sb = _oracle_operands(M, N, K, mode, seed=M + N + K)
    announce("gemm 32-bit spans", mode, shape, lda)
    a_buf = torch.zeros((M, lda), dtype=torch.uint8, device=DEV)   # 4 to 32 GiB
    a_buf[:, :K] = torch.from_numpy(qa).to(DEV)
    C = F.gemm(a_buf[:, :K], scale_to_dev(sa, mode), to_dev(qb, 16), scale_to_dev(sb, mode),
               mode, "bf16")
    torch.cuda.synchronize()
    del a_buf
    torch.cuda.empty_cache()                       # hand the large buffer back
    Cr, Ar = O.gemm_reference(qa, sa, qb, sb, mode)
    assert_within_bound(to_host(C), Cr, Ar, "bf16", f"spans {mode} {shape}")
