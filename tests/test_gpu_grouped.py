"""GPU grouped (MoE) GEMM parity against the oracle.

Small ragged expert mixes (empty experts, experts shorter than a tile, a K tail)
in every scale mode, one expert against the dense GEMM, and the 8-expert
16384 x 4096 -> 14336 workload end to end (GPU quantisation checked bit-exact,
C checked on the first, last and six random rows of every expert, all columns).
"""
import numpy as np
import pytest
import torch

import block_scaled_gemm_fp8gemm_amd as F
import oracle as O
from oracle import quant as Q
from workloads import WORKLOADS, grouped_inputs, normal

from gpu_support import DEV, announce, assert_within_bound, scale_to_dev, to_dev, to_host

pytestmark = pytest.mark.gpu

MODES = ["tensor", "rowwise", "mx32"]


def _quant_experts(W, mode):
    qs, ss = zip(*[Q.quantize(W[g], mode) for g in range(W.shape[0])])
    qw = np.stack(qs)
    if mode == "tensor":
        sw = np.array([float(s) for s in ss], np.float32)
    else:
        sw = np.stack(ss)
    return qw, sw


def _dev3(q):
    G, N, K = q.shape
    ld = (K + 15) // 16 * 16
    t = torch.zeros((G, N, ld), dtype=torch.uint8, device=DEV)
    t[:, :, :K] = torch.from_numpy(q).to(DEV)
    return t[:, :, :K]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("counts,N,K", [([5, 0, 300, 77], 200, 192), ([0, 0, 513], 64, 128),
                                        ([1, 1, 1, 1, 1, 1], 300, 64), ([256, 256], 512, 256),
                                        ([300, 0, 1200, 500], 768, 1024)])
def test_grouped_small(mode, out, counts, N, K):
    rng = np.random.default_rng(sum(counts) + N + K)
    counts = np.array(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = normal(rng, int(off[-1]), K)
    W = np.stack([normal(rng, N, K, 0.02) for _ in counts])
    qa, sa = Q.quantize(x, mode)
    qw, sw = _quant_experts(W, mode)
    announce("grouped", mode, out, counts.tolist(), N, K)
    C = F.grouped_gemm(to_dev(qa, 16), scale_to_dev(sa, mode), torch.from_numpy(off).to(DEV),
                       _dev3(qw), torch.from_numpy(np.ascontiguousarray(sw)).to(DEV), mode, out)
    Cr, Ar = O.grouped_reference(qa, sa, off, qw, sw, mode)
    assert_within_bound(to_host(C), Cr, Ar, out, f"grouped {mode}/{out} {counts.tolist()}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("N,K", [(8192, 1024), (768, 512)])
def test_grouped_cut_tiles_in_stream(mode, out, N, K):
    """K % 512 == 0, N a multiple of 256: tiles cut by an expert's last row with
    at least a tile of rows of A after them run inside the copy stream and store
    only their own rows (cuts of 1, 44, 255, 1 and 40 rows); the cuts of the last
    two experts (188 and 3 rows) reach past A and take the general path.  With
    N = 8192 (352 tiles) some workgroups stream two; with K = 512 (four K tiles,
    the stream's shortest) every workgroup streams one.  Every expert's rows
    equal, bit for bit, the same expert run alone (its cut tile then on the
    general path); the oracle bound holds everywhere; rows around C and the
    columns past N keep their canaries."""
    rng = np.random.default_rng(4242 + K)
    counts = np.array([1, 300, 0, 255, 257, 40, 700, 3])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(off[-1])
    x = normal(rng, total, K)
    W = np.stack([normal(rng, N, K, 0.02) for _ in counts])
    qa, sa = Q.quantize(x, mode)
    qw, sw = _quant_experts(W, mode)
    announce("grouped cut tiles in stream", mode, out, counts.tolist(), N, K)
    tdt = torch.float16 if out == "f16" else torch.bfloat16
    pad, ldc = 16, N + 64
    buf = torch.full((total + 2 * pad, ldc), -7.0, dtype=tdt, device=DEV)
    C = F.grouped_gemm(to_dev(qa, 16), scale_to_dev(sa, mode), torch.from_numpy(off).to(DEV),
                       _dev3(qw), torch.from_numpy(np.ascontiguousarray(sw)).to(DEV), mode, out,
                       out=buf[pad:pad + total, :N])
    torch.cuda.synchronize()
    assert bool((buf[:pad] == -7.0).all()) and bool((buf[pad + total:] == -7.0).all())
    assert bool((buf[:, N:] == -7.0).all())
    Cr, Ar = O.grouped_reference(qa, sa, off, qw, sw, mode)
    assert_within_bound(to_host(C), Cr, Ar, out, f"grouped cut {mode}/{out}")
    for g, c in enumerate(counts):
        if c == 0:
            continue
        r0, r1 = int(off[g]), int(off[g + 1])
        sa_g = sa if mode == "tensor" else np.ascontiguousarray(np.asarray(sa)[r0:r1])
        sw_g = np.ascontiguousarray(sw[g:g + 1])
        Cg = F.grouped_gemm(to_dev(np.ascontiguousarray(qa[r0:r1]), 16), scale_to_dev(sa_g, mode),
                            torch.tensor([0, r1 - r0], dtype=torch.int32, device=DEV),
                            _dev3(qw[g:g + 1]), torch.from_numpy(sw_g).to(DEV), mode, out)
        torch.cuda.synchronize()
        assert torch.equal(C[r0:r1], Cg), f"expert {g} ({c} rows)"


@pytest.mark.parametrize("mode", MODES)
def test_grouped_one_expert_equals_dense(mode):
    rng = np.random.default_rng(77)
    M, N, K = 700, 600, 512
    x, w = normal(rng, M, K), normal(rng, N, K, 0.02)
    qa, sa = Q.quantize(x, mode)
    qw, sw = Q.quantize(w, mode)
    announce("grouped G=1 vs dense", mode)
    sw_g = np.asarray(sw)[None] if mode != "tensor" else np.array([float(sw)], np.float32)
    Cg = F.grouped_gemm(to_dev(qa, 16), scale_to_dev(sa, mode),
                        torch.tensor([0, M], dtype=torch.int32, device=DEV), _dev3(qw[None]),
                        torch.from_numpy(np.ascontiguousarray(sw_g)).to(DEV), mode, "bf16")
    Cd = F.gemm(to_dev(qa, 16), scale_to_dev(sa, mode), to_dev(qw, 16), scale_to_dev(sw, mode),
                mode, "bf16")
    torch.cuda.synchronize()
    assert torch.equal(Cg, Cd)


@pytest.mark.slow
def test_workload_grouped_moe():
    w = WORKLOADS["grouped_moe"]
    counts, A, W = grouped_inputs(w)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    announce("grouped workload", counts.tolist(), (w.M, w.N, w.K))
    qa_d, sa_d = F.quantize(to_dev(A), w.mode)
    Wd = torch.from_numpy(W).to(DEV)
    qw_d, sw_d = F.quantize(Wd.view(w.groups * w.N, w.K), w.mode)
    del Wd
    C = F.grouped_gemm(qa_d, sa_d, torch.from_numpy(off).to(DEV),
                       qw_d.view(w.groups, w.N, w.K), sw_d.view(w.groups, w.N), w.mode, w.out)
    torch.cuda.synchronize()
    qa, sa = Q.quantize(A, w.mode)
    assert np.array_equal(to_host(qa_d), qa)
    assert np.array_equal(to_host(sa_d).view(np.uint32), sa.view(np.uint32))
    qw_g = to_host(qw_d).reshape(w.groups, w.N, w.K)
    sw_g = to_host(sw_d).reshape(w.groups, w.N)
    qw = np.empty_like(qw_g)
    sw = np.empty((w.groups, w.N), np.float32)
    for g in range(w.groups):
        qw[g], sw[g] = Q.quantize(W[g], w.mode)
        assert np.array_equal(qw_g[g], qw[g]), f"expert {g} codes"
        assert np.array_equal(sw_g[g].view(np.uint32), sw[g].view(np.uint32)), f"expert {g} scales"
    del W
    rng = np.random.default_rng(505)
    rows = []
    for g in range(w.groups):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            rows += [lo, hi - 1] + list(rng.integers(lo, hi, size=6))
    rows = np.array(sorted(set(rows)))
    Cr, Ar = O.grouped_reference(qa, sa, off, qw, sw, w.mode, rows=rows)
    Cg = to_host(C[torch.from_numpy(rows).to(DEV)])
    assert_within_bound(Cg, Cr, Ar, w.out, "grouped_moe sampled rows")


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("counts,N,K", [([5, 0, 300, 77], 200, 192), ([0, 0, 513], 64, 128),
                                        ([1, 1, 1, 1, 1, 1], 300, 64), ([256, 256], 512, 512),
                                        ([130, 0, 260], 256, 1056), ([130, 0, 300, 7], 512, 1024)])
def test_grouped_fp4(out, counts, N, K):
    """MXFP4 activations and experts (two e2m1 codes per byte): ragged and empty
    experts, experts shorter than a tile, whole code groups and a K tail, on both
    tile sizes (K a multiple of 256: the 256 x 256 tile with cut tiles)."""
    rng = np.random.default_rng(3 * sum(counts) + N + K)
    counts = np.array(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = normal(rng, int(off[-1]), K)
    W = np.stack([normal(rng, N, K, 0.02) for _ in counts])
    qa, sa = Q.quantize(x, "mx32", "e2m1")
    qs, ss = zip(*[Q.quantize(W[g], "mx32", "e2m1") for g in range(len(counts))])
    qw, sw = np.stack(qs), np.stack(ss)
    announce("grouped e2m1", out, counts.tolist(), N, K)
    C = F.grouped_gemm(to_dev(O.pack_fp4(qa), 16), scale_to_dev(sa, "mx32"),
                       torch.from_numpy(off).to(DEV), _dev3(O.pack_fp4(qw)),
                       torch.from_numpy(np.ascontiguousarray(sw)).to(DEV), "mx32", out,
                       fmt="e2m1")
    Cr, Ar = O.grouped_reference(qa, sa, off, qw, sw, "mx32", fmt="e2m1")
    assert_within_bound(to_host(C), Cr, Ar, out, f"grouped e2m1/{out} {counts.tolist()}")


@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_grouped_fp4_cut_tiles_interior(out):
    """MXFP4 experts with K % 512 == 0 run every tile on the interior mainloop,
    tiles cut by an expert's last row or by N included (their copies end at the
    last valid row or column): the oracle bound holds, rows around C and the
    columns past N keep their canaries, and one expert of 700 rows equals the
    dense MXFP4 GEMM of the same operands bit for bit."""
    rng = np.random.default_rng(909)
    counts = np.array([1, 300, 0, 255, 257, 40, 700, 3])
    N, K = 600, 1024
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(off[-1])
    x = normal(rng, total, K)
    W = np.stack([normal(rng, N, K, 0.02) for _ in counts])
    qa, sa = Q.quantize(x, "mx32", "e2m1")
    qs, ss = zip(*[Q.quantize(W[g], "mx32", "e2m1") for g in range(len(counts))])
    qw, sw = np.stack(qs), np.stack(ss)
    announce("grouped e2m1 cut tiles", out, counts.tolist(), N, K)
    tdt = torch.float16 if out == "f16" else torch.bfloat16
    pad, ldc = 16, N + 40
    buf = torch.full((total + 2 * pad, ldc), -7.0, dtype=tdt, device=DEV)
    C = F.grouped_gemm(to_dev(O.pack_fp4(qa), 16), scale_to_dev(sa, "mx32"),
                       torch.from_numpy(off).to(DEV), _dev3(O.pack_fp4(qw)),
                       torch.from_numpy(np.ascontiguousarray(sw)).to(DEV), "mx32", out,
                       out=buf[pad:pad + total, :N], fmt="e2m1")
    torch.cuda.synchronize()
    assert bool((buf[:pad] == -7.0).all()) and bool((buf[pad + total:] == -7.0).all())
    assert bool((buf[:, N:] == -7.0).all())
    Cr, Ar = O.grouped_reference(qa, sa, off, qw, sw, "mx32", fmt="e2m1")
    assert_within_bound(to_host(C), Cr, Ar, out, f"grouped e2m1 cut/{out}")
    g = 6                                           # 700 rows: two whole tile rows and a cut one
    r0, r1 = int(off[g]), int(off[g + 1])
    Cd = F.gemm(to_dev(O.pack_fp4(np.ascontiguousarray(qa[r0:r1])), 16),
                scale_to_dev(np.ascontiguousarray(sa[r0:r1]), "mx32"),
                to_dev(O.pack_fp4(qw[g]), 16), scale_to_dev(sw[g], "mx32"), "mx32", out,
                fmt_a="e2m1", fmt_b="e2m1")
    torch.cuda.synchronize()
    assert torch.equal(C[r0:r1], Cd)


@pytest.mark.parametrize("mode", ["rowwise", "mx32"])
def test_grouped_max_experts(mode):
    """The largest expert count the library takes (1024; more return
    NOT_SUPPORTED): the per-expert tables fill their LDS space; counts of 0 to 12
    rows (a third of the experts empty), so every tile is cut by its expert's
    last row."""
    G = 1024
    rng = np.random.default_rng(1024)
    counts = rng.integers(1, 13, G)
    counts[rng.random(G) < 1 / 3] = 0
    N, K = 256, 128
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(off[-1])
    x = normal(rng, total, K)
    W = normal(rng, G * N, K, 0.02).reshape(G, N, K)
    qa, sa = Q.quantize(x, mode)
    qw, sw = _quant_experts(W, mode)
    announce("grouped max experts", mode, G, total, N, K)
    C = F.grouped_gemm(to_dev(qa, 16), scale_to_dev(sa, mode), torch.from_numpy(off).to(DEV),
                       _dev3(qw), torch.from_numpy(np.ascontiguousarray(sw)).to(DEV), mode, "bf16")
    Cr, Ar = O.grouped_reference(qa, sa, off, qw, sw, mode)
    assert_within_bound(to_host(C), Cr, Ar, "bf16", f"grouped {G} experts {mode}")


@pytest.mark.parametrize("mode", MODES)
def test_grouped_spans_past_32_bit_offsets(mode):
    """A with an 8 MiB + 64 byte row pitch and C with a 4 Mi + 64 element one: a
    tile's rows of A, and its rows of C, span more than 2^31 bytes, so no tile
    streams (K % 512 == 0 would allow it) and every tile takes the general
    mainloop and the staged epilogue with 64-bit row addresses; cut tiles and an
    empty expert included.  Checked against the oracle; the columns past N keep
    their canaries."""
    counts = np.array([300, 0, 257])
    N, K = 256, 512
    lda, ldc = (1 << 23) + 64, (1 << 22) + 64
    rng = np.random.default_rng(2 ** 23)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(off[-1])
    x = normal(rng, total, K)
    W = np.stack([normal(rng, N, K, 0.02) for _ in counts])
    qa, sa = Q.quantize(x, mode)
    qw, sw = _quant_experts(W, mode)
    announce("grouped 32-bit spans", mode, counts.tolist(), lda, ldc)
    a_buf = torch.zeros((total, lda), dtype=torch.uint8, device=DEV)          # 4.7 GiB
    a_buf[:, :K] = torch.from_numpy(qa).to(DEV)
    c_buf = torch.full((total, ldc), -7.0, dtype=torch.bfloat16, device=DEV)  # 4.7 GiB
    C = F.grouped_gemm(a_buf[:, :K], scale_to_dev(sa, mode), torch.from_numpy(off).to(DEV),
                       _dev3(qw), torch.from_numpy(np.ascontiguousarray(sw)).to(DEV), mode, "bf16",
                       out=c_buf[:, :N])
    torch.cuda.synchronize()
    assert bool((c_buf[:, N:N + 64] == -7.0).all())
    Ch = to_host(C)
    del a_buf, c_buf, C
    torch.cuda.empty_cache()
    Cr, Ar = O.grouped_reference(qa, sa, off, qw, sw, mode)
    assert_within_bound(Ch, Cr, Ar, "bf16", f"grouped spans {mode}")
