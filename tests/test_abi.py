"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments with the documented status
before making any HIP call (so no device is touched).

Fake device addresses below are never dereferenced: every call either fails
validation or has no work (M or N = 0).
"""
import ctypes
import os

import pytest

import block_scaled_gemm_fp8gemm_amd as F

SUCCESS, INVALID, MISALIGNED, NOT_SUPPORTED, WORKSPACE = 0, 1, 2, 3, 4
P = 0x10000          # a 16-byte aligned fake device address
P2 = 0x20000
P3 = 0x30000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(F.library_path()):
        from block_scaled_gemm_fp8gemm_amd.build import build
        build()
    return F.load_library()


def test_exports_every_declared_symbol(lib):
    names = F.exported_symbols()
    assert set(names) == {
        "fp8gemm_quantize_workspace_size", "fp8gemm_quantize", "fp8gemm_quantize_ex",
        "fp8gemm_workspace_size", "fp8gemm_run", "fp8gemm_run_ex", "fp8gemm_workspace_size_kn",
        "fp8gemm_run_kn", "fp8gemm_run_mxout", "fp8gemm_qout_workspace_size", "fp8gemm_run_qout",
        "fp8gemm_grouped_workspace_size", "fp8gemm_grouped_run", "fp8gemm_grouped_run_ex",
        "fp8gemm_run_path", "fp8gemm_run_kn_path", "fp8gemm_run_noalloc", "fp8gemm_status_string",
        "fp8gemm_version"}
    raw = ctypes.CDLL(F.library_path())
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_strings(lib):
    assert F.fp8gemm_version() == 190
    for code, name in [(0, "FP8GEMM_SUCCESS"), (1, "FP8GEMM_ERROR_INVALID_VALUE"),
                       (2, "FP8GEMM_ERROR_MISALIGNED"), (3, "FP8GEMM_ERROR_NOT_SUPPORTED"),
                       (4, "FP8GEMM_ERROR_WORKSPACE"), (5, "FP8GEMM_ERROR_LAUNCH"),
                       (99, "FP8GEMM_ERROR_UNKNOWN")]:
        assert F.fp8gemm_status_string(code) == name


def test_workspace_queries(lib):
    assert F.fp8gemm_quantize_workspace_size(4096, 4096, 0) > 0
    assert F.fp8gemm_quantize_workspace_size(4096, 4096, 1) == 0
    assert F.fp8gemm_quantize_workspace_size(4096, 4096, 2) == 0
    # large shapes fill the GPU with output tiles: no workspace
    assert F.fp8gemm_workspace_size(4096, 4096, 4096, 1) == 0
    assert F.fp8gemm_workspace_size(8192, 8192, 8192, 2) == 0
    # the decode-like M = 128 shape is split along K: partials + counters
    for mode in (0, 1, 2):
        need = F.fp8gemm_workspace_size(128, 4096, 4096, mode)
        assert need >= 128 * 4096 * 4 * 2, (mode, need)
    assert F.fp8gemm_workspace_size(128, 4096, 256, 0) == 0      # K too short to split
    assert F.fp8gemm_workspace_size(128, 4096, 4096, 7) == 0     # bad mode
    assert F.fp8gemm_grouped_workspace_size(8, 16384, 14336, 4096, 1) >= 0


@pytest.mark.parametrize("shape,ld,fmt,mode,fused,path", [
    ((0, 4096, 4096), None, "e4m3", "tensor", 0, "none"),
    ((128, 4096, 4096), None, "e4m3", "tensor", 0, "splitk"),       # the decode-like shape
    ((128, 4096, 4096), None, "e4m3", "mx32", 1, "splitk"),
    ((1, 8192, 1024), None, "e5m2", "rowwise", 0, "splitk"),
    ((128, 4096, 4160), None, "e4m3", "tensor", 0, "tile128"),     # K % 256 != 0: no slices
    ((256, 640, 4096), None, "e4m3", "rowwise", 0, "splitk"),
    ((128, 16384, 4096), None, "e4m3", "tensor", 0, "tile128"),    # 128 tiles of 128 x 128
    ((128, 4096, 256), None, "e4m3", "tensor", 0, "tile128"),       # K too short to split
    ((1024, 1024, 512), None, "e4m3", "mx32", 0, "tile128"),
    ((4096, 4096, 4096), None, "e4m3", "rowwise", 0, "tile256"),    # 256 tiles: one per CU
    ((8192, 8192, 8192), None, "e4m3", "mx32", 0, "tile256"),       # 1024 tiles
    ((16384, 8192, 512), None, "e4m3", "tensor", 0, "persistent"),  # 2048 tiles, all interior
    ((8192, 16384, 1024), None, "e4m3", "mx32", 0, "persistent"),
    ((16384, 8192, 512), None, "e5m2", "rowwise", 0, "persistent"),
    ((16384, 8192, 512), None, "e4m3", "tensor", 1, "tile256"),     # fused: never streamed
    ((16384, 8192, 384), None, "e4m3", "tensor", 0, "tile256"),     # K % 512 != 0
    ((16384, 8320, 512), None, "e4m3", "tensor", 0, "tile256"),     # N cut: edge tiles
    ((4096, 4096, 4160), None, "e4m3", "mx32", 0, "tile128"),       # MX K tail: codes in registers
    ((8192, 8192, 8192), None, "e2m1", "mx32", 0, "tile256"),       # FP4: never persistent
    ((16384, 8192, 1024), None, "e2m1", "mx32", 0, "tile256"),
    ((4000, 4100, 8192), None, "e2m1", "mx32", 0, "tile256"),       # cut tiles, interior
    ((4000, 4096, 8192 + 256), None, "e2m1", "mx32", 0, "tile128"),  # K % 512 != 0
    ((128, 4096, 4096), None, "e2m1", "mx32", 0, "splitk"),
    ((128, 4096, 4096), None, "e2m1", "tensor", 0, "none"),        # FP4 takes MX scales only
])
def test_run_path_rules(lib, shape, ld, fmt, mode, fused, path):
    """The kernel a dense GEMM shape dispatches to (the query runs the launch code's
    own planner)."""
    M, N, K = shape
    kb = K // 2 if fmt == "e2m1" else K
    f = F.FORMATS[fmt]
    assert F.fp8gemm_run_path(M, N, K, kb, kb, f, f, F.SCALE_MODES[mode], fused) == path


def _noalloc(lib, M=128, N=4096, K=4096, A=P, lda=4096, B=P2, ldb=4096, mode=0, sa=P3, sb=P3,
             C=P, ldc=4096, out=1, afmt=0, bfmt=0, bias=0, act=0):
    return lib.fp8gemm_run_noalloc(M, N, K, A, lda, afmt, B, ldb, bfmt, mode, sa, sb, bias, act, C,
                                   ldc, out, None)


def test_noalloc_validation(lib):
    """Argument errors and a split too large for the static scratch are reported
    before any HIP call (the fake addresses are never touched)."""
    assert F.NOALLOC_SCRATCH_BYTES == 8 * 1024 * 1024 + 4096
    assert _noalloc(lib, out=5) == INVALID
    assert _noalloc(lib, mode=9) == INVALID
    assert _noalloc(lib, A=0) == INVALID
    assert _noalloc(lib, lda=100) == INVALID                  # lda < K
    assert _noalloc(lib, K=4008) == NOT_SUPPORTED             # K % 16 != 0
    assert _noalloc(lib, A=P + 8) == MISALIGNED
    assert _noalloc(lib, bias=P + 2) == MISALIGNED
    assert _noalloc(lib, afmt=4, bfmt=0, mode=2) == NOT_SUPPORTED
    assert _noalloc(lib, M=0) == SUCCESS                      # nothing to do
    # 504 split tiles x 2 K slices: 16.5 MB of partials, more than the scratch
    M, N, K = 256, 8064, 4096
    assert F.fp8gemm_workspace_size(M, N, K, 0) > F.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, M=M, N=N, K=K, lda=K, ldb=K, ldc=N) == WORKSPACE


def test_fp6_validation(lib):
    """FP6 (e2m3 / e3m2) takes MX scales, pairs with FP6 only, needs K % 128 == 0
    and is not offered for row-major B or grouped; rows hold 3K/4 bytes."""
    e2m3, e3m2, e4m3 = F.FORMATS["e2m3"], F.FORMATS["e3m2"], F.FORMATS["e4m3"]
    assert _noalloc(lib, K=1024, lda=768, ldb=768, mode=2, afmt=e2m3, bfmt=e3m2, M=0) == SUCCESS
    assert _noalloc(lib, K=1024, lda=768, ldb=768, mode=0, afmt=e2m3, bfmt=e2m3) == NOT_SUPPORTED
    assert _noalloc(lib, K=1024, lda=768, ldb=768, mode=2, afmt=e2m3, bfmt=e4m3) == NOT_SUPPORTED
    assert _noalloc(lib, K=1088, lda=816, ldb=816, mode=2, afmt=e2m3, bfmt=e2m3) == NOT_SUPPORTED
    assert _noalloc(lib, K=1024, lda=752, ldb=768, mode=2, afmt=e2m3, bfmt=e2m3) == INVALID
    assert F.fp8gemm_run_path(512, 512, 1024, 768, 768, e2m3, e3m2, 2, 0) == "tile128"
    assert F.fp8gemm_run_path(512, 512, 1024, 768, 768, e2m3, e4m3, 2, 0) == "none"
    assert lib.fp8gemm_run_kn(64, 64, 1024, P, 768, e2m3, P2, 64, e2m3, 2, P3, P3, 0, 0, P,
                              64, 1, P, 1 << 20, None) == NOT_SUPPORTED
    assert lib.fp8gemm_grouped_run_ex(2, 64, 64, 1024, P, 768, e2m3, P2, P3, 768, e2m3,
                                      64 * 768, 2, P3, P3, P, 64, 1, 0, 0, None) == NOT_SUPPORTED
    # quantiser: MX only; q rows of 3k/4 bytes
    assert lib.fp8gemm_quantize_ex(P, 4, 64, 64, 1, e3m2, P2, 48, P3, 0, 0, None) == NOT_SUPPORTED
    assert lib.fp8gemm_quantize_ex(P, 4, 64, 64, 2, e3m2, P2, 32, P3, 0, 0, None) == INVALID


def _quant(lib, x=P, rows=64, k=256, ldx=256, mode=1, q=P2, ldq=256, scales=P3, ws=0, wsb=0):
    return lib.fp8gemm_quantize(x, rows, k, ldx, mode, q, ldq, scales, ws, wsb, None)


def test_quantize_validation(lib):
    assert _quant(lib, mode=3) == INVALID
    assert _quant(lib, rows=-1) == INVALID
    assert _quant(lib, k=0) == INVALID
    assert _quant(lib, rows=0) == SUCCESS                 # nothing to do, nothing enqueued
    assert _quant(lib, x=0) == INVALID
    assert _quant(lib, q=0) == INVALID
    assert _quant(lib, scales=0) == INVALID
    assert _quant(lib, ldx=128) == INVALID                 # ldx < k
    assert _quant(lib, ldq=128) == INVALID
    assert _quant(lib, k=40, ldx=48, ldq=48) == NOT_SUPPORTED          # k % 16
    assert _quant(lib, k=48, ldx=48, ldq=48, mode=2) == NOT_SUPPORTED  # MX: k % 32
    assert _quant(lib, rows=1 << 20, k=4096, ldx=4096, ldq=4096) == NOT_SUPPORTED  # >= 2^32 elems
    assert _quant(lib, x=P + 4) == MISALIGNED
    assert _quant(lib, q=P2 + 8) == MISALIGNED
    assert _quant(lib, ldx=258) == MISALIGNED
    assert _quant(lib, ldq=264) == MISALIGNED
    assert _quant(lib, scales=P3 + 2) == MISALIGNED
    assert _quant(lib, mode=0) == WORKSPACE                 # per-tensor needs a workspace
    need = F.fp8gemm_quantize_workspace_size(64, 256, 0)
    assert _quant(lib, mode=0, ws=P, wsb=need - 4) == WORKSPACE


def _run(lib, M=64, N=64, K=128, A=P, lda=128, B=P2, ldb=128, mode=1, sa=P3, sb=P3 + 256,
         C=P3 + 4096, ldc=64, out=1):
    return lib.fp8gemm_run(M, N, K, A, lda, B, ldb, mode, sa, sb, C, ldc, out, 0, 0, None)


def test_run_validation(lib):
    assert _run(lib, mode=7) == INVALID
    assert _run(lib, out=2) == INVALID
    assert _run(lib, M=-1) == INVALID
    assert _run(lib, K=0) == INVALID
    assert _run(lib, M=0) == SUCCESS
    assert _run(lib, N=0) == SUCCESS
    for kw in ("A", "B", "C", "sa", "sb"):
        assert _run(lib, **{kw: 0}) == INVALID, kw
    assert _run(lib, lda=64) == INVALID
    assert _run(lib, ldb=64) == INVALID
    assert _run(lib, ldc=32) == INVALID
    assert _run(lib, K=120, lda=128, ldb=128) == NOT_SUPPORTED
    assert _run(lib, K=112, lda=112, ldb=112, mode=2) == NOT_SUPPORTED
    assert _run(lib, A=P + 1) == MISALIGNED
    assert _run(lib, B=P2 + 8) == MISALIGNED
    assert _run(lib, C=P3 + 4096 + 2) == MISALIGNED
    assert _run(lib, lda=136) == MISALIGNED
    assert _run(lib, ldc=68) == MISALIGNED
    assert _run(lib, sa=P3 + 1) == MISALIGNED
    assert _run(lib, M=1 << 31) == NOT_SUPPORTED


def _run_ex(lib, M=64, N=64, K=128, A=P, lda=128, fa=0, B=P2, ldb=128, fb=0, mode=1, sa=P3,
            sb=P3 + 256, bias=0, act=0, C=P3 + 4096, ldc=64, out=1):
    return lib.fp8gemm_run_ex(M, N, K, A, lda, fa, B, ldb, fb, mode, sa, sb, bias, act, C, ldc,
                              out, 0, 0, None)


def test_extended_entry_points_validation(lib):
    """Formats and the fused epilogue are validated before any HIP call."""
    assert _run_ex(lib, M=0) == SUCCESS
    assert _run_ex(lib, M=0, fa=1, fb=1, bias=P, act=3) == SUCCESS
    assert _run_ex(lib, fa=5) == INVALID
    assert _run_ex(lib, fa=2) == NOT_SUPPORTED      # e2m3 codes with e4m3 B: no such pairing
    assert _run_ex(lib, fb=-1) == INVALID
    assert _run_ex(lib, act=4) == INVALID
    assert _run_ex(lib, act=-1) == INVALID
    assert _run_ex(lib, bias=P + 2) == MISALIGNED
    assert _run_ex(lib, fa=1, K=112, lda=112, ldb=112, mode=2) == NOT_SUPPORTED
    assert _run_ex(lib, A=0) == INVALID
    q = lambda **kw: lib.fp8gemm_quantize_ex(kw.get("x", P), 64, kw.get("k", 256), 256,
                                             kw.get("mode", 1), kw.get("fmt", 0), P2, 256, P3, 0,
                                             0, None)
    assert q(fmt=5) == INVALID
    assert q(fmt=2) == NOT_SUPPORTED                # e2m3 codes need block (MX) scaling
    assert q(fmt=-1) == INVALID
    assert q(fmt=1, x=0) == INVALID
    assert q(fmt=1, k=48, mode=2) == NOT_SUPPORTED
    assert q(fmt=1, mode=0) == WORKSPACE


def test_fp4_validation(lib):
    """MXFP4 operands: MX scales only, FP4 x FP4 only, K counted in elements with
    two codes per byte; all checked before any HIP call."""
    run = lambda **kw: _run_ex(lib, **{"fa": 4, "fb": 4, "mode": 2, "K": 256, "lda": 128,
                                       "ldb": 128, **kw})
    assert run(M=0) == SUCCESS
    assert run(mode=1) == NOT_SUPPORTED                # row-wise FP4
    assert run(mode=0) == NOT_SUPPORTED                # per-tensor FP4
    assert run(fb=0) == NOT_SUPPORTED                  # FP4 x e4m3
    assert run(fa=1) == NOT_SUPPORTED                  # e5m2 x FP4
    assert run(lda=112) == INVALID                     # lda < K/2 bytes
    assert run(K=240, lda=128, ldb=128) == NOT_SUPPORTED   # K % 32
    assert run(lda=136) == MISALIGNED
    assert _run_ex(lib, fa=3) == NOT_SUPPORTED         # e3m2 x e4m3: no such pairing
    assert _run_ex(lib, fa=7) == INVALID               # no format 7
    q = lambda **kw: lib.fp8gemm_quantize_ex(P, 64, kw.get("k", 256), 256, kw.get("mode", 2), 4,
                                             P2, kw.get("ldq", 128), P3, 0, 0, None)
    assert q(mode=1) == NOT_SUPPORTED
    assert q(mode=0) == NOT_SUPPORTED
    assert q(ldq=112) == INVALID                       # ldq < k/2 bytes
    assert q(ldq=136) == MISALIGNED
    assert q(k=48) == NOT_SUPPORTED                    # MX: k % 32
    # (row-major FP4 B: test_row_major_b_fp4_validation)


def test_grouped_fp4_validation(lib):
    """fp8gemm_grouped_run_ex: e4m3 experts or MXFP4 activations and experts only."""
    def run(fa=4, fb=4, mode=2, K=256, lda=128, ldb=128, stride_b=64 * 128, **kw):
        return lib.fp8gemm_grouped_run_ex(2, kw.get("total_m", 64), 64, K, P, lda, fa, P3, P2, ldb,
                                          fb, stride_b, mode, P3 + 256, P3 + 512, P3 + 4096, 64, 1,
                                          0, 0, None)
    assert run(total_m=0) == SUCCESS
    assert run(mode=1) == NOT_SUPPORTED                  # FP4 needs MX scales
    assert run(fb=0) == NOT_SUPPORTED                    # FP4 x e4m3
    assert run(fa=1, fb=1, lda=256, ldb=256, stride_b=64 * 256) == NOT_SUPPORTED   # e5m2 experts
    assert run(lda=112) == INVALID                       # lda < K/2 bytes
    assert run(stride_b=64 * 128 - 16) == INVALID        # experts overlap
    assert run(fa=7) == INVALID


def test_mxout_validation(lib):
    """fp8gemm_run_mxout: e4m3 codes plus E8M0 per 32 columns; checked before any HIP call."""
    def run(N=64, C=P3 + 4096, ldc=64, cs=P3 + 65536, ldcs=2, **kw):
        return lib.fp8gemm_run_mxout(kw.get("M", 64), N, 128, P, 128, kw.get("fa", 0), P2, 128,
                                     kw.get("fb", 0), kw.get("mode", 1), P3, P3 + 256, 0, 0, C,
                                     ldc, cs, ldcs, 0, 0, None)
    assert run(M=0) == SUCCESS
    assert run(cs=0) == INVALID
    assert run(ldcs=1) == INVALID                 # ldcs < N/32
    assert run(N=48, ldc=48) == NOT_SUPPORTED     # N % 32
    assert run(ldc=72) == MISALIGNED              # byte rows of codes: ldc % 16
    assert run(ldc=32) == INVALID                 # ldc < N
    assert run(C=P3 + 4100) == MISALIGNED
    assert run(mode=7) == INVALID


def test_qout_validation(lib):
    """fp8gemm_run_qout: codes with a fresh per-tensor / per-row scale; every check
    runs before any HIP call (a failing one means nothing was enqueued)."""
    M, N, K = 64, 64, 128
    need = F.fp8gemm_qout_workspace_size(M, N, K, 1)

    def run(N=N, C=P3 + 4096, ldc=64, cs=P3 + 65536, om=1, cf=0, ws=0x100000, wsb=need, **kw):
        return lib.fp8gemm_run_qout(kw.get("M", M), N, K, P, 128, kw.get("fa", 0), P2, 128,
                                    kw.get("fb", 0), kw.get("mode", 1), P3, P3 + 256, 0,
                                    kw.get("act", 0), om, cf, C, ldc, cs, ws, wsb, None)
    assert run(M=0) == SUCCESS and run(N=0, ldc=16) == SUCCESS
    assert run(om=2) == INVALID                   # MX blocks: fp8gemm_run_mxout
    assert run(om=5) == INVALID and run(cf=9) == INVALID
    assert run(cf=4) == NOT_SUPPORTED             # FP4 codes out
    assert run(cs=0) == INVALID
    assert run(C=0) == INVALID
    assert run(N=40, ldc=48) == NOT_SUPPORTED     # N % 16
    assert run(ldc=72) == MISALIGNED              # byte rows of codes: ldc % 16
    assert run(ldc=32) == INVALID                 # ldc < N
    assert run(C=P3 + 4100) == MISALIGNED
    assert run(cs=P3 + 65538) == MISALIGNED
    assert run(ws=0) == WORKSPACE and run(wsb=need - 1) == WORKSPACE
    assert run(ws=0x100008) == MISALIGNED
    assert run(mode=7) == INVALID and run(act=9) == INVALID
    assert run(fa=4) == NOT_SUPPORTED             # FP4 pairs with FP4 only
    # the workspace: the GEMM's own (at least its counters), M maxima, M x N bf16
    for shape, mode in [((64, 64, 128), 1), ((128, 4096, 4096), 2), ((8192, 8192, 8192), 0)]:
        m, n, k = shape
        q = F.fp8gemm_qout_workspace_size(m, n, k, mode)
        g = max(F.fp8gemm_workspace_size(m, n, k, mode), 4096)
        assert q >= g + 4 * m + 2 * m * n and q <= g + 4 * m + 2 * m * (n + 63) + 512
    assert F.fp8gemm_qout_workspace_size(0, 64, 128, 1) == 0


def test_row_major_b_validation(lib):
    """fp8gemm_run_kn, transposing form (K % 128 != 0): validated before any HIP
    call; the workspace holds B's copy."""
    need = F.fp8gemm_workspace_size_kn(64, 64, 144, 1)
    assert need >= 64 * 144
    assert F.fp8gemm_workspace_size_kn(64, 64, 144, 2) >= need + 64 * 4     # + MX codes
    assert F.fp8gemm_workspace_size_kn(64, 64, 144, 9) == 0
    assert F.fp8gemm_run_kn_path(64, 64, 144, 144, 64, 0, 0, 1) == "none"
    def run(B=P2, ldb=64, ws=P3 + (1 << 20), wsb=need, K=144, mode=1, **kw):
        return lib.fp8gemm_run_kn(kw.get("M", 64), 64, K, P, 144, 0, B, ldb, 0, mode, P3,
                                  P3 + 256, 0, 0, P3 + 4096, 64, 1, ws, wsb, None)
    assert run(M=0) == SUCCESS
    assert run(B=0) == INVALID
    assert run(ldb=32) == INVALID                                 # ldb < N
    assert run(ldb=72) == MISALIGNED
    assert run(B=P2 + 8) == MISALIGNED
    assert run(ws=0) == WORKSPACE
    assert run(wsb=need - 16) == WORKSPACE
    assert run(ws=P3 + (1 << 20) + 8) == MISALIGNED
    assert run(K=120) == NOT_SUPPORTED


def test_row_major_b_fp4_validation(lib):
    """fp8gemm_run_kn with MXFP4 operands (always the transposing form): B packs two
    codes per byte along N, so ldb >= N/2; MX only, FP4 with FP4 only, no FP6."""
    need = F.fp8gemm_workspace_size_kn(64, 64, 128, 2)
    assert need >= 64 * 128 // 2 + 64 * 4
    def run(ldb=32, fa=4, fb=4, mode=2, K=128, wsb=need, **kw):
        return lib.fp8gemm_run_kn(kw.get("M", 64), 64, K, P, 64, fa, P2, ldb, fb, mode, P3,
                                  P3 + 256, 0, 0, P3 + 4096, 64, 1, P3 + (1 << 20), wsb, None)
    assert run(M=0) == SUCCESS
    assert run(ldb=16) == INVALID                                  # 2 * ldb < N
    assert run(ldb=40) == MISALIGNED
    assert run(mode=1) == NOT_SUPPORTED                            # FP4: MX scales only
    assert run(fb=0) == NOT_SUPPORTED and run(fa=0) == NOT_SUPPORTED
    assert run(fa=2, fb=2) == NOT_SUPPORTED                        # FP6: no row-major B
    assert run(K=112) == NOT_SUPPORTED                              # K % 32
    assert run(wsb=need - 16) == WORKSPACE


@pytest.mark.parametrize("shape,ld,fa,fb,mode,path", [
    ((128, 4096, 4096), None, "e4m3", "e4m3", "tensor", "splitk"),
    ((128, 4096, 4096), None, "e5m2", "e4m3", "mx32", "splitk"),
    ((4096, 4096, 4096), None, "e4m3", "e4m3", "rowwise", "tile256"),
    ((16384, 8192, 512), None, "e4m3", "e4m3", "tensor", "tile256"),     # never persistent
    ((2048, 4096, 1024), None, "e4m3", "e5m2", "mx32", "tile128"),
    ((300, 520, 384), None, "e5m2", "e5m2", "rowwise", "tile128"),         # edge tiles
    ((2048, 4096, 4160), None, "e4m3", "e4m3", "tensor", "none"),          # K % 128
    ((2048, 4096, 1152), None, "e4m3", "e4m3", "mx32", "none"),            # MX: K % 512
    ((2048, 4112, 1024), None, "e4m3", "e4m3", "mx32", "tile128"),         # MX: N % 16 == 0
    ((2048, 4100, 1024), (1024, 4112), "e4m3", "e4m3", "mx32", "none"),    # MX: N % 16
    ((2048, 4100, 1024), (1024, 4112), "e4m3", "e4m3", "tensor", "tile128"),
    ((256, 256, 1 << 19), (1 << 19, 8192), "e4m3", "e4m3", "tensor", "none"),  # K * ldb >= 2^31
    ((128, 4096, 4096), (2048, 2048), "e2m1", "e2m1", "mx32", "splitk"),   # MXFP4 (packed rows)
    ((4096, 4096, 4096), (2048, 2048), "e2m1", "e2m1", "mx32", "tile256"),
    ((300, 528, 1024), (512, 272), "e2m1", "e2m1", "mx32", "tile128"),
    ((2048, 4096, 4160), (2080, 2048), "e2m1", "e2m1", "mx32", "none"),    # K % 512
    ((2048, 4098, 1024), (512, 2064), "e2m1", "e2m1", "mx32", "none"),     # odd bytes: N % 16
    ((2048, 4096, 1024), (512, 2048), "e2m1", "e2m1", "rowwise", "none"),  # FP4: MX only
    ((2048, 4096, 1024), (768, 3072), "e2m3", "e2m3", "mx32", "none"),     # no FP6 here
    ((0, 4096, 4096), None, "e4m3", "e4m3", "tensor", "none"),
])
def test_row_major_b_in_kernel_rules(lib, shape, ld, fa, fb, mode, path):
    """Which shapes fp8gemm_run_kn serves with the transposing LDS reads (the query
    runs the same planner as the call)."""
    M, N, K = shape
    lda, ldb = ld if ld else (K, N)
    assert F.fp8gemm_run_kn_path(M, N, K, lda, ldb, F.FORMATS[fa], F.FORMATS[fb],
                                 F.SCALE_MODES[mode]) == path


def test_row_major_b_in_kernel_validation(lib):
    """fp8gemm_run_kn, in-kernel form (K % 128 == 0): the dense GEMM's checks and
    only the dense GEMM's workspace, all before any HIP call."""
    M, N, K = 128, 4096, 4096                      # split-K: needs the dense workspace
    need = F.fp8gemm_workspace_size(M, N, K, 0)
    assert need > 0 and F.fp8gemm_workspace_size_kn(M, N, K, 0) > need
    def run(A=P, lda=K, ldb=N, ws=P3 + (1 << 20), wsb=need, C=P3 + 4096, ldc=N, bias=0,
            sb=P3 + 256, **kw):
        return lib.fp8gemm_run_kn(kw.get("M", M), N, K, A, lda, 0, P2, ldb, 0, 0, P3, sb, bias,
                                  0, C, ldc, 1, ws, wsb, None)
    assert F.fp8gemm_run_kn_path(M, N, K, K, N, 0, 0, 0) == "splitk"
    assert run(M=0) == SUCCESS
    assert run(ws=0) == WORKSPACE
    assert run(wsb=need - 16) == WORKSPACE
    assert run(ws=P3 + (1 << 20) + 8) == MISALIGNED
    assert run(A=0) == INVALID
    assert run(lda=K - 16) == INVALID                  # lda < K
    assert run(A=P + 8) == MISALIGNED
    assert run(C=0) == INVALID
    assert run(ldc=N - 8) == INVALID
    assert run(C=P3 + 4100) == MISALIGNED
    assert run(bias=P3 + 2) == MISALIGNED
    assert run(sb=P3 + 258) == MISALIGNED


def test_run_split_workspace_validation(lib):
    """Split-K shapes need the queried workspace, 16-byte aligned; checked before any launch."""
    M, N, K = 128, 4096, 4096
    need = F.fp8gemm_workspace_size(M, N, K, 0)
    assert need > 0
    args = (M, N, K, P, K, P2, K, 0, P3, P3 + 64, P3 + 4096, N, 1)
    assert lib.fp8gemm_run(*args, 0, 0, None) == WORKSPACE
    assert lib.fp8gemm_run(*args, P3 + (1 << 20), need - 1, None) == WORKSPACE
    assert lib.fp8gemm_run(*args, P3 + (1 << 20) + 8, need, None) == MISALIGNED


def _grouped(lib, G=8, total_m=256, N=64, K=128, A=P, lda=128, off=P3 + 8192, B=P2, ldb=128,
             stride_b=64 * 128, mode=1, sa=P3, sb=P3 + 1024, C=P3 + 16384, ldc=64, out=1):
    return lib.fp8gemm_grouped_run(G, total_m, N, K, A, lda, off, B, ldb, stride_b, mode, sa, sb,
                                   C, ldc, out, 0, 0, None)


def test_grouped_validation(lib):
    assert _grouped(lib, G=0) == INVALID
    assert _grouped(lib, G=2000) == NOT_SUPPORTED
    assert _grouped(lib, G=1025) == NOT_SUPPORTED          # the documented maximum is 1024
    assert _grouped(lib, mode=5) == INVALID
    assert _grouped(lib, total_m=-1) == INVALID
    assert _grouped(lib, total_m=0) == SUCCESS
    assert _grouped(lib, N=0) == SUCCESS
    assert _grouped(lib, off=0) == INVALID
    assert _grouped(lib, stride_b=64 * 128 - 16) == INVALID
    assert _grouped(lib, stride_b=64 * 128 + 8) == MISALIGNED
    assert _grouped(lib, off=P3 + 8192 + 2) == MISALIGNED
    assert _grouped(lib, K=100, lda=128, ldb=128) == NOT_SUPPORTED
    assert _grouped(lib, A=P + 8) == MISALIGNED


def test_python_wrapper_raises(lib):
    with pytest.raises(F.Fp8GemmError) as ei:
        F.fp8gemm_run(-1, 1, 16, P, 16, P, 16, 0, P, P, P, 16, 0, 0, 0, 0)
    assert ei.value.status == INVALID
