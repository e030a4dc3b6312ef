"""Python binding of libfp8gemm: the MI355X (gfx950) scaled FP8 GEMM library.

Two layers, both argument marshalling only (every step of the computation runs
in the library's HIP kernels; there is no fallback):

* ``fp8gemm_quantize``, ``fp8gemm_run``, ``fp8gemm_grouped_run`` and the
  workspace-size queries mirror the C ABI in ``include/fp8gemm.h`` one to one:
  device pointers and sizes as Python ints, a non-success status raises
  :class:`Fp8GemmError`.
* ``quantize``, ``gemm`` and ``grouped_gemm`` take PyTorch CUDA tensors
  (PyTorch supplies device memory and the current stream), allocate the outputs
  and call the ABI functions.

Layouts: A is row-major [M, K]; B is column-major [K, N], passed as its
[N, K] row-major transpose; C is row-major [M, N].  Operand codes are OCP
e4m3fn bytes held in ``torch.uint8`` tensors.
"""
from __future__ import annotations

import ctypes
import functools
import os
import re

__all__ = [
    "gemm_workspace",
    "Fp8GemmError", "SCALE_MODES", "OUT_DTYPES", "FORMATS", "ACTIVATIONS", "library_path",
    "load_library", "fp8gemm_quantize_workspace_size", "fp8gemm_quantize",
    "fp8gemm_quantize_ex", "fp8gemm_workspace_size", "fp8gemm_run", "fp8gemm_run_ex",
    "fp8gemm_run_mxout", "fp8gemm_qout_workspace_size", "fp8gemm_run_qout",
    "fp8gemm_workspace_size_kn", "fp8gemm_run_kn",
    "fp8gemm_grouped_workspace_size", "fp8gemm_grouped_run",
    "fp8gemm_run_path", "fp8gemm_run_kn_path", "PATHS", "fp8gemm_run_noalloc", "NOALLOC_SCRATCH_BYTES",
    "fp8gemm_status_string", "fp8gemm_version", "quantize", "gemm", "gemm_mxout", "gemm_qout",
    "grouped_gemm",
    "exported_symbols",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "fp8gemm.h")

SCALE_MODES = {"tensor": 0, "rowwise": 1, "mx32": 2}
OUT_DTYPES = {"f16": 0, "bf16": 1}
# e2m3 / e3m2: FP6, four codes in three bytes; e2m1: FP4, two codes per byte (MX only)
FORMATS = {"e4m3": 0, "e5m2": 1, "e2m3": 2, "e3m2": 3, "e2m1": 4}
# bits of one code
CODE_BITS = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}
ACTIVATIONS = {"none": 0, "relu": 1, "gelu": 2, "silu": 3}

# FP8GEMM_NOALLOC_SCRATCH_BYTES: the static scratch of fp8gemm_run_noalloc
NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024 + 4096

# kernel paths of a dense GEMM (fp8gemm_run_path)
PATHS = {0: "none", 1: "splitk", 2: "tile128", 3: "tile256", 4: "persistent"}

_STATUS_NAMES = {
    0: "FP8GEMM_SUCCESS", 1: "FP8GEMM_ERROR_INVALID_VALUE", 2: "FP8GEMM_ERROR_MISALIGNED",
    3: "FP8GEMM_ERROR_NOT_SUPPORTED", 4: "FP8GEMM_ERROR_WORKSPACE", 5: "FP8GEMM_ERROR_LAUNCH",
}


class Fp8GemmError(RuntimeError):
    """A libfp8gemm call returned a non-success status."""

    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {_STATUS_NAMES.get(status, status)}")


def library_path() -> str:
    return os.path.join(_PKG, "libfp8gemm.so")


_lib = None

_i64, _i32, _sz, _p, _int = (ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p,
                             ctypes.c_int)

_SIGNATURES = {
    "fp8gemm_quantize_workspace_size": (_sz, [_i64, _i64, _int]),
    "fp8gemm_quantize": (_int, [_p, _i64, _i64, _i64, _int, _p, _i64, _p, _p, _sz, _p]),
    "fp8gemm_quantize_ex": (_int, [_p, _i64, _i64, _i64, _int, _int, _p, _i64, _p, _p, _sz, _p]),
    "fp8gemm_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "fp8gemm_run": (_int, [_i64, _i64, _i64, _p, _i64, _p, _i64, _int, _p, _p, _p, _i64, _int,
                           _p, _sz, _p]),
    "fp8gemm_run_ex": (_int, [_i64, _i64, _i64, _p, _i64, _int, _p, _i64, _int, _int, _p, _p, _p,
                              _int, _p, _i64, _int, _p, _sz, _p]),
    "fp8gemm_run_mxout": (_int, [_i64, _i64, _i64, _p, _i64, _int, _p, _i64, _int, _int, _p, _p,
                                 _p, _int, _p, _i64, _p, _i64, _p, _sz, _p]),
    "fp8gemm_qout_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "fp8gemm_run_qout": (_int, [_i64, _i64, _i64, _p, _i64, _int, _p, _i64, _int, _int, _p, _p,
                                _p, _int, _int, _int, _p, _i64, _p, _p, _sz, _p]),
    "fp8gemm_workspace_size_kn": (_sz, [_i64, _i64, _i64, _int]),
    "fp8gemm_run_kn": (_int, [_i64, _i64, _i64, _p, _i64, _int, _p, _i64, _int, _int, _p, _p, _p,
                              _int, _p, _i64, _int, _p, _sz, _p]),
    "fp8gemm_grouped_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _int]),
    "fp8gemm_grouped_run": (_int, [_i32, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _i64, _int,
                                   _p, _p, _p, _i64, _int, _p, _sz, _p]),
    "fp8gemm_grouped_run_ex": (_int, [_i32, _i64, _i64, _i64, _p, _i64, _int, _p, _p, _i64, _int,
                                      _i64, _int, _p, _p, _p, _i64, _int, _p, _sz, _p]),
    "fp8gemm_run_path": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int, _int, _int]),
    "fp8gemm_run_kn_path": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int, _int]),
    "fp8gemm_run_noalloc": (_int, [_i64, _i64, _i64, _p, _i64, _int, _p, _i64, _int, _int, _p, _p,
                                   _p, _int, _p, _i64, _int, _p]),
    "fp8gemm_status_string": (ctypes.c_char_p, [_int]),
    "fp8gemm_version": (_int, []),
}


def load_library():
    """Load libfp8gemm.so from this package directory (built in-tree).

    Raises RuntimeError when it has not been built: there is no other path.
    """
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m block_scaled_gemm_fp8gemm_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols() -> list:
    """Function names declared in include/fp8gemm.h."""
    with open(_HEADER) as fh:
        text = fh.read()
    return re.findall(r"^\s*(?:size_t|fp8gemm_status|const char\*|int)\s+(fp8gemm_\w+)\s*\(",
                      text, flags=re.M)


def _check(name: str, status: int):
    if status != 0:
        raise Fp8GemmError(name, status)


# ---- one-to-one ABI mirrors -------------------------------------------------
def fp8gemm_quantize_workspace_size(rows: int, k: int, mode: int) -> int:
    return load_library().fp8gemm_quantize_workspace_size(rows, k, mode)


def fp8gemm_quantize(x: int, rows: int, k: int, ldx: int, mode: int, q: int, ldq: int,
                     scales: int, workspace: int, workspace_bytes: int, stream: int) -> None:
    _check("fp8gemm_quantize", load_library().fp8gemm_quantize(
        x, rows, k, ldx, mode, q, ldq, scales, workspace, workspace_bytes, stream))


def fp8gemm_quantize_ex(x: int, rows: int, k: int, ldx: int, mode: int, fmt: int, q: int,
                        ldq: int, scales: int, workspace: int, workspace_bytes: int,
                        stream: int) -> None:
    _check("fp8gemm_quantize_ex", load_library().fp8gemm_quantize_ex(
        x, rows, k, ldx, mode, fmt, q, ldq, scales, workspace, workspace_bytes, stream))


def fp8gemm_workspace_size(M: int, N: int, K: int, mode: int) -> int:
    return load_library().fp8gemm_workspace_size(M, N, K, mode)


def fp8gemm_run(M: int, N: int, K: int, A: int, lda: int, B: int, ldb: int, mode: int,
                scale_a: int, scale_b: int, C: int, ldc: int, out_dtype: int, workspace: int,
                workspace_bytes: int, stream: int) -> None:
    _check("fp8gemm_run", load_library().fp8gemm_run(
        M, N, K, A, lda, B, ldb, mode, scale_a, scale_b, C, ldc, out_dtype, workspace,
        workspace_bytes, stream))


def fp8gemm_run_ex(M: int, N: int, K: int, A: int, lda: int, a_format: int, B: int, ldb: int,
                   b_format: int, mode: int, scale_a: int, scale_b: int, bias: int,
                   activation: int, C: int, ldc: int, out_dtype: int, workspace: int,
                   workspace_bytes: int, stream: int) -> None:
    _check("fp8gemm_run_ex", load_library().fp8gemm_run_ex(
        M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias, activation, C,
        ldc, out_dtype, workspace, workspace_bytes, stream))


def fp8gemm_run_mxout(M: int, N: int, K: int, A: int, lda: int, a_format: int, B: int, ldb: int,
                      b_format: int, mode: int, scale_a: int, scale_b: int, bias: int,
                      activation: int, C: int, ldc: int, c_scales: int, ldcs: int,
                      workspace: int, workspace_bytes: int, stream: int) -> None:
    _check("fp8gemm_run_mxout", load_library().fp8gemm_run_mxout(
        M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias, activation, C,
        ldc, c_scales, ldcs, workspace, workspace_bytes, stream))


def fp8gemm_qout_workspace_size(M: int, N: int, K: int, mode: int) -> int:
    return load_library().fp8gemm_qout_workspace_size(M, N, K, mode)


def fp8gemm_run_qout(M: int, N: int, K: int, A: int, lda: int, a_format: int, B: int, ldb: int,
                     b_format: int, mode: int, scale_a: int, scale_b: int, bias: int,
                     activation: int, out_mode: int, c_format: int, C: int, ldc: int,
                     c_scales: int, workspace: int, workspace_bytes: int, stream: int) -> None:
    _check("fp8gemm_run_qout", load_library().fp8gemm_run_qout(
        M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias, activation,
        out_mode, c_format, C, ldc, c_scales, workspace, workspace_bytes, stream))


def fp8gemm_workspace_size_kn(M: int, N: int, K: int, mode: int) -> int:
    return load_library().fp8gemm_workspace_size_kn(M, N, K, mode)


def fp8gemm_run_kn(M: int, N: int, K: int, A: int, lda: int, a_format: int, B: int, ldb: int,
                   b_format: int, mode: int, scale_a: int, scale_b: int, bias: int,
                   activation: int, C: int, ldc: int, out_dtype: int, workspace: int,
                   workspace_bytes: int, stream: int) -> None:
    _check("fp8gemm_run_kn", load_library().fp8gemm_run_kn(
        M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias, activation, C,
        ldc, out_dtype, workspace, workspace_bytes, stream))


def fp8gemm_grouped_workspace_size(num_groups: int, total_m: int, N: int, K: int,
                                   mode: int) -> int:
    return load_library().fp8gemm_grouped_workspace_size(num_groups, total_m, N, K, mode)


def fp8gemm_grouped_run(num_groups: int, total_m: int, N: int, K: int, A: int, lda: int,
                        offsets: int, B: int, ldb: int, stride_b: int, mode: int, scale_a: int,
                        scale_b: int, C: int, ldc: int, out_dtype: int, workspace: int,
                        workspace_bytes: int, stream: int) -> None:
    _check("fp8gemm_grouped_run", load_library().fp8gemm_grouped_run(
        num_groups, total_m, N, K, A, lda, offsets, B, ldb, stride_b, mode, scale_a, scale_b, C,
        ldc, out_dtype, workspace, workspace_bytes, stream))


def fp8gemm_grouped_run_ex(num_groups: int, total_m: int, N: int, K: int, A: int, lda: int,
                           a_format: int, offsets: int, B: int, ldb: int, b_format: int,
                           stride_b: int, mode: int, scale_a: int, scale_b: int, C: int, ldc: int,
                           out_dtype: int, workspace: int, workspace_bytes: int,
                           stream: int) -> None:
    _check("fp8gemm_grouped_run_ex", load_library().fp8gemm_grouped_run_ex(
        num_groups, total_m, N, K, A, lda, a_format, offsets, B, ldb, b_format, stride_b, mode,
        scale_a, scale_b, C, ldc, out_dtype, workspace, workspace_bytes, stream))


def fp8gemm_run_noalloc(M: int, N: int, K: int, A: int, lda: int, a_format: int, B: int,
                        ldb: int, b_format: int, mode: int, scale_a: int, scale_b: int, bias: int,
                        activation: int, C: int, ldc: int, out_dtype: int, stream: int) -> None:
    _check("fp8gemm_run_noalloc", load_library().fp8gemm_run_noalloc(
        M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias, activation, C,
        ldc, out_dtype, stream))


def fp8gemm_run_path(M: int, N: int, K: int, lda: int, ldb: int, a_format: int, b_format: int,
                     mode: int, fused: int) -> str:
    """Name of the kernel path a dense GEMM call of this shape takes (see PATHS)."""
    return PATHS[load_library().fp8gemm_run_path(M, N, K, lda, ldb, a_format, b_format, mode,
                                                 fused)]


def fp8gemm_run_kn_path(M: int, N: int, K: int, lda: int, ldb: int, a_format: int,
                        b_format: int, mode: int) -> str:
    """Kernel path of fp8gemm_run_kn's in-kernel form for this shape ("none": the
    call makes B K-contiguous in the workspace first)."""
    return PATHS[load_library().fp8gemm_run_kn_path(M, N, K, lda, ldb, a_format, b_format, mode)]


def fp8gemm_status_string(status: int) -> str:
    return load_library().fp8gemm_status_string(status).decode()


def fp8gemm_version() -> int:
    return load_library().fp8gemm_version()


# ---- PyTorch conveniences ---------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _require_cuda(t, name, dtype=None, dim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D")
    if t.dim() and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")


_WORKSPACES = {}


def gemm_workspace(device, nbytes: int):
    """A zero-filled device workspace of at least `nbytes`, cached per (device,
    current stream).

    The split-K GEMM keeps per-tile arrival counters and fp32 partial tiles at
    fixed places of its workspace: the counters must be zero before the first
    call and every call leaves them zero, so one buffer serves every call that
    cannot run concurrently with another one on it, i.e. the calls of one stream.
    Calls on different streams get different buffers.  Each buffer is allocated
    (and zero-filled) on its own stream, so PyTorch's caching allocator reuses a
    replaced, smaller buffer only after the work already queued on that stream.
    """
    torch = _torch()
    dev = torch.device(device)
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _WORKSPACES[key] = ws
    return ws


def _ptr(t) -> int:
    return t.data_ptr() if t is not None else 0


def quantize(x, mode: str = "tensor", out=None, scales=None, workspace=None,
             fmt: str = "e4m3"):
    """fp32 [R, K] CUDA tensor -> (codes uint8 [R, K], scales).

    scales: float32 [1] (tensor), float32 [R] (rowwise) or uint8 [R, K/32] (mx32);
    fmt: element format of the codes, "e4m3", "e5m2", or with mx32 "e2m1" (FP4,
    codes packed two per byte, uint8 [R, K/2]) or "e2m3" / "e3m2" (FP6, four codes
    in three bytes, uint8 [R, 3K/4]).
    """
    torch = _torch()
    _require_cuda(x, "x", torch.float32, 2)
    m = SCALE_MODES[mode]
    R, K = x.shape
    if out is None:
        kb = K * CODE_BITS[fmt] // 8                  # bytes of a row of codes
        ldq = (kb + 15) // 16 * 16
        out = torch.empty((R, ldq), dtype=torch.uint8, device=x.device)[:, :kb]
    if scales is None:
        if mode == "tensor":
            scales = torch.empty(1, dtype=torch.float32, device=x.device)
        elif mode == "rowwise":
            scales = torch.empty(R, dtype=torch.float32, device=x.device)
        else:
            scales = torch.empty((R, K // 32), dtype=torch.uint8, device=x.device)
    need = fp8gemm_quantize_workspace_size(R, K, m)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    fp8gemm_quantize_ex(_ptr(x), R, K, x.stride(0), m, FORMATS[fmt], _ptr(out), out.stride(0),
                        _ptr(scales), _ptr(workspace) if need else 0,
                        workspace.numel() if need else 0, _stream_handle(x.device))
    return out, scales


@functools.lru_cache(maxsize=256)
def _gemm_workspace_need(M, N, K, lda, ldb, a_format, b_format, mode, kn):
    """Workspace bytes of a dense GEMM call: row-major B read in the kernels needs
    only the GEMM's own workspace, the transposing form also B's copy."""
    if kn and fp8gemm_run_kn_path(M, N, K, lda, ldb, a_format, b_format, mode) == "none":
        return fp8gemm_workspace_size_kn(M, N, K, mode)
    return fp8gemm_workspace_size(M, N, K, mode)


def gemm(qa, sa, qb, sb, mode: str = "tensor", out_dtype: str = "bf16", out=None,
         workspace=None, fmt_a: str = "e4m3", fmt_b: str = "e4m3", bias=None,
         activation: str = "none", b_layout: str = "nk"):
    """C [M, N] = act(dq(qa [M, K]) @ dq(qb) + bias), returned as fp16 / bf16.

    qb is [N, K] (K contiguous, b_layout "nk") or [K, N] (N contiguous, "kn"; its
    MX codes sb then [K/32, N]).  fmt_a / fmt_b: element formats of the codes:
    "e4m3" or "e5m2" in any pairing; "e2m1" for both (FP4 packed two per byte, so
    qa is [M, K/2] and qb [N, K/2], or [K, N/2] with b_layout "kn" and N even;
    mode "mx32"); or "e2m3" / "e3m2" for both (FP6, four codes in three bytes:
    [M, 3K/4] and [N, 3K/4]; mode "mx32", K % 128 == 0).
    bias: float32 [N] CUDA tensor or None;
    activation: "none", "relu", "gelu" or "silu".
    """
    torch = _torch()
    _require_cuda(qa, "qa", torch.uint8, 2)
    _require_cuda(qb, "qb", torch.uint8, 2)
    M, K = qa.shape
    K = K * 8 // CODE_BITS[fmt_a]           # packed codes: K counts elements
    if b_layout == "kn":                    # packed FP4 B: two codes per byte along N
        Kb, N = qb.shape
        N = N * 8 // CODE_BITS[fmt_b]
    else:
        N, Kb = qb.shape
        Kb = Kb * 8 // CODE_BITS[fmt_b]
    if K != Kb:
        raise ValueError("qa and qb must share K")
    tdt = torch.float16 if out_dtype == "f16" else torch.bfloat16
    if out is None:
        ldc = (N + 7) // 8 * 8
        out = torch.empty((M, ldc), dtype=tdt, device=qa.device)[:, :N]
    m = SCALE_MODES[mode]
    kn = b_layout == "kn"
    need = _gemm_workspace_need(M, N, K, qa.stride(0), qb.stride(0), FORMATS[fmt_a],
                                FORMATS[fmt_b], m, kn)
    if need and workspace is None:
        workspace = gemm_workspace(qa.device, need)
    if bias is not None:
        _require_cuda(bias, "bias", torch.float32, 1)
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
    (fp8gemm_run_kn if kn else fp8gemm_run_ex)(
                   M, N, K, _ptr(qa), qa.stride(0), FORMATS[fmt_a], _ptr(qb), qb.stride(0),
                   FORMATS[fmt_b], m, _ptr(sa), _ptr(sb), _ptr(bias), ACTIVATIONS[activation],
                   _ptr(out), out.stride(0), OUT_DTYPES[out_dtype],
                   _ptr(workspace) if need else 0, workspace.numel() if need else 0,
                   _stream_handle(qa.device))
    return out


def gemm_mxout(qa, sa, qb, sb, mode: str = "tensor", out=None, out_scales=None,
               workspace=None, fmt_a: str = "e4m3", fmt_b: str = "e4m3", bias=None,
               activation: str = "none"):
    """(codes uint8 [M, N], E8M0 uint8 [M, N/32]): y = act(dq(qa) @ dq(qb) + bias)
    quantised for the next layer, e4m3 with one E8M0 scale per 32 columns (the
    MX rule of ``quantize``); N must be a multiple of 32.  Operands as ``gemm``
    (qb [N, K], K contiguous)."""
    torch = _torch()
    _require_cuda(qa, "qa", torch.uint8, 2)
    _require_cuda(qb, "qb", torch.uint8, 2)
    M, K = qa.shape
    N, Kb = qb.shape
    K, Kb = K * 8 // CODE_BITS[fmt_a], Kb * 8 // CODE_BITS[fmt_b]
    if K != Kb:
        raise ValueError("qa and qb must share K")
    if out is None:
        ldc = (N + 15) // 16 * 16
        out = torch.empty((M, ldc), dtype=torch.uint8, device=qa.device)[:, :N]
    if out_scales is None:
        out_scales = torch.empty((M, N // 32), dtype=torch.uint8, device=qa.device)
    m = SCALE_MODES[mode]
    need = fp8gemm_workspace_size(M, N, K, m)
    if need and workspace is None:
        workspace = gemm_workspace(qa.device, need)
    if bias is not None:
        _require_cuda(bias, "bias", torch.float32, 1)
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
    fp8gemm_run_mxout(M, N, K, _ptr(qa), qa.stride(0), FORMATS[fmt_a], _ptr(qb), qb.stride(0),
                      FORMATS[fmt_b], m, _ptr(sa), _ptr(sb), _ptr(bias), ACTIVATIONS[activation],
                      _ptr(out), out.stride(0), _ptr(out_scales),
                      out_scales.stride(0) if out_scales.dim() == 2 else max(N // 32, 1),
                      _ptr(workspace) if need else 0, workspace.numel() if need else 0,
                      _stream_handle(qa.device))
    return out, out_scales


def gemm_qout(qa, sa, qb, sb, mode: str = "tensor", out_mode: str = "rowwise",
              out_fmt: str = "e4m3", out=None, out_scales=None, workspace=None,
              fmt_a: str = "e4m3", fmt_b: str = "e4m3", bias=None, activation: str = "none"):
    """(codes uint8 [M, N], scales float32 [M] or [1]): the bf16 output of ``gemm``
    (act(dq(qa) @ dq(qb) + bias)) quantised for the next layer with a fresh scale
    per row (out_mode "rowwise") or for the whole output ("tensor"), by the rule
    of ``quantize`` (bit-identical to ``quantize(gemm(...).float(), out_mode)``);
    out_fmt "e4m3" or "e5m2"; N must be a multiple of 16.  Operands as ``gemm``
    (qb [N, K], K contiguous).  The row scales are the scale_a of a row-wise GEMM
    that takes the codes as its A operand."""
    torch = _torch()
    _require_cuda(qa, "qa", torch.uint8, 2)
    _require_cuda(qb, "qb", torch.uint8, 2)
    M, K = qa.shape
    N, Kb = qb.shape
    K, Kb = K * 8 // CODE_BITS[fmt_a], Kb * 8 // CODE_BITS[fmt_b]
    if K != Kb:
        raise ValueError("qa and qb must share K")
    if out is None:
        ldc = (N + 15) // 16 * 16
        out = torch.empty((M, ldc), dtype=torch.uint8, device=qa.device)[:, :N]
    om = SCALE_MODES[out_mode]
    if out_scales is None:
        out_scales = torch.empty(M if out_mode == "rowwise" else 1, dtype=torch.float32,
                                 device=qa.device)
    m = SCALE_MODES[mode]
    need = fp8gemm_qout_workspace_size(M, N, K, m)
    if need and workspace is None:
        workspace = gemm_workspace(qa.device, need)
    if bias is not None:
        _require_cuda(bias, "bias", torch.float32, 1)
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
    fp8gemm_run_qout(M, N, K, _ptr(qa), qa.stride(0), FORMATS[fmt_a], _ptr(qb), qb.stride(0),
                     FORMATS[fmt_b], m, _ptr(sa), _ptr(sb), _ptr(bias), ACTIVATIONS[activation],
                     om, FORMATS[out_fmt], _ptr(out), out.stride(0), _ptr(out_scales),
                     _ptr(workspace) if need else 0, workspace.numel() if need else 0,
                     _stream_handle(qa.device))
    return out, out_scales


def grouped_gemm(qa, sa, offsets, qb, sb, mode: str = "rowwise", out_dtype: str = "bf16",
                 out=None, workspace=None, fmt: str = "e4m3"):
    """Grouped GEMM: rows [offsets[g], offsets[g+1]) of qa use expert qb[g] ([G, N, K]).

    fmt: "e4m3", or "e2m1" (MXFP4 activations and experts, mode "mx32", codes
    packed two per byte: qa [total_m, K/2], qb [G, N, K/2])."""
    torch = _torch()
    _require_cuda(qa, "qa", torch.uint8, 2)
    _require_cuda(qb, "qb", torch.uint8, 3)
    _require_cuda(offsets, "offsets", torch.int32, 1)
    total_m, K = qa.shape
    G, N, Kb = qb.shape
    if fmt == "e2m1":
        K, Kb = 2 * K, 2 * Kb
    if K != Kb or offsets.numel() != G + 1:
        raise ValueError("shape mismatch between qa, qb and offsets")
    tdt = torch.float16 if out_dtype == "f16" else torch.bfloat16
    if out is None:
        ldc = (N + 7) // 8 * 8
        out = torch.empty((total_m, ldc), dtype=tdt, device=qa.device)[:, :N]
    m = SCALE_MODES[mode]
    need = fp8gemm_grouped_workspace_size(G, total_m, N, K, m)
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=qa.device)
    fp8gemm_grouped_run_ex(G, total_m, N, K, _ptr(qa), qa.stride(0), FORMATS[fmt], _ptr(offsets),
                           _ptr(qb), qb.stride(1), FORMATS[fmt], qb.stride(0), m, _ptr(sa),
                           _ptr(sb), _ptr(out), out.stride(0), OUT_DTYPES[out_dtype],
                           _ptr(workspace) if need else 0, workspace.numel() if need else 0,
                           _stream_handle(qa.device))
    return out
