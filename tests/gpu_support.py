"""Helpers for the GPU parity tests: device transfer, announcements, comparisons.

Inputs come from ``workloads`` (seeded), expected values from ``oracle``; the
GPU path is only ever called through the C ABI via the package's binding.
"""
import sys

import numpy as np
import torch

import oracle as O

DEV = torch.device("cuda:0")


def announce(*parts):
    """Name the case about to run on the GPU (flushed, so a crash still shows it)."""
    print("[gpu]", *parts, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, pad_cols_to: int = 1) -> torch.Tensor:
    """Copy a 2-D host array to the device with its row pitch padded to a multiple."""
    a = np.ascontiguousarray(a)
    if a.ndim == 2 and pad_cols_to > 1:
        rows, cols = a.shape
        ld = (cols + pad_cols_to - 1) // pad_cols_to * pad_cols_to
        buf = torch.zeros((rows, ld), dtype=_torch_dtype(a.dtype), device=DEV)
        buf[:, :cols] = torch.from_numpy(a).to(DEV)
        return buf[:, :cols]
    return torch.from_numpy(a).to(DEV)


def _torch_dtype(dt):
    return {np.dtype(np.float32): torch.float32, np.dtype(np.uint8): torch.uint8,
            np.dtype(np.int32): torch.int32}[np.dtype(dt)]


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def scale_to_dev(s, mode: str) -> torch.Tensor:
    s = np.asarray(s)
    if mode == "tensor":
        return torch.tensor([float(s)], dtype=torch.float32, device=DEV)
    if mode == "rowwise":
        return torch.from_numpy(np.ascontiguousarray(s.astype(np.float32))).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(s.astype(np.uint8))).to(DEV)


def assert_within_bound(C_gpu: np.ndarray, C_ref: np.ndarray, abs_ref: np.ndarray, out: str,
                        what: str = ""):
    ok = O.within_bound(C_gpu, C_ref, abs_ref, out)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        tol = O.tolerance(C_ref, abs_ref, out)
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} outputs outside the bound; first at {i}: "
            f"gpu={C_gpu[i]!r} ref={C_ref[i]!r} tol={tol[i]!r}")
    assert np.all(np.isfinite(C_gpu)), f"{what}: non-finite output"
