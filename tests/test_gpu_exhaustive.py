"""Every non-negative finite fp32 input of the encoders, through the GPU quantisers.

The quantisers encode with gfx950's conversion instructions (e4m3, e5m2) or in
software (e2m1); the oracle encodes by searching the sorted table of the format's
values.  Here every fp32 bit pattern from +0 up to the format's largest value goes
through the GPU at scale 1 and is compared bit for bit with the oracle:

* e4m3 / e5m2, per-tensor scaling: every chunk also holds the format's largest
  value (448, 57344), so amax / max = 1 and the codes are encode(x) itself;
* e2m1 (MXFP4), e2m3 / e3m2 (MXFP6): every 32-element block starts with the
  format's largest value (6, 7.5, 28), so the block exponent is floor(log2 max)
  - emax = 0 (E8M0 code 127) and the codes are encode(x).

Negative inputs differ only in the sign bit, which both sides copy.  The oracle
side runs in a pool of worker processes, a chunk ahead of the GPU.
"""
import concurrent.futures as cf
import multiprocessing as mp

import numpy as np
import pytest
import torch

import block_scaled_gemm_fp8gemm_amd as F
import oracle as O
from exhaustive_inputs import (COLS, fp8_chunk as _fp8_chunk, mx_chunk as _mx_chunk,
                               oracle_fp8 as _oracle_fp8, oracle_mx as _oracle_mx)

from gpu_support import DEV, announce

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CHUNK = 1 << 26           # fp32 patterns per GPU call
WORKERS = 8               # oracle processes (started fresh: they never touch the GPU)


def _pool():
    return cf.ProcessPoolExecutor(WORKERS, mp_context=mp.get_context("spawn"))


def _first_mismatch(got, want, x):
    bad = np.flatnonzero(got != want)
    i = int(bad[0])
    return (f"{len(bad)} mismatches; first at x = {x[i]!r} (bits {x[i:i + 1].view(np.uint32)[0]:#010x}):"
            f" gpu {got[i]:#04x}, oracle {want[i]:#04x}")


@pytest.mark.parametrize("fmt,top", [("e4m3", 448.0), ("e5m2", 57344.0)])
def test_every_fp32_input_fp8(fmt, top):
    end = int(np.float32(top).view(np.uint32)) + 1
    starts = list(range(0, end, CHUNK))
    with _pool() as pool:
        futs = {s: pool.submit(_oracle_fp8, s, min(s + CHUNK, end), top, fmt)
                for s in starts[:WORKERS]}
        for n, s in enumerate(starts):
            e = min(s + CHUNK, end)
            if n + WORKERS < len(starts):
                s2 = starts[n + WORKERS]
                futs[s2] = pool.submit(_oracle_fp8, s2, min(s2 + CHUNK, end), top, fmt)
            x = _fp8_chunk(s, e, top)
            announce("exhaustive", fmt, f"patterns {s:#010x}..{e - 1:#010x}")
            xd = torch.from_numpy(x).to(DEV).view(-1, COLS)
            q, sc = F.quantize(xd, "tensor", fmt=fmt)
            assert float(sc.item()) == 1.0, f"scale {float(sc.item())}"
            got = q.cpu().numpy().reshape(-1)
            want = futs.pop(s).result()
            assert np.array_equal(got, want), _first_mismatch(got, want, x)
            del xd, q


@pytest.mark.parametrize("fmt,top", [("e2m1", 6.0), ("e2m3", 7.5), ("e3m2", 28.0)])
def test_every_fp32_input_mx_narrow(fmt, top):
    end = int(np.float32(top).view(np.uint32)) + 1
    step = CHUNK // 32 * 31
    starts = list(range(0, end, step))
    unpack = O.unpack_fp4 if fmt == "e2m1" else O.unpack_fp6
    with _pool() as pool:
        futs = {s: pool.submit(_oracle_mx, s, min(s + step, end), top, fmt)
                for s in starts[:WORKERS]}
        for n, s in enumerate(starts):
            e = min(s + step, end)
            if n + WORKERS < len(starts):
                s2 = starts[n + WORKERS]
                futs[s2] = pool.submit(_oracle_mx, s2, min(s2 + step, end), top, fmt)
            x = _mx_chunk(s, e, top)
            announce("exhaustive", fmt, f"patterns {s:#010x}..{e - 1:#010x}")
            xd = torch.from_numpy(x).to(DEV).view(-1, COLS)
            q, codes = F.quantize(xd, "mx32", fmt=fmt)
            assert np.all(codes.cpu().numpy() == 127), "block exponent of a block with the maximum"
            got = unpack(q.cpu().numpy()).reshape(-1)
            want = futs.pop(s).result()
            assert np.array_equal(got, want), _first_mismatch(got, want, x)
            del xd, q
