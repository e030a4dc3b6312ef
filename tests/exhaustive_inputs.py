"""Inputs of the exhaustive encoder test, and the oracle's codes for them (run in
worker processes, so this module imports neither torch nor the library).

A chunk holds the fp32 values with bit patterns lo .. hi - 1, laid out as the
test feeds them to the GPU quantiser."""
import numpy as np

import oracle as O

COLS = 1024               # row length of a chunk (32 MX blocks)


def patterns(lo: int, hi: int) -> np.ndarray:
    """fp32 values with bit patterns lo .. hi - 1."""
    return np.arange(lo, hi, dtype=np.uint32).view(np.float32)


def oracle_fp8(lo, hi, top, fmt):
    x = fp8_chunk(lo, hi, top)
    return O.encode(x, fmt)


def fp8_chunk(lo, hi, top):
    x = patterns(lo, hi)
    pad = (-len(x)) % COLS + COLS          # at least one element of padding holds `top`
    return np.concatenate([x, np.full(pad, top, np.float32)])


def mx_chunk(lo, hi, top=6.0):
    """Blocks of 32 whose first element is `top` (the format's largest value, so
    the shared exponent is 0) and whose other 31 are the patterns lo .. hi - 1."""
    x = patterns(lo, hi)
    blocks = -(-len(x) // 31)
    blocks += (-blocks) % (COLS // 32)
    buf = np.zeros((blocks, 32), np.float32)
    buf[:, 0] = top
    flat = buf[:, 1:].reshape(-1)
    flat[:len(x)] = x
    buf[:, 1:] = flat.reshape(blocks, 31)
    return buf.reshape(-1)


def oracle_mx(lo, hi, top, fmt):
    return O.encode(mx_chunk(lo, hi, top), fmt)


