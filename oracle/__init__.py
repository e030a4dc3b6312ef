"""CPU oracle for the scaled FP8 GEMM: TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 reference of what the GPU path computes: e4m3fn and E8M0
decoding by table, round-to-nearest-even encoding by table search, per-tensor,
row-wise and 32-element microscaled quantisation, the scaled GEMM with its
error bound, the fused bias-and-activation epilogue, the output quantised for
the next layer (MX blocks, or a fresh per-tensor / per-row scale), and the
grouped (mixture-of-experts) form.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The library under
``block_scaled_gemm_fp8gemm_amd`` never does, and this package imports nothing
from it: the two share no code.

Sources.  The pages behind this work name the formats but do not define them
bit by bit: "E4M3" and "E5M2" (the JAX/Triton Blackwell FP8 GEMM post, second
paragraph), the dtype ``torch.float8_e4m3fn`` (the Cutlass-named Triton FP8
post, parameter list, precision settings) and MXFP8 micro-scaling
("Hopper/Blackwell architecture features" §12.6.1, hardware table).  The bit
layouts therefore follow the public standards those names refer to: the OCP
8-bit floating point specification (OFP8: E4M3 with no infinities, one NaN
pattern per sign, max 448; E5M2 with IEEE-like infinities and NaNs, max 57344) and the OCP Microscaling (MX) formats
specification v1.0 (E8M0 shared scale, 32-element blocks, scale exponent =
floor(log2(amax)) - emax of the element format; the FP4 E2M1 element of
MXFP4, max 6, and the FP6 E2M3 / E3M2 elements of MXFP6, max 7.5 / 28, which
§12.6.1 of the architecture page lists next to FP8).

Parity pins.  Every function here is pinned by ``tests/test_oracle_*.py``
against exhaustive enumeration, exact rational arithmetic, integer-exact
products, closed forms or the specifications' tabulated points
(``tests/golden/``).  No function is "parity unpinned".
"""
from .formats import (E2M1_DECODE, E2M1_MAX, E2M3_DECODE, E2M3_MAX, E3M2_DECODE, E3M2_MAX,
                      E4M3_DECODE, E4M3_MAX, E5M2_DECODE, E5M2_MAX, E8M0_DECODE, FORMATS,
                      decode, decode_e2m1, decode_e2m3, decode_e3m2, decode_e4m3, decode_e5m2,
                      decode_e8m0, encode, encode_e2m1, encode_e2m3, encode_e3m2, encode_e4m3,
                      encode_e5m2, pack_fp4, pack_fp6, unpack_fp4, unpack_fp6)
from .quant import quantize, quantize_mx, quantize_rowwise, quantize_tensor
from .gemm import (ACT_LIPSCHITZ, activation, dequantize, epilogue_reference,
                   epilogue_tolerance, gemm_reference, grouped_reference, mx_output_reference,
                   mx_output_within_bound, output_ulp, scaled_output_reference,
                   scaled_output_within_bound, tolerance, within_bound, round_to_output)

__all__ = [
    "E2M1_DECODE", "E2M1_MAX", "decode_e2m1", "encode_e2m1", "pack_fp4", "unpack_fp4",
    "E2M3_DECODE", "E2M3_MAX", "E3M2_DECODE", "E3M2_MAX", "decode_e2m3", "decode_e3m2",
    "encode_e2m3", "encode_e3m2", "pack_fp6", "unpack_fp6",
    "E4M3_DECODE", "E4M3_MAX", "E5M2_DECODE", "E5M2_MAX", "E8M0_DECODE", "FORMATS", "decode",
    "decode_e4m3", "decode_e5m2", "decode_e8m0", "encode", "encode_e4m3", "encode_e5m2",
    "quantize", "quantize_mx", "quantize_rowwise", "quantize_tensor",
    "dequantize", "gemm_reference", "grouped_reference", "output_ulp", "tolerance",
    "within_bound", "round_to_output", "ACT_LIPSCHITZ", "activation", "epilogue_reference",
    "epilogue_tolerance", "mx_output_reference", "mx_output_within_bound",
    "scaled_output_reference", "scaled_output_within_bound",
]
