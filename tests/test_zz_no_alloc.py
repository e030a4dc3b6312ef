"""fp8gemm_run_noalloc (no workspace argument, a static device scratch) against
fp8gemm_run_ex (the caller's workspace) and the oracle.

Calls in a row on split-K shapes (the path that needs scratch), each smaller
than the one before it, in every scale mode: the output must be bit-identical to
fp8gemm_run_ex's (both run the same kernels) and within the GEMM bound of the
oracle.  A shape without split-K runs without touching the scratch, and a shape
whose split needs more than the scratch holds is rejected before any launch.
"""
import numpy as np
import pytest
import torch

import block_scaled_gemm_fp8gemm_amd as F
import oracle as O
from oracle import quant as Q
from workloads import random_inputs

from gpu_support import announce, assert_within_bound, scale_to_dev, to_dev, to_host

pytestmark = pytest.mark.gpu


def _device_operands(M, N, K, mode, seed):
    A, B = random_inputs(M, N, K, seed, "mx_block")
    qa, sa = Q.quantize(A, mode)
    qb, sb = Q.quantize(B, mode)
    dev = [to_dev(qa, 16), scale_to_dev(sa, mode), to_dev(qb, 16), scale_to_dev(sb, mode)]
    return (qa, sa, qb, sb), dev


def _run_noalloc(M, N, K, d, mode, out, C):
    qa, sa, qb, sb = d
    F.fp8gemm_run_noalloc(M, N, K, qa.data_ptr(), qa.stride(0), F.FORMATS["e4m3"], qb.data_ptr(),
                          qb.stride(0), F.FORMATS["e4m3"], F.SCALE_MODES[mode], sa.data_ptr(),
                          sb.data_ptr(), 0, F.ACTIVATIONS["none"], C.data_ptr(), C.stride(0),
                          F.OUT_DTYPES[out], torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("mode", ["tensor", "rowwise", "mx32"])
def test_noalloc_two_calls_match_run_ex(mode):
    for i, (M, N, K) in enumerate([(256, 640, 4096), (128, 4096, 4096), (64, 2048, 2048),
                                   (100, 512, 2048)]):
        assert F.fp8gemm_run_path(M, N, K, K, K, 0, 0, F.SCALE_MODES[mode], 0) == "splitk"
        assert 0 < F.fp8gemm_workspace_size(M, N, K, F.SCALE_MODES[mode]) <= \
            F.NOALLOC_SCRATCH_BYTES
        host, d = _device_operands(M, N, K, mode, seed=100 + i)
        announce("noalloc", mode, (M, N, K))
        expect = F.gemm(*d, mode, "bf16")                  # fp8gemm_run_ex, own workspace
        got = torch.empty((M, N), dtype=torch.bfloat16, device=expect.device)
        _run_noalloc(M, N, K, d, mode, "bf16", got)
        torch.cuda.synchronize()
        assert torch.equal(got, expect), f"{mode} {(M, N, K)}: differs from fp8gemm_run_ex"
        Cr, Ar = O.gemm_reference(*host, mode)
        assert_within_bound(to_host(got), Cr, Ar, "bf16", f"noalloc {mode} {(M, N, K)}")


def test_noalloc_unsplit_shape_and_oversized_split():
    M, N, K = 256, 512, 384                      # 128 x 128 tiles: no scratch used
    assert F.fp8gemm_workspace_size(M, N, K, 1) == 0
    host, d = _device_operands(M, N, K, "rowwise", seed=7)
    announce("noalloc unsplit", (M, N, K))
    got = torch.empty((M, N), dtype=torch.float16, device=d[0].device)
    _run_noalloc(M, N, K, d, "rowwise", "f16", got)
    torch.cuda.synchronize()
    assert torch.equal(got, F.gemm(*d, "rowwise", "f16"))
    Cr, Ar = O.gemm_reference(*host, "rowwise")
    assert_within_bound(to_host(got), Cr, Ar, "f16", "noalloc unsplit")
    # 504 split tiles x 2 slices of fp32 partials: more than the scratch holds
    M, N, K = 256, 8064, 4096
    assert F.fp8gemm_workspace_size(M, N, K, 0) > F.NOALLOC_SCRATCH_BYTES
    qa = torch.zeros((M, K), dtype=torch.uint8, device=got.device)
    qb = torch.zeros((N, K), dtype=torch.uint8, device=got.device)
    s = torch.ones(1, dtype=torch.float32, device=got.device)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=got.device)
    with pytest.raises(F.Fp8GemmError) as err:
        _run_noalloc(M, N, K, (qa, s, qb, s), "tensor", "bf16", C)
    assert err.value.status == 4                 # FP8GEMM_ERROR_WORKSPACE
    torch.cuda.synchronize()
