"""The hot path captured in a HIP graph (torch.cuda.graph): quantise A, quantise
B and the GEMM, all launched on the capturing stream with every buffer and
workspace allocated beforehand.  Each replay, with eager work and
synchronisations of the program between replays, must give outputs bit-equal to
the eager run: the split-K arrival counters leave the workspace as they found it
and no memset node is recorded (the library clears memory with kernels)."""
import numpy as np
import pytest
import torch

import block_scaled_gemm_fp8gemm_amd as F

from gpu_support import DEV, announce

pytestmark = pytest.mark.gpu


def _scales_buf(mode, rows, K):
    if mode == "tensor":
        return torch.empty(1, dtype=torch.float32, device=DEV)
    if mode == "rowwise":
        return torch.empty(rows, dtype=torch.float32, device=DEV)
    return torch.empty((rows, K // 32), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("mode,shape", [("tensor", (128, 4096, 4096)),      # split-K
                                        ("rowwise", (1024, 1024, 512)),     # 128-row tiles
                                        ("mx32", (4096, 4096, 1024))])      # 256-row tiles
def test_hot_path_graph_replays(mode, shape):
    M, N, K = shape
    g = torch.Generator(device=DEV).manual_seed(M + N + K)
    a = torch.randn(M, K, device=DEV, generator=g)
    b = torch.randn(N, K, device=DEV, generator=g)
    announce("graph", mode, shape, F.fp8gemm_run_path(M, N, K, K, K, 0, 0, F.SCALE_MODES[mode], 0))
    qa = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    qb = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    sa, sb = _scales_buf(mode, M, K), _scales_buf(mode, N, K)
    qws = torch.zeros(F.fp8gemm_quantize_workspace_size(max(M, N), K, F.SCALE_MODES[mode]) + 16,
                      dtype=torch.uint8, device=DEV)
    gws = torch.zeros(F.fp8gemm_workspace_size(M, N, K, F.SCALE_MODES[mode]) + 16,
                      dtype=torch.uint8, device=DEV)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def step():
        F.quantize(a, mode, out=qa, scales=sa, workspace=qws)
        F.quantize(b, mode, out=qb, scales=sb, workspace=qws)
        F.gemm(qa, sa, qb, sb, mode, "bf16", out=C, workspace=gws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # eager run on the capturing stream
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = (qa.clone(), sa.clone(), qb.clone(), sb.clone(), C.clone())

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for t in (qa, qb, C):                      # the replay must write every output
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (qa, sa, qb, sb, C)
        for name, x, y in zip(("qa", "sa", "qb", "sb", "C"), got, ref):
            assert torch.equal(x, y), f"replay {r}: {name} differs from the eager run"
        with torch.cuda.stream(side):              # eager work between replays
            step()
        torch.cuda.synchronize()
        assert torch.equal(C, ref[4])
    del graph
