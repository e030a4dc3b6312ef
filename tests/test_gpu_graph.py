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


def test_grouped_graph_follows_device_offsets():
    """The grouped GEMM reads its expert offsets on the device, so one captured
    graph serves changing expert counts: after new offsets are copied into the
    same tensor, a replay gives the eager result for the new counts, bit for bit."""
    G, N, K, total = 8, 512, 512, 2048
    gen = torch.Generator(device=DEV).manual_seed(8)
    qa, sa = F.quantize(torch.randn(total, K, device=DEV, generator=gen), "rowwise")
    w = torch.randn(G * N, K, device=DEV, generator=gen) * 0.02
    qw, sw = F.quantize(w, "rowwise")
    qw, sw = qw.reshape(G, N, K), sw.reshape(G, N)
    sets = [np.array([256, 256, 256, 256, 256, 256, 256, 256]),
            np.array([1, 700, 0, 300, 47, 600, 250, 150]),
            np.array([2048, 0, 0, 0, 0, 0, 0, 0])]
    offs = [torch.from_numpy(np.concatenate([[0], np.cumsum(c)]).astype(np.int32)).to(DEV)
            for c in sets]
    announce("grouped graph", [c.tolist() for c in sets])
    eager = [F.grouped_gemm(qa, sa, o, qw, sw, "rowwise", "bf16") for o in offs]
    offsets = offs[0].clone()
    C = torch.empty((total, N), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        F.grouped_gemm(qa, sa, offsets, qw, sw, "rowwise", "bf16", out=C)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        F.grouped_gemm(qa, sa, offsets, qw, sw, "rowwise", "bf16", out=C)
    torch.cuda.synchronize()
    for r in (0, 1, 2, 1, 0):
        offsets.copy_(offs[r])
        C.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, eager[r]), f"counts {sets[r].tolist()}"
    del graph
