"""The library's calls inside a captured HIP graph: every call launches kernels
only (no allocation, no memset), so it can be captured.  The graph is replayed
several times with eager work and synchronisations in between, and every
replay is checked against the eager result."""
import numpy as np
import pytest
import torch

import microscaling_fp4_quantization_amd as fq

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_graph_replays_match_eager():
    rng = np.random.default_rng(97)
    xs = [torch.from_numpy((rng.standard_t(4, (64, 5120)) * 0.3).astype(np.float32))
          .to(torch.bfloat16).to(DEV) for _ in range(2)]
    x = xs[0].clone()
    ws = torch.zeros(fq.workspace_bytes(), dtype=torch.uint8, device=DEV)
    outs = dict(codes=torch.empty((64, 2560), dtype=torch.uint8, device=DEV),
                scales=torch.empty((64, 320), dtype=torch.uint8, device=DEV),
                block_mse=torch.empty((64, 320), dtype=torch.float32, device=DEV),
                stats=fq.new_stats(DEV))
    g_row = torch.empty(64, dtype=torch.float32, device=DEV)
    g_t = torch.empty(1, dtype=torch.float32, device=DEV)
    mx = dict(codes=torch.empty((64, 2560), dtype=torch.uint8, device=DEV),
              scales=torch.empty((64, 160), dtype=torch.uint8, device=DEV))

    def calls():
        fq.nvfp4_quantize(x, 16, fq.FMT_UE4M3, fq.G_ROW, g_row, 16, ws=ws, **outs)
        fq.nvfp4_quantize(x, 16, fq.FMT_UE4M3, fq.G_DYNAMIC, g_t, 0, codes=mx["codes"],
                          scales=outs["scales"], block_mse=False, stats=False, ws=ws)
        fq.mxfp4_quantize(x, 32, block_mse=False, stats=False, **mx)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (outs["codes"], outs["scales"], outs["block_mse"], outs["stats"],
                                    g_row, g_t, mx["codes"], mx["scales"])]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(4):
        src = xs[rep % 2]
        x.copy_(src)
        calls()  # eager
        want = snapshot()
        for t in outs.values():
            t.zero_()
        g_row.zero_()
        mx["codes"].zero_()
        graph.replay()
        got = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep}"
        x.mul_(0.5)  # eager work between replays
        torch.cuda.synchronize()


def test_batched_mx_nv_in_a_graph():
    """fp4_quantize_mx_nv_batch (four launches, the per-tensor scales passed
    from the MXFP4 reduction to the NVFP4 pass through device memory) captured
    once and replayed on changing inputs: every replay equals the eager call."""
    rng = np.random.default_rng(98)
    shapes = [(64, 1024), (8, 512), (200, 2048)]
    srcs = [[torch.from_numpy((rng.standard_normal(s) * (0.01 + 0.02 * k)).astype(np.float32))
             .to(torch.bfloat16).to(DEV) for s in shapes] for k in range(2)]
    xs = [t.clone() for t in srcs[0]]
    ws = torch.zeros(fq.workspace_bytes(), dtype=torch.uint8, device=DEV)
    outs = []
    for (r, c) in shapes:
        mx = dict(codes=torch.empty((r, c // 2), dtype=torch.uint8, device=DEV),
                  scales=torch.empty((r, c // 32), dtype=torch.uint8, device=DEV),
                  block_mse=torch.empty((r, c // 32), dtype=torch.float32, device=DEV),
                  stats=fq.new_stats(DEV))
        nv = dict(codes=torch.empty((r, c // 2), dtype=torch.uint8, device=DEV),
                  scales=torch.empty((r, c // 16), dtype=torch.uint8, device=DEV),
                  block_mse=torch.empty((r, c // 16), dtype=torch.float32, device=DEV),
                  stats=fq.new_stats(DEV))
        outs.append((mx, nv, torch.empty(1, dtype=torch.float32, device=DEV)))

    def call():
        fq.fp4_quantize_mx_nv_batch(xs, 16, mse_kind=fq.MSE_REL, outs=outs, ws=ws)

    def flat():
        return [t for mx, nv, g in outs for t in list(mx.values()) + list(nv.values()) + [g]]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(4):
        for x, s in zip(xs, srcs[rep % 2]):
            x.copy_(s)
        call()  # eager
        torch.cuda.synchronize()
        want = [t.clone() for t in flat()]
        for t in flat():
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(flat(), want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
