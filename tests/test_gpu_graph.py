"""The library's launches under HIP graph capture (torch's capture of the current stream, on which every entry
point launches): quantize, dequantize, the W4A16 decode and batched products, captured once and replayed three
times with eager work and synchronisations in between. Every replay must give the eager results bit for bit.
The library allocates nothing and clears nothing with memset, so its kernels are all the graph holds.
"""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import announce, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


@pytest.mark.parametrize("sym", [True, False])
def test_graph_replays_match_eager(gpu_lib, sym):
    announce("graph replays sym=%s" % sym)
    d = W.ffn7b(ms=(16,))
    wg, xg = to_gpu_bf16(d["w"]), to_gpu_bf16(d["x"])
    n, k = wg.shape
    g = 128
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty(n * k // g, dtype=torch.float32, device="cuda")
    zeros = None if sym else torch.empty(n * k // g, dtype=torch.uint8, device="cuda")
    deq = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
    y1 = torch.empty((1, n), dtype=torch.float32, device="cuda")
    y16 = torch.empty((16, n), dtype=torch.bfloat16, device="cuda")

    def step():
        gpu_lib.quantize(wg, 4, sym, gpu_lib.GROUP, g, out=(codes, scales, zeros))
        gpu_lib.dequantize(codes, scales, zeros, n, k, 4, sym, gpu_lib.GROUP, g, out=deq)
        gpu_lib.qlinear_w4a16(xg[:1], codes, scales, zeros, g, sym, out_dtype=torch.float32, out=y1)
        gpu_lib.qlinear_w4a16(xg[:16], codes, scales, zeros, g, sym, out=y16)

    outs = (codes, scales, deq, y1, y16) + (() if sym else (zeros,))
    step()
    torch.cuda.synchronize()
    eager = [_bits(t) for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    other = to_gpu_bf16(W.bf16_bits(np.random.default_rng(3).standard_normal((n, k)).astype(np.float32)))
    for rep in range(3):
        for t in outs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for a, t in zip(eager, outs):
            assert np.array_equal(a, _bits(t)), "replay %d differs from the eager run" % rep
        gpu_lib.quantize(other, 4, sym, gpu_lib.GROUP, g)  # eager work between the replays
        torch.cuda.synchronize()
    del graph
