"""Determinism: every kernel that shares LDS between waves, or splits a product over waves, run again on the same
inputs -- with other kernels launched in between, so that the order and the cache state differ -- gives the same
bits. A race between waves (a barrier missing from a ring stage, a reduction read before it is complete) shows up
here as outputs that change from run to run.
"""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import announce, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


def _same(runs):
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert np.array_equal(a, b), "outputs differ between runs"


def test_w8a8_layer_reruns(gpu_lib):
    """2048 x 11008 x 4096 (the wide, ping-pong kernel): int32 accumulators and the bf16 and fp32 epilogues."""
    announce("determinism w8a8 layer")
    d = W.w8a8()
    xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
    s = gpu_lib.smooth(xg, wg, 0.5)
    w_q, s_w, _ = gpu_lib.quantize(wg, 8, True, 1, 0, s, 2)
    _, x_q, s_x = gpu_lib.qlinear_w8a8(xg, s, w_q, s_w, out_dtype=torch.bfloat16)
    runs = []
    for i in range(3):
        acc = gpu_lib.gemm_s8s8s32(x_q, w_q)
        if i == 1:
            gpu_lib.quantize(wg, 4, True, 2, 128)  # other work between the runs
        y16, _, _ = gpu_lib.qlinear_w8a8(None, None, w_q, s_w, out_dtype=torch.bfloat16, x_q=x_q, x_scales=s_x)
        y32, _, _ = gpu_lib.qlinear_w8a8(None, None, w_q, s_w, out_dtype=torch.float32, x_q=x_q, x_scales=s_x)
        torch.cuda.synchronize()
        runs.append((_bits(acc), _bits(y16), _bits(y32)))
    _same(runs)


def test_smooth_and_row_quantize_reruns(gpu_lib):
    """The smoothing factor (column maxima over many blocks) and the per-row quantize with the division."""
    announce("determinism smooth")
    d = W.w8a8()
    xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
    runs = []
    for _ in range(3):
        s = gpu_lib.smooth(xg, wg, 0.5)
        q, sc, _ = gpu_lib.quantize(xg, 8, True, 1, 0, s, 1)
        torch.cuda.synchronize()
        runs.append((_bits(s), _bits(q), _bits(sc)))
    _same(runs)


def test_w4a8_layer_reruns(gpu_lib):
    """W4A8 at 2048 x 11008 x 4096, g = 128 (four waves of a block share each LDS stage)."""
    announce("determinism w4a8")
    d = W.w8a8()
    xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
    s = gpu_lib.smooth(xg, wg, 0.5)
    _, x_q, s_x = gpu_lib.qlinear_w8a8(xg, s, *gpu_lib.quantize(wg, 8, True, 1, 0, s, 2)[:2],
                                       out_dtype=torch.bfloat16)
    c4, s4, _ = gpu_lib.quantize(wg, 4, True, 2, 128, s, 2)
    runs = []
    for _ in range(3):
        y = gpu_lib.qlinear_w4a8(x_q, s_x, c4, s4, None, 128, True, out_dtype=torch.float32)
        torch.cuda.synchronize()
        runs.append((_bits(y),))
    _same(runs)


@pytest.mark.parametrize("m", [1, 8, 32])
def test_w4a16_grouped_reruns(gpu_lib, m):
    """The grouped products of the 7B FFN shapes (K split over waves and combined in a fixed order)."""
    announce("determinism w4a16 grouped M=%d" % m)
    d = W.ffn7b(ms=(32,))
    wg = to_gpu_bf16(d["w"])
    xg = to_gpu_bf16(d["x"])
    c1, s1, _ = gpu_lib.quantize(wg, 4, True, 2, 128)
    c2, s2, _ = gpu_lib.quantize(wg[:4096].contiguous(), 4, True, 2, 128)
    runs = []
    for i in range(3):
        ys = gpu_lib.qlinear_w4a16_grouped([xg[:m], xg[:m]], [c1, c2], [s1, s2], None, 128, True)
        if i == 1:
            gpu_lib.qlinear_w4a16(xg[:m], c1, s1, None, 128, True)  # other work between the runs
        torch.cuda.synchronize()
        runs.append(tuple(_bits(y) for y in ys))
    _same(runs)


def test_kv_keys_reruns(gpu_lib):
    """Keys per channel over groups of 128 tokens (the channel ranges combined across four waves)."""
    announce("determinism kv keys")
    kv = W.kv_cache(8 * 1024, W.KV_CHANNELS)
    kg = to_gpu_bf16(kv["k"])
    runs = []
    for _ in range(3):
        q, s, z = gpu_lib.kv_quantize_keys(kg, 128, False)
        torch.cuda.synchronize()
        runs.append((_bits(q), _bits(s), _bits(z)))
    _same(runs)
