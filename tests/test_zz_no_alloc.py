"""The allocation-free W8A8 entry point (pqg_qlinear_w8a8_noalloc) against pqg_qlinear_w8a8, through the C ABI.

Both run the same kernels; the first keeps the activation codes and scales in the library's own device array,
the second in caller buffers. Two calls in a row -- the full 2048 x 11008 x 4096 layer, then a smaller ragged
one -- must each give the other entry point's output bit for bit, so nothing left in the array by a call
leaks into the next.
"""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import announce, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_w8a8_on_two_calls(gpu_lib, out_dtype):
    for m, n, k in [(2048, 11008, 4096), (300, 264, 1024)]:
        announce("w8a8 noalloc %dx%dx%d %s" % (m, n, k, out_dtype))
        d = W.w8a8(m=m, n=n, k=k)
        xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
        sm = gpu_lib.smooth(xg, wg, 0.5)
        w_q, s_w, _ = gpu_lib.quantize(wg, 8, True, gpu_lib.ROW, 0, sm, gpu_lib.SMOOTH_MUL)
        y_ref, _, _ = gpu_lib.qlinear_w8a8(xg, sm, w_q, s_w, out_dtype=out_dtype)
        y = gpu_lib.qlinear_w8a8_noalloc(xg, sm, w_q, s_w, out_dtype=out_dtype)
        torch.cuda.synchronize()
        a, b = _bits(y), _bits(y_ref)
        bad = np.flatnonzero(a.ravel() != b.ravel())
        assert bad.size == 0, "%d outputs differ, first at %s" % (bad.size, bad[:8])
        assert np.any(a != 0)


def test_noalloc_without_smoothing_and_limits(gpu_lib):
    """No smoothing vector; then a shape beyond the array is refused before anything is enqueued."""
    d = W.w8a8(m=64, n=96, k=512)
    xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
    w_q, s_w, _ = gpu_lib.quantize(wg, 8, True, gpu_lib.ROW, 0)
    y_ref, _, _ = gpu_lib.qlinear_w8a8(xg, None, w_q, s_w, out_dtype=torch.float32)
    y = gpu_lib.qlinear_w8a8_noalloc(xg, None, w_q, s_w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(y_ref))
    big = torch.zeros((4097, 4096), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((64, 4096), dtype=torch.int8, device="cuda")
    sw = torch.ones(64, dtype=torch.float32, device="cuda")
    with pytest.raises(gpu_lib.PqgError, match="activation codes"):
        gpu_lib.qlinear_w8a8_noalloc(big, None, wq, sw)
