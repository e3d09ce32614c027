"""Grouped products (pqg_qlinear_w4a16_grouped) through the C ABI against the oracle within the float tolerances
("第11章 模型量化与压缩" §11.10.1, §11.1.6, §11.3.7), and against pqg_qlinear_w4a16 on each problem alone: equal up
to the order of the fp32 partial sums (a single small launch may split K over more waves than the grouped grid),
i.e. within 1e-6 normwise for fp32 outputs and at most one bf16 ulp apart element by element for bf16 outputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (BOUND_BF16, BOUND_W4A16_F32, abs_terms_w4, announce, assert_per_element, normwise, to_f64, to_gpu,
                     to_gpu_bf16)

pytestmark = pytest.mark.gpu

TOL_BF16 = 5e-3
TOL_F32 = 1e-5


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _close_to_single(y, y1):
    """fp32: 1e-6 normwise; bf16: every element within one ulp (adjacent bit patterns of the same sign)."""
    if y.dtype == torch.float32:
        assert normwise(to_f64(y), to_f64(y1)) <= 1e-6
    else:
        a = _bits(y).astype(np.int32)
        b = _bits(y1).astype(np.int32)
        assert np.all(np.abs(a - b) <= 1), int(np.abs(a - b).max())


# up to 4 tokens the decode kernel, 5-32 the staged matrix-core kernel in one launch, 33 and more one launch per
# problem
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 13, 16, 17, 32, 40])
@pytest.mark.parametrize("gs,sym", [(128, True), (32, False), (64, True)])
def test_grouped_small_ragged(gpu_lib, m, gs, sym):
    """Five problems of different shapes (ragged row blocks, several K, one empty) against the oracle and
    against one launch per problem."""
    shapes = [(257, 2048), (33, 4096), (0, 1024), (1000, 1024), (6, 8192)]
    announce("grouped small m=%d g=%d sym=%s" % (m, gs, sym))
    rng = np.random.default_rng(1000 * m + gs + int(sym))
    xs, cs, ss, zs, refs = [], [], [], [], []
    for n, k in shapes:
        w = W.bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
        x = W.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        q, so, zo = oracle.quantize(w, 4, sym, oracle.GROUP, gs)
        xs.append(to_gpu_bf16(x))
        cs.append(to_gpu(oracle.pack_int4(q)))
        ss.append(to_gpu(so))
        zs.append(None if sym else to_gpu(zo))
        refs.append((oracle.w4a16(x, q, so, zo, gs), abs_terms_w4(x, q, so, zo, gs)) if n else None)
    ys = gpu_lib.qlinear_w4a16_grouped(xs, cs, ss, None if sym else zs, gs, sym, out_dtype=torch.float32)
    singles = [gpu_lib.qlinear_w4a16(xs[i], cs[i], ss[i], zs[i], gs, sym, out_dtype=torch.float32)
               for i in range(len(shapes))]
    torch.cuda.synchronize()
    for i, (n, k) in enumerate(shapes):
        assert ys[i].shape == (m, n)
        if n == 0:
            continue
        _close_to_single(ys[i], singles[i])
        assert normwise(to_f64(ys[i]), refs[i][0]) <= TOL_F32, i
        assert_per_element(to_f64(ys[i]), refs[i][0], refs[i][1], BOUND_W4A16_F32, "problem %d" % i)


def test_grouped_staged_falls_back_per_problem(gpu_lib):
    """8 tokens with one problem whose K is not a multiple of 128: every problem runs as its own product."""
    shapes = [(100, 1056), (40, 2048)]
    announce("grouped fallback")
    rng = np.random.default_rng(77)
    xs, cs, ss, zs, refs = [], [], [], [], []
    for n, k in shapes:
        w = W.bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
        x = W.bf16_bits(rng.standard_normal((8, k)).astype(np.float32))
        q, so, zo = oracle.quantize(w, 4, False, oracle.GROUP, 32)
        xs.append(to_gpu_bf16(x))
        cs.append(to_gpu(oracle.pack_int4(q)))
        ss.append(to_gpu(so))
        zs.append(to_gpu(zo))
        refs.append((oracle.w4a16(x, q, so, zo, 32), abs_terms_w4(x, q, so, zo, 32)))
    ys = gpu_lib.qlinear_w4a16_grouped(xs, cs, ss, zs, 32, False, out_dtype=torch.float32)
    singles = [gpu_lib.qlinear_w4a16(xs[i], cs[i], ss[i], zs[i], 32, False, out_dtype=torch.float32)
               for i in range(len(shapes))]
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert np.array_equal(_bits(ys[i]), _bits(singles[i])), i  # the same launches
        assert normwise(to_f64(ys[i]), refs[i][0]) <= TOL_F32, i
        assert_per_element(to_f64(ys[i]), refs[i][0], refs[i][1], BOUND_W4A16_F32, "problem %d" % i)


def test_grouped_eight_problems_bf16(gpu_lib):
    """The largest table (8 problems) with bf16 outputs."""
    announce("grouped eight problems")
    rng = np.random.default_rng(8)
    xs, cs, ss, refs = [], [], [], []
    for i in range(8):
        n, k = 64 * (i + 1) + i, 1024 * (1 + i % 3)
        w = W.bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
        x = W.bf16_bits(rng.standard_normal((1, k)).astype(np.float32))
        q, so, _ = oracle.quantize(w, 4, True, oracle.GROUP, 128)
        xs.append(to_gpu_bf16(x))
        cs.append(to_gpu(oracle.pack_int4(q)))
        ss.append(to_gpu(so))
        refs.append((oracle.w4a16(x, q, so, None, 128), abs_terms_w4(x, q, so, None, 128)))
    ys = gpu_lib.qlinear_w4a16_grouped(xs, cs, ss, None, 128, True)
    torch.cuda.synchronize()
    for i in range(8):
        assert normwise(to_f64(ys[i]), refs[i][0]) <= TOL_BF16, i
        assert_per_element(to_f64(ys[i]), refs[i][0], refs[i][1], BOUND_BF16, "problem %d" % i)


def test_grouped_l70b_layer_m1(gpu_lib):
    """The seven Llama-70B projections (INT4 g = 128, quantized on the GPU) at M = 1 in one launch: 24 sampled rows
    per projection against the oracle, every output within one bf16 ulp of the seven single launches."""
    announce("grouped l70b layer m=1")
    xs, cs, ss, samples = [], [], [], []
    for p, (name, n, k) in enumerate(W.L70B_PROJ):
        w = W.l70b_weight(p)
        codes, s, _ = gpu_lib.quantize(to_gpu_bf16(w), 4, True, 2, 128)
        x = W.l70b_x(p, 1)
        rows = np.unique(np.concatenate([np.random.default_rng(50 + p).choice(n, 22, replace=False), [0, n - 1]]))
        q, so, _ = oracle.quantize(w[rows], 4, True, 2, 128)
        samples.append((rows, oracle.w4a16(x, q, so, None, 128), abs_terms_w4(x, q, so, None, 128)))
        xs.append(to_gpu_bf16(x))
        cs.append(codes)
        ss.append(s)
        del w
    ys = gpu_lib.qlinear_w4a16_grouped(xs, cs, ss, None, 128, True)
    singles = [gpu_lib.qlinear_w4a16(xs[i], cs[i], ss[i], None, 128, True) for i in range(7)]
    torch.cuda.synchronize()
    for i in range(7):
        _close_to_single(ys[i], singles[i])
        rows, ref, terms = samples[i]
        assert normwise(to_f64(ys[i])[:, rows], ref) <= TOL_BF16, W.L70B_PROJ[i][0]
        assert_per_element(to_f64(ys[i])[:, rows], ref, terms, BOUND_BF16, W.L70B_PROJ[i][0])
