"""GPU parity: the HIP library (through its C ABI) against the CPU oracle, on the same seeded inputs.

Bar: integer codes, packed bytes, fp32 scales, zero points, smoothing factors (alpha in {0, 0.5, 1}) and
INT32 accumulators bit-exact; float outputs within a normwise relative error of 5e-3 (bf16 outputs) or
1e-5 (fp32 outputs). Full-size workloads are checked on sampled rows the oracle computes one by one.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (BOUND_BF16, BOUND_W4A8_F32, BOUND_W4A16_F32, BOUND_W8A8_BF16, BOUND_W8A8_F32, abs_terms_i8, abs_terms_w4, abs_terms_w4a8,
                     announce, assert_per_element, bf16_tensor_bits, normwise, to_f64, to_gpu, to_gpu_bf16)

pytestmark = pytest.mark.gpu

TOL_BF16 = 5e-3
TOL_F32 = 1e-5


def gpu_quant(pqg, x_gpu, bits, sym, gran, gs=0, smooth=None, mode=0):
    codes, s, z = pqg.quantize(x_gpu, bits, sym, gran, gs, smooth, mode)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), s.cpu().numpy(), None if z is None else z.cpu().numpy()


def oracle_codes_bytes(q, bits, sym):
    """The oracle's codes in the library's storage format (packed nibbles or plain bytes)."""
    if bits == 4:
        return oracle.pack_int4(q)
    return q.astype(np.int8) if sym else q.astype(np.uint8)


def assert_quant_equal(gpu, ora, bits, sym):
    codes, s, z = gpu
    q, so, zo = ora
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), "scales differ"
    if not sym:
        assert np.array_equal(z, zo), "zero points differ"
    want = oracle_codes_bytes(q, bits, sym)
    assert codes.shape == want.shape
    bad = np.nonzero(codes.view(np.uint8) != want.view(np.uint8))
    assert bad[0].size == 0, "codes differ at %s" % (list(zip(*[b[:5] for b in bad])),)


# --------------------------------------------------------------------------- quantize / dequantize

QUANT_CASES = [
    # bits, sym, gran, gs, smooth_mode
    (4, True, 2, 128, 0), (4, True, 2, 64, 0), (4, True, 2, 32, 0),
    (4, False, 2, 128, 0), (4, False, 2, 64, 0), (4, False, 2, 32, 0),
    (8, True, 2, 128, 0), (8, False, 2, 32, 0),
    (8, True, 1, 0, 0), (8, False, 1, 0, 0), (4, True, 1, 0, 0), (4, False, 1, 0, 0),
    (8, True, 0, 0, 0), (8, False, 0, 0, 0), (4, True, 0, 0, 0), (4, False, 0, 0, 0),
    (8, True, 1, 0, 1), (8, True, 1, 0, 2), (4, True, 2, 128, 1), (8, False, 0, 0, 2),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", QUANT_CASES)
@pytest.mark.parametrize("shape", [(37, 256), (3, 2112), (1, 32)])
def test_quantize_bitexact_small(gpu_lib, case, dtype, shape):
    bits, sym, gran, gs, mode = case
    rows, cols = shape
    if gran == 2 and cols % gs:
        pytest.skip("cols not a multiple of g")
    announce("quantize %s %s %s" % (case, dtype, shape))
    rng = np.random.default_rng(zlib.crc32(repr((case, dtype, shape)).encode()))  # stable across processes
    x32 = (rng.standard_normal(shape) * rng.uniform(0.01, 2.0, size=(rows, 1))).astype(np.float32)
    x32[0, : min(cols, 64)] += 1.5  # a shifted block: one-signed groups for the asymmetric path
    if rows > 2:
        x32[2, :] = 0.0  # an all-zero row / groups
    if dtype == "bf16":
        xh = W.bf16_bits(x32)
        xg = to_gpu_bf16(xh)
    else:
        xh = x32
        xg = to_gpu(x32)
    sm = None
    if mode:
        sm = rng.uniform(0.25, 4.0, size=cols).astype(np.float32)
    gpu = gpu_quant(gpu_lib, xg, bits, sym, gran, gs, None if sm is None else to_gpu(sm), mode)
    ora = oracle.quantize(xh, bits, sym, gran, gs, sm, mode)
    assert_quant_equal(gpu, ora, bits, sym)


# Per-row quantize at each edge of its launch shapes: 64 threads with two or eight chunks of 8 columns each
# (up to 1024 / 4096 columns), 256 threads (up to 16384), 1024 threads beyond.
@pytest.mark.parametrize("cols", [1024, 1056, 4096, 4128, 16384, 16416])
@pytest.mark.parametrize("case", [(8, True, 0), (8, False, 1), (4, True, 2), (4, False, 0)])
def test_quantize_row_launch_edges(gpu_lib, cols, case):
    bits, sym, mode = case
    announce("row quantize edges %s %s" % (cols, case))
    rng = np.random.default_rng(zlib.crc32(repr(("row edges", cols, case)).encode()))
    x32 = (rng.standard_normal((3, cols)) * np.array([[0.05], [1.0], [3.0]])).astype(np.float32)
    x32[1, -1] = 40.0  # the row maximum in the row's last chunk
    x32[2, 0] = -50.0  # and in its first
    xh = W.bf16_bits(x32)
    sm = rng.uniform(0.25, 4.0, size=cols).astype(np.float32) if mode else None
    gpu = gpu_quant(gpu_lib, to_gpu_bf16(xh), bits, sym, 1, 0, None if sm is None else to_gpu(sm), mode)
    ora = oracle.quantize(xh, bits, sym, 1, 0, sm, mode)
    assert_quant_equal(gpu, ora, bits, sym)


def test_quantize_tiny_config(gpu_lib):
    """256x512 fp32 with 0.5 % x20 outliers, symmetric INT4 g=128: codes, packed bytes and scales exact."""
    announce("tiny quantize")
    d = W.tiny()
    gpu = gpu_quant(gpu_lib, to_gpu(d["w"]), 4, True, 2, 128)
    ora = oracle.quantize(d["w"], 4, True, 2, 128)
    assert_quant_equal(gpu, ora, 4, True)
    assert gpu[1].size == 256 * 512 // 128


def test_quantize_attn7b_full(gpu_lib):
    """4096x4096 bf16, symmetric INT4 g=128: all 131,072 groups bit-exact."""
    announce("attn7b quantize")
    d = W.attn7b(ms=(1,))
    gpu = gpu_quant(gpu_lib, to_gpu_bf16(d["w"]), 4, True, 2, 128)
    ora = oracle.quantize(d["w"], 4, True, 2, 128)
    assert_quant_equal(gpu, ora, 4, True)


@pytest.mark.parametrize("gs", [32, 128])
def test_quantize_ffn7b_asym_full(gpu_lib, gs):
    """11008x4096 bf16 with 41 columns x10, asymmetric UINT4: codes, zeros and scales bit-exact."""
    announce("ffn7b quantize g=%d" % gs)
    d = W.ffn7b(ms=(1,))
    gpu = gpu_quant(gpu_lib, to_gpu_bf16(d["w"]), 4, False, 2, gs)
    ora = oracle.quantize(d["w"], 4, False, 2, gs)
    assert_quant_equal(gpu, ora, 4, False)


@pytest.mark.parametrize("case", [(4, True, 2, 128), (4, False, 2, 32), (8, True, 1, 0), (8, False, 0, 0),
                                  (4, False, 1, 0), (8, True, 2, 64)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_bitexact(gpu_lib, case, out):
    bits, sym, gran, gs = case
    announce("dequantize %s %s" % (case, out))
    rng = np.random.default_rng(17)
    rows, cols = 19, 384
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    q, s, z = oracle.quantize(x, bits, sym, gran, gs)
    codes = oracle_codes_bytes(q, bits, sym)
    ref32, ref16 = oracle.dequantize(q, s, z, gran, gs)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    y = gpu_lib.dequantize(to_gpu(codes), to_gpu(s), None if z is None else to_gpu(z), rows, cols, bits, sym, gran,
                           gs, out_dtype=odt)
    torch.cuda.synchronize()
    if out == "f32":
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref32.view(np.uint32))
    else:
        assert np.array_equal(bf16_tensor_bits(y), ref16)


def test_empty_tensors_are_noops(gpu_lib):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    codes, s, z = gpu_lib.quantize(x, 4, True, 2, 128)
    assert codes.shape == (0, 128) and s.numel() == 0
    y = gpu_lib.qlinear_w4a16(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"),
                              torch.zeros((8, 128), dtype=torch.uint8, device="cuda"),
                              torch.ones(16, dtype=torch.float32, device="cuda"), None, 128, True)
    assert y.shape == (0, 8)


# --------------------------------------------------------------------------- W4A16

def w4a16_case(pqg, w_host, w_is_bf16, x_u16, sym, gs, out_dtype):
    """GPU: quantize + pack + W4A16; oracle: quantize + binary64 product. Returns (y_gpu, y_ref, gpu quant, ora quant)."""
    wg = to_gpu_bf16(w_host) if w_is_bf16 else to_gpu(w_host)
    codes, s, z = pqg.quantize(wg, 4, sym, 2, gs)
    y = pqg.qlinear_w4a16(to_gpu_bf16(x_u16), codes, s, z, gs, sym, out_dtype=out_dtype)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize(w_host, 4, sym, 2, gs)
    y_ref = oracle.w4a16(x_u16, q, so, zo, gs)
    gq = (codes.cpu().numpy(), s.cpu().numpy(), None if z is None else z.cpu().numpy())
    rel = BOUND_BF16 if out_dtype == torch.bfloat16 else BOUND_W4A16_F32
    assert_per_element(to_f64(y), y_ref, abs_terms_w4(x_u16, q, so, zo, gs), rel, "W4A16")
    return to_f64(y), y_ref, gq, (q, so, zo)


def test_w4a16_tiny_fp32_out(gpu_lib):
    announce("w4a16 tiny")
    d = W.tiny()
    y, y_ref, gq, oq = w4a16_case(gpu_lib, d["w"], False, d["x"], True, 128, torch.float32)
    assert_quant_equal(gq, oq, 4, True)
    err = normwise(y, y_ref)
    assert err <= TOL_F32, err


@pytest.mark.parametrize("m", [1, 16])
def test_w4a16_attn7b(gpu_lib, m):
    announce("w4a16 attn7b M=%d" % m)
    d = W.attn7b(ms=(1, 16))
    y, y_ref, _, _ = w4a16_case(gpu_lib, d["w"], True, d["x"][:m], True, 128, torch.bfloat16)
    err = normwise(y, y_ref)
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("gs", [32, 128])
@pytest.mark.parametrize("m", [1, 8, 64])
def test_w4a16_ffn7b_asym(gpu_lib, gs, m):
    announce("w4a16 ffn7b asym g=%d M=%d" % (gs, m))
    d = W.ffn7b(ms=(1, 8, 64))
    y, y_ref, _, _ = w4a16_case(gpu_lib, d["w"], True, d["x"][:m], False, gs, torch.bfloat16)
    err = normwise(y, y_ref)
    assert err <= TOL_BF16, err


# (1, 64, 6144, 128) and (3, 33, 10240, 32) give the vector kernel an odd chunk-iteration count per wave
# (the second with a partly filled last iteration). (1, 2053, 16384, 64), (1, 4099, 16512, 128) and
# (1, 2051, 2080, 32) have a partial last row block at M = 1 with 8, 4 and 1 waves per row (the second also
# a partial last iteration).
@pytest.mark.parametrize("shape", [(1, 257, 96, 32), (3, 7, 4096, 64), (5, 130, 2080, 32), (2, 1, 32, 32),
                                   (4, 513, 640, 128), (1, 64, 6144, 128), (3, 33, 10240, 32),
                                   (1, 2053, 16384, 64), (1, 4099, 16512, 128), (1, 2051, 2080, 32)])
@pytest.mark.parametrize("sym", [True, False])
def test_w4a16_ragged_fp32(gpu_lib, shape, sym):
    """Ragged N (not a multiple of the row block), K with a partial last iteration, all M in 1..5."""
    m, n, k, gs = shape
    if k % gs:
        pytest.skip()
    announce("w4a16 ragged %s sym=%s" % (shape, sym))
    rng = np.random.default_rng(n * 7 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = W.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    y, y_ref, gq, oq = w4a16_case(gpu_lib, w, False, x, sym, gs, torch.float32)
    assert_quant_equal(gq, oq, 4, sym)
    err = normwise(y, y_ref)
    assert err <= TOL_F32, err


# 5 <= M <= 64 with K % 128 == 0 takes the LDS-staged matrix-core kernel (32 tokens per launch): ragged N
# (partial 32-row tile), group counts that are not a multiple of the four-group metadata load nor of the K
# split, one 128-code step, M = 33 and 64 (two launches); K % 128 != 0 and M > 64 take the general one.
# More than 256 row blocks of 32 take 4 waves per block (2 at up to 8 tokens from 768 blocks on), fewer when K
# is short: (8, 8224, 256) 257 blocks and 2 steps (one wave), (8, 24608, 512) 769 blocks at 2 waves,
# (16, 24608, 384) 769 blocks and 3 steps (one wave)
@pytest.mark.parametrize("shape", [(5, 130, 640), (13, 33, 1152), (20, 1, 384), (32, 257, 2688), (9, 64, 128),
                                   (32, 96, 8192), (33, 70, 512), (64, 130, 1024), (8, 40, 160), (70, 65, 256),
                                   (8, 8224, 256), (8, 24608, 512), (16, 24608, 384)])
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("sym", [True, False])
def test_w4a16_staged_ragged_fp32(gpu_lib, shape, gs, sym):
    m, n, k = shape
    if k % gs:
        pytest.skip("K not a multiple of g")
    announce("w4a16 staged %s g=%d sym=%s" % (shape, gs, sym))
    rng = np.random.default_rng(n * 11 + k + m + gs)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = W.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    y, y_ref, gq, oq = w4a16_case(gpu_lib, w, False, x, sym, gs, torch.float32)
    assert_quant_equal(gq, oq, 4, sym)
    err = normwise(y, y_ref)
    assert err <= TOL_F32, err


# 17-32 tokens on layers of more than 8192 rows (symmetric, g = 128) take the shared-activation kernel: 2, 4 or
# 8 row waves per block (N up to 16384, 32768, beyond), ragged last blocks (and N not a multiple of 32), K-step
# counts that split unevenly over the K groups (9 and 10 steps over 2 and 4 groups), M = 17, 24, 31, 32
@pytest.mark.parametrize("shape", [(17, 8224, 1024, "f32"), (32, 9000, 1280, "f32"), (31, 16448, 1152, "f32"),
                                   (24, 32800, 1024, "f32"), (32, 12000, 2048, "bf16")])
def test_w4a16_shared_activation(gpu_lib, shape):
    m, n, k, out = shape
    announce("w4a16 shared-activation %s" % (shape,))
    rng = np.random.default_rng(zlib.crc32(repr(("shared", shape)).encode()))
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = W.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    odt = torch.float32 if out == "f32" else torch.bfloat16
    y, y_ref, gq, oq = w4a16_case(gpu_lib, w, False, x, True, 128, odt)
    assert_quant_equal(gq, oq, 4, True)
    err = normwise(y, y_ref)
    assert err <= (TOL_F32 if out == "f32" else TOL_BF16), err


@pytest.mark.parametrize("proj", range(len(W.L70B_PROJ)))
def test_w4a16_l70b_sampled(gpu_lib, proj):
    """Full-size 70B projection: GPU quantizes all of it and runs the GEMV at M=1, 8, 32; the oracle checks
    64 sampled rows (codes and scales bit-exact, outputs within the bf16 tolerance on those rows)."""
    name, n, k = W.L70B_PROJ[proj]
    announce("w4a16 l70b %s" % name)
    w = W.l70b_weight(proj)
    wg = to_gpu_bf16(w)
    codes, s, _ = gpu_lib.quantize(wg, 4, True, 2, 128)
    del wg
    rng = np.random.default_rng(proj)
    rows = np.unique(np.concatenate([rng.choice(n, size=62, replace=False), [0, n - 1]]))
    wrows = w[rows]
    q, so, _ = oracle.quantize(wrows, 4, True, 2, 128)
    cg = codes.cpu().numpy()[rows]
    sg = s.cpu().numpy().reshape(n, -1)[rows].reshape(-1)
    assert np.array_equal(cg, oracle.pack_int4(q))
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    x = W.l70b_x(proj, 32)
    for m in (1, 8, 32):
        y = gpu_lib.qlinear_w4a16(to_gpu_bf16(x[:m]), codes, s, None, 128, True, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        ys = to_f64(y)[:, rows]
        y_ref = oracle.w4a16(x[:m], q, so, None, 128)
        err = normwise(ys, y_ref)
        assert err <= TOL_BF16, (m, err)
        assert_per_element(ys, y_ref, abs_terms_w4(x[:m], q, so, None, 128), BOUND_BF16, "70B %s M=%d" % (name, m))


# --------------------------------------------------------------------------- smoothing and W8A8

@pytest.mark.parametrize("alpha", [0.5, 1.0, 0.0])
def test_smooth_bitexact(gpu_lib, alpha):
    announce("smooth alpha=%s" % alpha)
    d = W.w8a8()
    s = gpu_lib.smooth(to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"]), alpha)
    torch.cuda.synchronize()
    so = oracle.smooth(d["x"], d["w"], alpha)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


def test_smooth_generic_alpha_within_ulp(gpu_lib):
    announce("smooth alpha=0.3")
    d = W.w8a8(m=256, n=512, k=1024)
    s = gpu_lib.smooth(to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"]), 0.3).cpu().numpy()
    so = oracle.smooth(d["x"], d["w"], 0.3)
    ulps = np.abs(s.view(np.int32).astype(np.int64) - so.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1


# Column maxima in row slices: row counts below, at and across one wave's 16 rows and one block's 64, column
# counts of one chunk, one 512-column block and a partial second block, every input dtype pair. The largest
# magnitudes of some columns sit in the first and the last row.
@pytest.mark.parametrize("tnk", [(1, 3, 8), (17, 130, 520), (64, 65, 512), (200, 1000, 1032)])
@pytest.mark.parametrize("dts", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")])
def test_smooth_ragged_dtypes_bitexact(gpu_lib, tnk, dts):
    t, n, k = tnk
    announce("smooth ragged %s %s" % (tnk, dts))
    g = np.random.default_rng(zlib.crc32(repr(("smooth", tnk, dts)).encode()))
    x = g.standard_normal((t, k)).astype(np.float32)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    x[-1, ::7] = -60.0
    x[0, 3::11] = 55.0
    w[-1, 1::5] = -0.5
    w[0, 2::9] = 0.4
    ins = []
    for a, dt in ((x, dts[0]), (w, dts[1])):
        ins.append(W.bf16_bits(a) if dt == "bf16" else a)
    gx = to_gpu_bf16(ins[0]) if dts[0] == "bf16" else to_gpu(ins[0])
    gw = to_gpu_bf16(ins[1]) if dts[1] == "bf16" else to_gpu(ins[1])
    for alpha in (0.5, 1.0, 0.0):
        s = gpu_lib.smooth(gx, gw, alpha)
        torch.cuda.synchronize()
        so = oracle.smooth(ins[0], ins[1], alpha)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32)), alpha


def test_smooth_zero_channel(gpu_lib):
    d = W.w8a8(m=64, n=64, k=256)
    x = d["x"].copy()
    x[:, 5] = 0
    s = gpu_lib.smooth(to_gpu_bf16(x), to_gpu_bf16(d["w"]), 0.5).cpu().numpy()
    assert s[5] == 1.0
    assert np.array_equal(s.view(np.uint32), oracle.smooth(x, d["w"], 0.5).view(np.uint32))


# M >= 256 with K % 64 == 0 takes the three-stage ring kernel (256 x 128 tiles): ragged M and N, one K step,
# K = 65 steps; (255, 64, 64) is just below it
@pytest.mark.parametrize("mnk", [(1, 1, 16), (3, 5, 32), (128, 128, 64), (129, 257, 80), (200, 1000, 4096),
                                 (64, 11008, 4096), (2048, 130, 4096), (256, 128, 64), (257, 136, 4160),
                                 (513, 385, 1024), (700, 1000, 192), (255, 64, 64)])
def test_gemm_s8_bitexact(gpu_lib, mnk):
    m, n, k = mnk
    announce("gemm s8 %s" % (mnk,))
    rng = np.random.default_rng(m * 1000 + n + k)
    a = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    b = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    a[0, :] = 127
    b[0, :] = -127  # extreme accumulators
    c = gpu_lib.gemm_s8s8s32(to_gpu(a), to_gpu(b))
    torch.cuda.synchronize()
    ref = oracle.gemm_s8(a, b)
    assert np.array_equal(c.cpu().numpy().astype(np.int64), ref)


# 256 x 384 tiles that fill 192..256 CUs in one round take the wide kernel: ragged M and N (partial last
# tiles), one K step, three (one pass of the three-stage loop) and five (loop plus a two-step tail)
@pytest.mark.parametrize("mnk", [(2000, 11000, 64), (1800, 10500, 192), (1537, 12288, 320), (2048, 9000, 128),
                                 (2048, 10997, 64)])
def test_gemm_s8_wide_bitexact(gpu_lib, mnk):
    m, n, k = mnk
    announce("gemm s8 wide %s" % (mnk,))
    rng = np.random.default_rng(m + n * 7 + k)
    a = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    b = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    a[m - 1, :] = -127
    b[n - 1, :] = -127  # extreme accumulators in the last (partial) tiles
    c = gpu_lib.gemm_s8s8s32(to_gpu(a), to_gpu(b))
    torch.cuda.synchronize()
    ref = oracle.gemm_s8(a, b)
    assert np.array_equal(c.cpu().numpy().astype(np.int64), ref)


def test_w8a8_full_layer(gpu_lib):
    """The whole W8A8 path at 2048x11008x4096: smoothing factor, weight codes/scales, activation codes/scales
    bit-exact; int32 accumulators bit-exact and bf16 outputs within tolerance on 96 sampled tokens."""
    announce("w8a8 full layer")
    d = W.w8a8()
    xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
    s = gpu_lib.smooth(xg, wg, 0.5)
    w_q, s_w, _ = gpu_lib.quantize(wg, 8, True, 1, 0, s, 2)
    y, x_q, s_x = gpu_lib.qlinear_w8a8(xg, s, w_q, s_w, out_dtype=torch.bfloat16)
    acc = gpu_lib.gemm_s8s8s32(x_q, w_q)
    torch.cuda.synchronize()
    so = oracle.smooth(d["x"], d["w"], 0.5)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    qw, sw, _ = oracle.quantize(d["w"], 8, True, 1, 0, so, 2)
    assert np.array_equal(w_q.cpu().numpy(), qw.astype(np.int8))
    assert np.array_equal(s_w.cpu().numpy().view(np.uint32), sw.view(np.uint32))
    qx, sx, _ = oracle.quantize(d["x"], 8, True, 1, 0, so, 1)
    assert np.array_equal(x_q.cpu().numpy(), qx.astype(np.int8))
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), sx.view(np.uint32))
    rng = np.random.default_rng(4)
    toks = np.unique(np.concatenate([rng.choice(2048, size=94, replace=False), [0, 2047]]))
    acc_ref = oracle.gemm_s8(qx[toks].astype(np.int8), qw.astype(np.int8))
    assert np.array_equal(acc.cpu().numpy()[toks].astype(np.int64), acc_ref)
    y_ref = oracle.w8a8_epilogue(acc_ref, sx[toks], sw)
    err = normwise(to_f64(y)[toks], y_ref)
    assert err <= TOL_BF16, err
    assert_per_element(to_f64(y)[toks], y_ref, abs_terms_i8(qx[toks], sx[toks], qw, sw), BOUND_W8A8_BF16, "W8A8 layer")


@pytest.mark.parametrize("mnk", [(5, 77, 96), (130, 200, 512), (300, 264, 128), (513, 385, 192),
                                 (1800, 10500, 64)])
def test_w8a8_small_fp32_out(gpu_lib, mnk):
    m, n, k = mnk
    announce("w8a8 small %s" % (mnk,))
    d = W.w8a8(m=m, n=n, k=k)
    r = oracle.w8a8(d["x"], d["w"], 0.5)
    xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
    s = gpu_lib.smooth(xg, wg, 0.5)
    w_q, s_w, _ = gpu_lib.quantize(wg, 8, True, 1, 0, s, 2)
    y, x_q, s_x = gpu_lib.qlinear_w8a8(xg, s, w_q, s_w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(x_q.cpu().numpy(), r["q_x"])
    assert np.array_equal(w_q.cpu().numpy(), r["q_w"])
    err = normwise(to_f64(y), r["y"])
    assert err <= TOL_F32, err
    assert_per_element(to_f64(y), r["y"], abs_terms_i8(r["q_x"], r["s_x"], r["q_w"], r["s_w"]), BOUND_W8A8_F32, "W8A8")
    # pre-quantized activations (x = NULL): only the GEMM + epilogue runs, same result bit for bit
    y2, _, _ = gpu_lib.qlinear_w8a8(None, None, w_q, s_w, out_dtype=torch.float32, x_q=x_q, x_scales=s_x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("mnk", [(130, 200, 512), (77, 196, 96), (256, 264, 128), (513, 384, 1024),
                                 (300, 385, 128), (2000, 11000, 128), (1800, 10501, 64)])
def test_w8a8_small_bf16_out(gpu_lib, mnk):
    """bf16 epilogue on ragged tiles: N % 8 == 0 takes the LDS-staged store path, N % 8 != 0 the direct one
    (M >= 256: in the ring kernel; 2000 x 11000 and 1800 x 10501: in the wide kernel)."""
    m, n, k = mnk
    announce("w8a8 small bf16 %s" % (mnk,))
    d = W.w8a8(m=m, n=n, k=k)
    r = oracle.w8a8(d["x"], d["w"], 0.5)
    xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
    s = gpu_lib.smooth(xg, wg, 0.5)
    w_q, s_w, _ = gpu_lib.quantize(wg, 8, True, 1, 0, s, 2)
    y, x_q, s_x = gpu_lib.qlinear_w8a8(xg, s, w_q, s_w, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(x_q.cpu().numpy(), r["q_x"])
    assert np.array_equal(w_q.cpu().numpy(), r["q_w"])
    err = normwise(to_f64(y), r["y"])
    assert err <= TOL_BF16, err
    assert_per_element(to_f64(y), r["y"], abs_terms_i8(r["q_x"], r["s_x"], r["q_w"], r["s_w"]), BOUND_W8A8_BF16, "W8A8 bf16")


def test_w8a8_bf16_out_unaligned_matches(gpu_lib):
    """The wide kernel's bf16 epilogue into an output that is not 16-byte aligned (stores straight from the
    accumulators) gives the same bits as into an aligned one (rows staged through LDS); the aligned result is
    checked against the oracle at this shape in test_w8a8_small_bf16_out."""
    announce("w8a8 bf16 unaligned output")
    m, n, k = 2000, 11000, 128
    d = W.w8a8(m=m, n=n, k=k)
    xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
    s = gpu_lib.smooth(xg, wg, 0.5)
    w_q, s_w, _ = gpu_lib.quantize(wg, 8, True, 1, 0, s, 2)
    y, x_q, s_x = gpu_lib.qlinear_w8a8(xg, s, w_q, s_w, out_dtype=torch.bfloat16)
    assert y.data_ptr() % 16 == 0
    buf = torch.empty(m * n + 4, dtype=torch.bfloat16, device=y.device)
    y_off = buf[4:].view(m, n)
    assert y_off.data_ptr() % 16 == 8
    gpu_lib.qlinear_w8a8(None, None, w_q, s_w, out=y_off, x_q=x_q, x_scales=s_x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_off.view(torch.int16))


# --------------------------------------------------------------------------- static per-tensor path

# The scale is 0.7 x the calibration batch's own per-tensor scale, so that about the top 30 % of the range
# clips; ragged row counts, one 32-column chunk, fp32 and bf16 inputs, the per-token scale fill.
@pytest.mark.parametrize("shape", [(1, 32), (7, 96), (130, 4096), (2048, 4096)])
@pytest.mark.parametrize("bits,sym", [(8, True), (8, False), (4, True), (4, False)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_static_bitexact(gpu_lib, shape, bits, sym, dtype):
    rows, cols = shape
    announce("quantize static %s bits=%d sym=%s %s" % (shape, bits, sym, dtype))
    x = W.w8a8_calibration(m=rows, k=cols)
    xc = W.w8a8(m=max(rows, 8), n=8, k=cols)["x"]
    _, sc, zc = oracle.quantize(xc, bits, sym, oracle.TENSOR)
    scale = np.float32(sc[0] * np.float32(0.7))
    zero = 0 if sym else int(zc[0])
    xin = x if dtype == "bf16" else W.bf16_to_f32(x)
    xg = to_gpu_bf16(x) if dtype == "bf16" else to_gpu(W.bf16_to_f32(x))
    codes, rs = gpu_lib.quantize_static(xg, bits, sym, float(scale), zero, row_scales=True)
    torch.cuda.synchronize()
    q = oracle.quantize_static(xin, bits, sym, scale, zero)
    want = oracle_codes_bytes(q, bits, sym)
    got = codes.cpu().numpy()
    assert got.shape == want.shape
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
    assert np.array_equal(rs.cpu().numpy().view(np.uint32), np.full(rows, scale, np.float32).view(np.uint32))
    qmax = (1 << (bits - 1)) - 1 if sym else (1 << bits) - 1
    assert (q == qmax).any()  # the 0.7 x scale did make values clip


def w8a8_static_gpu(gpu_lib, xc_prime, x_prime, xcal, w, out_dtype):
    """The static pipeline through the library: smoothing factor from the calibration batch, weight codes of
    diag(s) W, the per-tensor scale of the calibration X' (dynamic per-tensor quantize = calibration), static
    codes of X', then the GEMM + epilogue with the per-token copy of that scale."""
    wg = to_gpu_bf16(w)
    s = gpu_lib.smooth(to_gpu_bf16(xcal), wg, 0.5)
    w_q, s_w, _ = gpu_lib.quantize(wg, 8, True, 1, 0, s, 2)
    _, s_cal, _ = gpu_lib.quantize(to_gpu_bf16(xc_prime), 8, True, 0)
    s_x = float(s_cal.cpu().numpy()[0])
    x_q, x_scales = gpu_lib.quantize_static(to_gpu_bf16(x_prime), 8, True, s_x, row_scales=True)
    y, _, _ = gpu_lib.qlinear_w8a8(None, None, w_q, s_w, out_dtype=out_dtype, x_q=x_q, x_scales=x_scales)
    torch.cuda.synchronize()
    return s, w_q, s_w, np.float32(s_x), x_q, y


@pytest.mark.parametrize("mnk", [(64, 264, 256), (300, 385, 192), (5, 77, 96)])
def test_w8a8_static_pipeline_small(gpu_lib, mnk):
    """The pages' SmoothQuant pipeline with static per-tensor activations ("第11章 模型量化与压缩" §11.4.5):
    every integer and scale bit-exact, fp32 output within 1e-5 normwise."""
    m, n, k = mnk
    announce("w8a8 static small %s" % (mnk,))
    d = W.w8a8(m=m, n=n, k=k)
    xcal = W.w8a8_calibration(m=128, k=k)
    r = oracle.w8a8_static(xcal, d["x"], d["w"], 0.5)
    xc_prime = oracle.fold_smoothing_bf16(xcal, r["s"])
    s, w_q, s_w, s_x, x_q, y = w8a8_static_gpu(gpu_lib, xc_prime, r["x_prime"], xcal, d["w"], torch.float32)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), r["s"].view(np.uint32))
    assert np.array_equal(w_q.cpu().numpy(), r["q_w"])
    assert np.array_equal(s_w.cpu().numpy().view(np.uint32), r["s_w"].view(np.uint32))
    assert s_x.view(np.uint32) == np.float32(r["s_x"]).view(np.uint32)
    assert np.array_equal(x_q.cpu().numpy(), r["q_x"])
    err = normwise(to_f64(y), r["y"])
    assert err <= TOL_F32, err


def test_w8a8_static_full_layer(gpu_lib):
    """2048 x 11008 x 4096 with a 512-token calibration batch: the smoothing factor, weight codes and scales,
    the calibrated scale and all activation codes bit-exact; int32 accumulators bit-exact and bf16 outputs
    within tolerance on 96 sampled tokens."""
    announce("w8a8 static full layer")
    d = W.w8a8()
    xcal = W.w8a8_calibration()
    so = oracle.smooth(xcal, d["w"], 0.5)
    xc_prime = oracle.fold_smoothing_bf16(xcal, so)
    x_prime = oracle.fold_smoothing_bf16(d["x"], so)
    s, w_q, s_w, s_x, x_q, y = w8a8_static_gpu(gpu_lib, xc_prime, x_prime, xcal, d["w"], torch.bfloat16)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    qw, sw, _ = oracle.quantize(d["w"], 8, True, oracle.ROW, 0, so, oracle.SMOOTH_MUL)
    assert np.array_equal(w_q.cpu().numpy(), qw.astype(np.int8))
    assert np.array_equal(s_w.cpu().numpy().view(np.uint32), sw.view(np.uint32))
    _, sc, _ = oracle.quantize(xc_prime, 8, True, oracle.TENSOR)
    assert s_x.view(np.uint32) == sc[0].view(np.uint32)
    qx = oracle.quantize_static(x_prime, 8, True, sc[0])
    assert np.array_equal(x_q.cpu().numpy(), qx.astype(np.int8))
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([rng.choice(2048, size=94, replace=False), [0, 2047]]))
    acc_ref = oracle.gemm_s8(qx[toks].astype(np.int8), qw.astype(np.int8))
    acc = gpu_lib.gemm_s8s8s32(x_q[torch.from_numpy(toks).cuda()].contiguous(), w_q)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    y_ref = oracle.w8a8_epilogue(acc_ref, np.full(toks.size, sc[0], np.float32), sw)
    err = normwise(to_f64(y)[toks], y_ref)
    assert err <= TOL_BF16, err


# --------------------------------------------------------------------------- W4A8

# Ragged M and N (partial 128-token and 64 / 128-channel tiles), one K step (K = 128), three, eight.
@pytest.mark.parametrize("mnk", [(5, 77, 128), (130, 200, 384), (257, 129, 1024), (64, 264, 256), (300, 385, 512),
                                 (1, 8, 128), (1, 11008, 4096)])
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("sym", [True, False])
def test_w4a8_small_fp32(gpu_lib, mnk, gs, sym):
    m, n, k = mnk
    announce("w4a8 %s g=%d sym=%s" % (mnk, gs, sym))
    rng = np.random.default_rng(m * 31 + n + k + gs)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    qx = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    sx = rng.uniform(0.001, 0.05, m).astype(np.float32)
    codes, s_w, z_w = gpu_lib.quantize(to_gpu(w), 4, sym, 2, gs)
    y = gpu_lib.qlinear_w4a8(to_gpu(qx), to_gpu(sx), codes, s_w, z_w, gs, sym, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize(w, 4, sym, oracle.GROUP, gs)
    assert np.array_equal(codes.cpu().numpy(), oracle.pack_int4(q))
    y_ref = oracle.w4a8(qx, sx, q, so, zo, gs)
    err = normwise(to_f64(y), y_ref)
    assert err <= TOL_F32, err
    assert_per_element(to_f64(y), y_ref, abs_terms_w4a8(qx, sx, q, so, zo, gs), BOUND_W4A8_F32, "W4A8")


@pytest.mark.parametrize("mnk,gs,sym", [((130, 200, 384), 128, True), ((257, 136, 256), 32, False),
                                        ((64, 1000, 512), 64, True)])
def test_w4a8_small_bf16(gpu_lib, mnk, gs, sym):
    m, n, k = mnk
    announce("w4a8 bf16 %s g=%d sym=%s" % (mnk, gs, sym))
    rng = np.random.default_rng(m + n * 3 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    qx = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    sx = rng.uniform(0.001, 0.05, m).astype(np.float32)
    codes, s_w, z_w = gpu_lib.quantize(to_gpu(w), 4, sym, 2, gs)
    y = gpu_lib.qlinear_w4a8(to_gpu(qx), to_gpu(sx), codes, s_w, z_w, gs, sym, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize(w, 4, sym, oracle.GROUP, gs)
    y_ref = oracle.w4a8(qx, sx, q, so, zo, gs)
    err = normwise(to_f64(y), y_ref)
    assert err <= TOL_BF16, err
    assert_per_element(to_f64(y), y_ref, abs_terms_w4a8(qx, sx, q, so, zo, gs), BOUND_BF16, "W4A8 bf16")


def test_w4a8_full_layer(gpu_lib):
    """The W8A8 layer's shapes with INT4 g = 128 weights (2048 x 11008 x 4096): smoothing factor, weight and
    activation codes and scales bit-exact; bf16 outputs within tolerance on 96 sampled tokens."""
    announce("w4a8 full layer")
    d = W.w8a8()
    xg, wg = to_gpu_bf16(d["x"]), to_gpu_bf16(d["w"])
    s = gpu_lib.smooth(xg, wg, 0.5)
    codes, s_w, _ = gpu_lib.quantize(wg, 4, True, 2, 128, s, 2)
    x_q, s_x, _ = gpu_lib.quantize(xg, 8, True, 1, 0, s, 1)
    y = gpu_lib.qlinear_w4a8(x_q, s_x, codes, s_w, None, 128, True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    so = oracle.smooth(d["x"], d["w"], 0.5)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    q, sw, _ = oracle.quantize(d["w"], 4, True, oracle.GROUP, 128, so, oracle.SMOOTH_MUL)
    assert np.array_equal(codes.cpu().numpy(), oracle.pack_int4(q))
    assert np.array_equal(s_w.cpu().numpy().view(np.uint32), sw.view(np.uint32))
    qx, sx, _ = oracle.quantize(d["x"], 8, True, oracle.ROW, 0, so, oracle.SMOOTH_DIV)
    assert np.array_equal(x_q.cpu().numpy(), qx.astype(np.int8))
    rng = np.random.default_rng(6)
    toks = np.unique(np.concatenate([rng.choice(2048, size=94, replace=False), [0, 2047]]))
    y_ref = oracle.w4a8(qx[toks].astype(np.int8), sx[toks], q, sw, None, 128)
    err = normwise(to_f64(y)[toks], y_ref)
    assert err <= TOL_BF16, err
    assert_per_element(to_f64(y)[toks], y_ref, abs_terms_w4a8(qx[toks], sx[toks], q, sw, None, 128), BOUND_BF16,
                       "W4A8 layer")


# --------------------------------------------------------------------------- KV cache


def _kv_input(k_bits, dtype):
    return to_gpu_bf16(k_bits) if dtype == "bf16" else to_gpu(W.bf16_to_f32(k_bits))


@pytest.mark.parametrize("T", [32, 64, 128, 256])
@pytest.mark.parametrize("C,nb", [(64, 1), (192, 3), (1024, 2)])
@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_keys_bitexact(gpu_lib, T, C, nb, sym, dtype):
    announce("kv keys T=%d C=%d nb=%d sym=%s %s" % (T, C, nb, sym, dtype))
    d = W.kv_cache(T * nb, C, outlier_channels=max(1, C // 64))
    src = d["k"] if dtype == "bf16" else W.bf16_to_f32(d["k"])
    q, s, z = gpu_lib.kv_quantize_keys(_kv_input(d["k"], dtype), T, sym)
    torch.cuda.synchronize()
    qo, so, zo = oracle.kv_quantize_keys(src, T, sym)
    assert np.array_equal(q.cpu().numpy().astype(np.int32), qo)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    if not sym:
        assert np.array_equal(z.cpu().numpy(), zo)


@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_kv_dequant_keys_bitexact(gpu_lib, sym, out):
    announce("kv dequant keys sym=%s %s" % (sym, out))
    d = W.kv_cache(256, 192, outlier_channels=3)
    qo, so, zo = oracle.kv_quantize_keys(d["k"], 64, sym)
    codes = to_gpu(qo.astype(np.int8 if sym else np.uint8))
    xh = gpu_lib.kv_dequantize_keys(codes, to_gpu(so), None if sym else to_gpu(zo), 64, sym,
                                    out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    r32, r16 = oracle.kv_dequantize_keys(qo, so, zo, 64)
    if out == "bf16":
        assert np.array_equal(bf16_tensor_bits(xh), r16)
    else:
        assert np.array_equal(xh.cpu().numpy().view(np.uint32), r32.view(np.uint32))


@pytest.mark.parametrize("T,vg,sym,dtype", [(32, 0, True, "bf16"), (64, 64, False, "bf16"), (32, 128, True, "f32"),
                                            (128, 32, False, "f32")])
def test_kv_append_online(gpu_lib, T, vg, sym, dtype):
    """A run of online steps over three sequences that end at different lengths (one is pointed past the cache,
    one at -1, once they end), then the whole cache against the oracle's step-by-step simulation, bit-exact."""
    B, S, C = 3, 3 * T, 256
    announce("kv append T=%d vg=%d sym=%s %s" % (T, vg, sym, dtype))
    d = W.kv_cache(B * S, C, outlier_channels=4)
    ks, vs = d["k"].reshape(B, S, C), d["v"].reshape(B, S, C)
    if dtype == "f32":
        ks, vs = W.bf16_to_f32(ks), W.bf16_to_f32(vs)
    n_tok = [S, T + 7, T]
    nv = C // vg if vg else 1
    ref = {"k_res": np.zeros((B, T, C), ks.dtype), "k_q": np.zeros((B, S, C), np.int32),
           "k_s": np.zeros((B, S // T, C), np.float32), "v_q": np.zeros((B, S, C), np.int32),
           "v_s": np.zeros((B, S, nv), np.float32)}
    if not sym:
        ref["k_z"] = np.zeros((B, S // T, C), np.uint8)
        ref["v_z"] = np.zeros((B, S, nv), np.uint8)
    cache = gpu_lib.kv_cache_alloc(B, S, C, T, vg, sym, torch.bfloat16 if dtype == "bf16" else torch.float32)
    conv = to_gpu_bf16 if dtype == "bf16" else to_gpu
    for step in range(S + 1):
        pos = np.array([step if step < n_tok[b] else (S + 5 if b == 0 else -1) for b in range(B)], np.int64)
        kn = np.ascontiguousarray(np.stack([ks[b, min(step, S - 1)] for b in range(B)]))
        vn = np.ascontiguousarray(np.stack([vs[b, min(step, S - 1)] for b in range(B)]))
        gpu_lib.kv_append(cache, conv(kn), conv(vn), to_gpu(pos), T, vg, sym)
        oracle.kv_append(ref, kn, vn, pos, T, vg, sym)
    torch.cuda.synchronize()
    for key in ("k_q", "v_q"):
        assert np.array_equal(cache[key].cpu().numpy().astype(np.int32), ref[key]), key
    for key in ("k_s", "v_s"):
        assert np.array_equal(cache[key].cpu().numpy().view(np.uint32), ref[key].view(np.uint32)), key
    if not sym:
        for key in ("k_z", "v_z"):
            assert np.array_equal(cache[key].cpu().numpy(), ref[key]), key
    res = bf16_tensor_bits(cache["k_res"]) if dtype == "bf16" else cache["k_res"].cpu().numpy()
    assert np.array_equal(res, ref["k_res"])


@pytest.mark.parametrize("C,dtype,sym", [(64, "bf16", True), (8192, "bf16", False), (8192, "f32", True)])
def test_kv_append_channel_extremes(gpu_lib, C, dtype, sym):
    """The smallest (64) and largest (8192) channel counts of an append step, over two complete groups."""
    B, S, T, vg = 2, 64, 32, 0 if sym else 128
    announce("kv append C=%d %s sym=%s" % (C, dtype, sym))
    d = W.kv_cache(B * S, C, outlier_channels=2)
    ks, vs = d["k"].reshape(B, S, C), d["v"].reshape(B, S, C)
    if dtype == "f32":
        ks, vs = W.bf16_to_f32(ks), W.bf16_to_f32(vs)
    nv = C // vg if vg else 1
    ref = {"k_res": np.zeros((B, T, C), ks.dtype), "k_q": np.zeros((B, S, C), np.int32),
           "k_s": np.zeros((B, S // T, C), np.float32), "v_q": np.zeros((B, S, C), np.int32),
           "v_s": np.zeros((B, S, nv), np.float32)}
    if not sym:
        ref["k_z"] = np.zeros((B, S // T, C), np.uint8)
        ref["v_z"] = np.zeros((B, S, nv), np.uint8)
    cache = gpu_lib.kv_cache_alloc(B, S, C, T, vg, sym, torch.bfloat16 if dtype == "bf16" else torch.float32)
    conv = to_gpu_bf16 if dtype == "bf16" else to_gpu
    for step in range(S):
        pos = np.full(B, step, np.int64)
        kn, vn = np.ascontiguousarray(ks[:, step]), np.ascontiguousarray(vs[:, step])
        gpu_lib.kv_append(cache, conv(kn), conv(vn), to_gpu(pos), T, vg, sym)
        oracle.kv_append(ref, kn, vn, pos, T, vg, sym)
    torch.cuda.synchronize()
    for key in ("k_q", "v_q"):
        assert np.array_equal(cache[key].cpu().numpy().astype(np.int32), ref[key]), key
    for key in ("k_s", "v_s"):
        assert np.array_equal(cache[key].cpu().numpy().view(np.uint32), ref[key].view(np.uint32)), key
    if not sym:
        for key in ("k_z", "v_z"):
            assert np.array_equal(cache[key].cpu().numpy(), ref[key]), key


def test_kv_keys_full_size_sampled(gpu_lib):
    """The measured workload (32 sequences x 4096 tokens of one layer's keys, 1024 channels, T = 128) in one
    launch; sampled token groups against the oracle, bit-exact."""
    announce("kv keys full size")
    d = W.kv_cache(32 * 4096, W.KV_CHANNELS)
    for sym in (True, False):
        q, s, z = gpu_lib.kv_quantize_keys(to_gpu_bf16(d["k"]), 128, sym)
        torch.cuda.synchronize()
        for b in (0, 517, 1023):
            qo, so, zo = oracle.kv_quantize_keys(d["k"][128 * b:128 * b + 128], 128, sym)
            assert np.array_equal(q[128 * b:128 * b + 128].cpu().numpy().astype(np.int32), qo)
            assert np.array_equal(s[b].cpu().numpy().view(np.uint32), so[0].view(np.uint32))
            if not sym:
                assert np.array_equal(z[b].cpu().numpy(), zo[0])


# --------------------------------------------------------------------------- 16-bit metadata


@pytest.mark.parametrize("shape,gs", [((64, 1024), 128), ((77, 384), 64), ((3, 96), 32), ((130, 2048), 32)])
@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_meta16_quantize_bitexact(gpu_lib, shape, gs, sym, dtype):
    """Codes, binary16 scales and packed zero points bit-exact (odd group counts included)."""
    announce("meta16 quantize %s g=%d sym=%s %s" % (shape, gs, sym, dtype))
    rng = np.random.default_rng(shape[0] * 7 + gs)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    w[rng.random(shape) < 0.005] *= 20
    src = W.bf16_bits(w) if dtype == "bf16" else w
    xg = to_gpu_bf16(src) if dtype == "bf16" else to_gpu(src)
    codes, s16, z4 = gpu_lib.quantize_meta16(xg, sym, gs)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize_meta16(src, sym, gs)
    assert np.array_equal(codes.cpu().numpy(), oracle.pack_int4(q))
    assert np.array_equal(s16.cpu().numpy().view(np.uint16), so)
    if not sym:
        assert np.array_equal(z4.cpu().numpy(), oracle.pack_zeros4(zo))


@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_meta16_dequant_bitexact(gpu_lib, sym, out):
    announce("meta16 dequant sym=%s %s" % (sym, out))
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((48, 768)) * 0.02).astype(np.float32)
    q, so, zo = oracle.quantize_meta16(w, sym, 32)
    xh = gpu_lib.dequantize_meta16(to_gpu(oracle.pack_int4(q)), to_gpu(so.view(np.float16)),
                                   None if sym else to_gpu(oracle.pack_zeros4(zo)), 48, 768, sym, 32,
                                   out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    r32, r16 = oracle.dequantize(q, oracle.f16_to_f32(so), zo, oracle.GROUP, 32)
    if out == "bf16":
        assert np.array_equal(bf16_tensor_bits(xh), r16)
    else:
        assert np.array_equal(xh.cpu().numpy().view(np.uint32), r32.view(np.uint32))


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("nk,gs", [((1000, 4096), 128), ((257, 2048), 32), ((64, 384), 64)])
@pytest.mark.parametrize("sym", [True, False])
def test_meta16_gemv(gpu_lib, m, nk, gs, sym):
    """Decode with binary16 scales and packed zero points against the W4A16 reference on the stored values."""
    n, k = nk
    announce("meta16 gemv m=%d %s g=%d sym=%s" % (m, nk, gs, sym))
    rng = np.random.default_rng(n + k + m)
    w = W.bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = W.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    codes, s16, z4 = gpu_lib.quantize_meta16(to_gpu_bf16(w), sym, gs)
    y = gpu_lib.qlinear_w4a16_meta16(to_gpu_bf16(x), codes, s16, z4, gs, sym, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize_meta16(w, sym, gs)
    y_ref = oracle.w4a16(x, q, oracle.f16_to_f32(so), zo, gs)
    err = normwise(to_f64(y), y_ref)
    assert err <= TOL_F32, err
    assert_per_element(to_f64(y), y_ref, abs_terms_w4(x, q, oracle.f16_to_f32(so), zo, gs), BOUND_W4A16_F32, "meta16")


def test_meta16_gemv_70b_gate(gpu_lib):
    """The 70B layer's gate projection (28672 x 8192, INT4 g = 128) at M = 1 with 16-bit metadata: codes and
    scales bit-exact on sampled rows, the output within tolerance on those rows."""
    announce("meta16 gemv 70b gate")
    rows = np.sort(np.random.default_rng(9).choice(28672, 256, replace=False))
    wg = to_gpu_bf16(W.l70b_weight(4))
    x = W.l70b_x(4, 1)
    codes, s16, _ = gpu_lib.quantize_meta16(wg, True, 128)
    y = gpu_lib.qlinear_w4a16_meta16(to_gpu_bf16(x), codes, s16, None, 128, True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    wr = W.l70b_weight(4, rows)
    q, so, _ = oracle.quantize_meta16(wr, True, 128)
    assert np.array_equal(codes.cpu().numpy()[rows], oracle.pack_int4(q))
    assert np.array_equal(s16.cpu().numpy().view(np.uint16).reshape(28672, 64)[rows].ravel(), so)
    y_ref = oracle.w4a16(x, q, oracle.f16_to_f32(so), None, 128)
    err = normwise(to_f64(y)[:, rows], y_ref)
    assert err <= TOL_F32, err
    assert_per_element(to_f64(y)[:, rows], y_ref, abs_terms_w4(x, q, oracle.f16_to_f32(so), None, 128), BOUND_W4A16_F32,
                       "meta16 70B gate")


# --------------------------------------------------------------------------- determinism

def test_reruns_are_bit_identical(gpu_lib):
    d = W.ffn7b(ms=(8,))
    wg = to_gpu_bf16(d["w"])
    xg = to_gpu_bf16(d["x"][:8])
    outs = []
    for _ in range(3):
        codes, s, z = gpu_lib.quantize(wg, 4, False, 2, 32)
        y = gpu_lib.qlinear_w4a16(xg, codes, s, z, 32, False)
        outs.append((codes.cpu().numpy(), bf16_tensor_bits(y)))
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 1 << 20, (1 << 20) + 48])
def test_stream_read_probe_runs(gpu_lib, nbytes):
    """The measurement probe reads any multiple of 16 bytes (grid-stride tail included) and returns cleanly."""
    announce("stream read probe %d B" % nbytes)
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = gpu_lib.stream_read_probe(buf)
    torch.cuda.synchronize()
    assert sink.shape == (1,)
