"""GPU parity on the rounding edge cases of the method, through the C ABI, against the oracle.

Every kernel that turns a value into a code computes clamp(round(x / s) + z) with the correctly rounded
binary32 quotient and round half to even ("量化、蒸馏与模型压缩", core formula; "大模型压缩：从研究到生产的完整攻略（1）",
symmetric and asymmetric quantization). The GPU forms x * (1/s) and falls back to the exact quotient near a
half-integer; these tests feed exactly the inputs that separate the two forms -- thousands of near-ties per
case, counted and required -- plus exact ties, odd zero points, zero and underflowing ranges, subnormal
scales and values, constant and one-signed segments, and ranges near the top of binary32 (tests/adversarial.py
builds them). Codes, packed bytes, scales and zero points must match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import adversarial as A
import oracle
from helpers import announce, normwise, to_f64, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _gpu_input(x_in, dtype):
    return to_gpu_bf16(x_in) if dtype == "bf16" else to_gpu(x_in)


def _codes_bytes(q, bits, sym):
    if bits == 4:
        return oracle.pack_int4(q)
    return q.astype(np.int8) if sym else q.astype(np.uint8)


def _assert_codes(got, q, bits, sym, what):
    want = _codes_bytes(q, bits, sym)
    assert got.shape == want.shape, what
    bad = np.flatnonzero(got.view(np.uint8).ravel() != want.view(np.uint8).ravel())
    assert bad.size == 0, "%s: %d code bytes differ, first at %s" % (what, bad.size, bad[:8])


def _assert_scales(got, want, what):
    bad = np.flatnonzero(got.view(np.uint32).ravel() != want.view(np.uint32).ravel())
    assert bad.size == 0, "%s: %d scales differ, first at %s" % (what, bad.size, bad[:8])


# Minimum number of separating values (where fl(x * fl(1/s)) and fl(x / s) round to different integers) a
# case must contain, so that a kernel that skipped the exact fall-back would fail it.
MIN_SEP = {"bf16": 50, "f32": 500}

# ----------------------------------------------------------------------------- pqg_quantize

QUANT_EDGE = [
    # bits, sym, granularity, group_size
    (4, True, 2, 32), (4, True, 2, 64), (4, True, 2, 128), (4, False, 2, 32), (4, False, 2, 128),
    (8, True, 2, 32), (8, False, 2, 64), (8, True, 2, 128),
    (8, True, 1, 0), (8, False, 1, 0), (4, True, 1, 0), (4, False, 1, 0),
    (8, True, 0, 0), (8, False, 0, 0), (4, True, 0, 0), (4, False, 0, 0),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", QUANT_EDGE)
def test_quantize_rounding_edges(gpu_lib, case, dtype):
    bits, sym, gran, gs = case
    mats, nsep = A.quant_layout(bits, sym, gran, gs, dtype, seed=11 + 7 * bits + gs + 3 * gran + int(sym))
    announce("quantize edges %s %s: %d separating values" % (case, dtype, nsep))
    assert nsep >= (MIN_SEP[dtype] if gran != 0 else MIN_SEP[dtype] // 10)
    for i, x in enumerate(mats):
        x_in = A.as_input(x, dtype)
        codes, s, z = gpu_lib.quantize(_gpu_input(x_in, dtype), bits, sym, gran, gs)
        torch.cuda.synchronize()
        q, so, zo = oracle.quantize(x_in, bits, sym, gran, gs)
        what = "matrix %d" % i
        _assert_scales(s.cpu().numpy(), so, what)
        if not sym:
            assert np.array_equal(z.cpu().numpy(), zo), what + ": zero points differ"
        _assert_codes(codes.cpu().numpy(), q, bits, sym, what)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("case", [(8, True, 1, 0), (4, True, 2, 128), (8, False, 2, 32), (4, False, 1, 0)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_rounding_edges_smoothed(gpu_lib, case, mode, dtype):
    """The same segments seen through the smoothing factor: x = v * s_j (activations, divided back) or
    x = v / s_j (weights, multiplied back) with s_j = 2^k, so the smoothed values are exactly the adversarial
    ones."""
    bits, sym, gran, gs = case
    mats, nsep = A.quant_layout(bits, sym, gran, gs, dtype, seed=101 + bits + gs + mode)
    v = mats[0]
    v = np.where(np.abs(v) > 1e37, v / np.float32(64), v).astype(np.float32)  # keep v * 4 finite
    sm = A.smoothing_powers_of_two(v.shape[1], seed=5 + mode)
    x = (v * sm) if mode == 1 else (v / sm)
    x_in = A.as_input(x.astype(np.float32), dtype)
    announce("quantize edges smoothed %s mode=%d %s: %d separating values" % (case, mode, dtype, nsep))
    assert nsep >= MIN_SEP[dtype]
    codes, s, z = gpu_lib.quantize(_gpu_input(x_in, dtype), bits, sym, gran, gs, to_gpu(sm), mode)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize(x_in, bits, sym, gran, gs, sm, mode)
    _assert_scales(s.cpu().numpy(), so, "smoothed")
    if not sym:
        assert np.array_equal(z.cpu().numpy(), zo), "zero points differ"
    _assert_codes(codes.cpu().numpy(), q, bits, sym, "smoothed")


def test_w8a8_activation_codes_edges(gpu_lib):
    """The per-token activation quantize fused into pqg_qlinear_w8a8 (bf16 tokens divided by the smoothing
    factor): adversarial tokens give codes and scales bit-exact, then the int32 product and epilogue."""
    K, N = 512, 96
    segs, nsep = A.segments(64, K, 8, True, "bf16", seed=77)
    segs = np.where(np.abs(segs) > 1e37, segs / np.float32(64), segs).astype(np.float32)
    sm = A.smoothing_powers_of_two(K, seed=3)
    x_in = A.as_input(segs * sm, "bf16")
    announce("w8a8 activation edges: %d separating values" % nsep)
    assert nsep >= MIN_SEP["bf16"]
    rng = np.random.default_rng(4)
    w_q = rng.integers(-127, 128, (N, K)).astype(np.int8)
    s_w = rng.uniform(1e-3, 2e-3, N).astype(np.float32)
    y, x_q, s_x = gpu_lib.qlinear_w8a8(to_gpu_bf16(x_in), to_gpu(sm), to_gpu(w_q), to_gpu(s_w),
                                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    q, so, _ = oracle.quantize(x_in, 8, True, oracle.ROW, 0, sm, oracle.SMOOTH_DIV)
    _assert_codes(x_q.cpu().numpy(), q, 8, True, "activation codes")
    _assert_scales(s_x.cpu().numpy(), so, "activation scales")
    acc = oracle.gemm_s8(q.astype(np.int8), w_q)
    y_ref = oracle.w8a8_epilogue(acc, so, s_w)
    keep = np.linalg.norm(y_ref, axis=1) > 0
    assert normwise(to_f64(y)[keep], y_ref[keep]) <= 1e-5


# ----------------------------------------------------------------------------- pqg_quantize_static

@pytest.mark.parametrize("bits,sym", [(8, True), (8, False), (4, True), (4, False)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_static_rounding_edges(gpu_lib, bits, sym, dtype):
    """A fixed scale: values at and next to every half-integer multiple of it, beyond the code range too (they
    clip), with an odd zero point for the asymmetric codes; plus s = 1 exact ties and a subnormal scale."""
    zero, cases, nsep = A.static_cases(bits, sym, dtype, seed=31 + bits + int(sym))
    for s, x in cases:
        x_in = A.as_input(x, dtype)
        codes, _ = gpu_lib.quantize_static(_gpu_input(x_in, dtype), bits, sym, float(s), zero)
        torch.cuda.synchronize()
        q = oracle.quantize_static(x_in, bits, sym, s, zero)
        _assert_codes(codes.cpu().numpy(), q, bits, sym, "scale %r" % float(s))
    announce("static edges bits=%d sym=%s %s: %d separating values" % (bits, sym, dtype, nsep))
    assert nsep >= MIN_SEP[dtype]


# ----------------------------------------------------------------------------- pqg_quantize_meta16

@pytest.mark.parametrize("gs", [32, 128])
@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_meta16_rounding_edges(gpu_lib, gs, sym, dtype):
    """INT4 groups whose codes come from the stored binary16 scale: values aimed at half-integer multiples of
    that scale, plus the special groups (where the binary16 scale underflows or saturates)."""
    cols = 512
    segs, nsep = A.segments(64 * cols // gs, gs, 4, sym, dtype, seed=51 + gs + int(sym), meta16=True)
    x_in = A.as_input(segs.reshape(-1, cols), dtype)
    announce("meta16 edges g=%d sym=%s %s: %d separating values" % (gs, sym, dtype, nsep))
    assert nsep >= MIN_SEP[dtype] // 2
    codes, s16, z4 = gpu_lib.quantize_meta16(_gpu_input(x_in, dtype), sym, gs)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize_meta16(x_in, sym, gs)
    assert np.array_equal(s16.cpu().numpy().view(np.uint16), so), "binary16 scales differ"
    if not sym:
        assert np.array_equal(z4.cpu().numpy(), oracle.pack_zeros4(zo)), "packed zero points differ"
    _assert_codes(codes.cpu().numpy(), q, 4, True, "meta16 codes")


# ----------------------------------------------------------------------------- KV cache

@pytest.mark.parametrize("T", [32, 128])
@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_keys_rounding_edges(gpu_lib, T, sym, dtype):
    C, nb = 128, 4 if T == 128 else 12
    k, nsep = A.key_blocks(T, C, nb, sym, dtype, seed=61 + T + int(sym))
    k_in = A.as_input(k, dtype)
    announce("kv keys edges T=%d sym=%s %s: %d separating values" % (T, sym, dtype, nsep))
    assert nsep >= MIN_SEP[dtype]
    q, s, z = gpu_lib.kv_quantize_keys(_gpu_input(k_in, dtype), T, sym)
    torch.cuda.synchronize()
    qo, so, zo = oracle.kv_quantize_keys(k_in, T, sym)
    _assert_scales(s.cpu().numpy(), so, "key scales")
    if not sym:
        assert np.array_equal(z.cpu().numpy(), zo), "key zero points differ"
    assert np.array_equal(q.cpu().numpy().astype(np.int32), qo), "key codes differ"


@pytest.mark.parametrize("T,vg,sym,dtype", [(32, 0, True, "bf16"), (32, 64, False, "f32"), (64, 32, True, "f32"),
                                            (32, 0, False, "bf16")])
def test_kv_append_rounding_edges(gpu_lib, T, vg, sym, dtype):
    """Online appends whose value rows (per token, or per group of channels) and completed key groups (per
    channel) are adversarial segments; the whole cache against the oracle's step-by-step run, bit-exact."""
    B, C = 2, 128
    S = 2 * T
    keys, nsep_k = A.key_blocks(T, C, B * S // T, sym, dtype, seed=71 + T)
    vsegs, nsep_v = A.segments(B * S * (C // vg if vg else 1), vg or C, 8, sym, dtype, seed=81 + T + vg)
    ks = keys.reshape(B, S, C)
    vs = vsegs.reshape(B, S, C)
    ks_in, vs_in = A.as_input(ks, dtype), A.as_input(vs, dtype)
    announce("kv append edges T=%d vg=%d sym=%s %s: %d + %d separating values" % (T, vg, sym, dtype, nsep_k,
                                                                                   nsep_v))
    assert nsep_k + nsep_v >= MIN_SEP[dtype]
    nv = C // vg if vg else 1
    ref = {"k_res": np.zeros((B, T, C), ks_in.dtype), "k_q": np.zeros((B, S, C), np.int32),
           "k_s": np.zeros((B, S // T, C), np.float32), "v_q": np.zeros((B, S, C), np.int32),
           "v_s": np.zeros((B, S, nv), np.float32)}
    if not sym:
        ref["k_z"] = np.zeros((B, S // T, C), np.uint8)
        ref["v_z"] = np.zeros((B, S, nv), np.uint8)
    cache = gpu_lib.kv_cache_alloc(B, S, C, T, vg, sym, torch.bfloat16 if dtype == "bf16" else torch.float32)
    for step in range(S):
        pos = np.full(B, step, np.int64)
        kn, vn = np.ascontiguousarray(ks_in[:, step]), np.ascontiguousarray(vs_in[:, step])
        gpu_lib.kv_append(cache, _gpu_input(kn, dtype), _gpu_input(vn, dtype), to_gpu(pos), T, vg, sym)
        oracle.kv_append(ref, kn, vn, pos, T, vg, sym)
    torch.cuda.synchronize()
    for key in ("k_q", "v_q"):
        assert np.array_equal(cache[key].cpu().numpy().astype(np.int32), ref[key]), key
    for key in ("k_s", "v_s"):
        _assert_scales(cache[key].cpu().numpy(), ref[key], key)
    if not sym:
        for key in ("k_z", "v_z"):
            assert np.array_equal(cache[key].cpu().numpy(), ref[key]), key
