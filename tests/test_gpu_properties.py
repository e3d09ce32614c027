"""Property-based GPU parity (hypothesis, derandomized: every run draws the same cases, so a failure replays).

Small random shapes and value distributions -- plain normal at several magnitudes, half-step grids that put
quotients on exact ties, all-zero rows, constant groups, subnormal and large magnitudes, sparse outliers --
through quantize, dequantize, the binary16-metadata quantize and decode, the KV keys and the W4A16, W8A8 and
W4A8 products, against the oracle on the same inputs.
Bar: codes, packed bytes, scales and zero points bit-exact; dequantized values bit-exact; fp32 products within
1e-5 normwise and within the per-element bounds.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import workloads as W
from helpers import (BOUND_W4A8_F32, BOUND_W4A16_F32, BOUND_W8A8_F32, abs_terms_i8, abs_terms_w4, abs_terms_w4a8,
                     assert_per_element, normwise, to_f64, to_gpu, to_gpu_bf16)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
PROPS = settings(max_examples=30, deadline=None, derandomize=True, database=None,
                 suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])

KINDS = ("normal", "ties", "zeros", "constant", "subnormal", "large", "outliers")


def make_rows(seed: int, rows: int, cols: int, kinds, seg: int) -> np.ndarray:
    """fp32 [rows, cols]; row r follows kinds[r % len(kinds)]. `seg` is the segment length constant rows repeat."""
    rng = np.random.default_rng(seed)
    x = np.empty((rows, cols), np.float64)
    for r in range(rows):
        kind = kinds[r % len(kinds)]
        if kind == "normal":
            v = rng.standard_normal(cols) * rng.choice([1e-3, 0.02, 1.0, 30.0])
        elif kind == "ties":  # a grid of half steps: with the extreme on the grid, x / s lands on exact halves
            v = rng.integers(-15, 16, cols) * 0.5 * 2.0 ** int(rng.integers(-8, 4))
        elif kind == "zeros":
            v = np.zeros(cols)
        elif kind == "constant":
            v = np.repeat(rng.standard_normal(max(1, cols // seg)), seg)[:cols]
        elif kind == "subnormal":
            v = rng.standard_normal(cols) * 1e-39
        elif kind == "large":
            v = rng.standard_normal(cols) * 1e30
        else:  # outliers
            v = rng.standard_normal(cols) * 0.02
            idx = rng.choice(cols, size=max(1, cols // 50), replace=False)
            v[idx] *= 100.0
        x[r] = v
    return x.astype(np.float32)


def codes_bytes(q, bits, sym):
    if bits == 4:
        return oracle.pack_int4(q)
    return q.astype(np.int8) if sym else q.astype(np.uint8)


@PROPS
@given(seed=st.integers(0, 2 ** 32 - 1), rows=st.integers(1, 40), nseg=st.integers(1, 6),
       gs=st.sampled_from([32, 64, 128]), bits=st.sampled_from([4, 8]), sym=st.booleans(),
       gran=st.sampled_from([0, 1, 2]), bf16=st.booleans(),
       kinds=st.lists(st.sampled_from(KINDS), min_size=1, max_size=4))
def test_quantize_dequantize_property(gpu_lib, seed, rows, nseg, gs, bits, sym, gran, bf16, kinds):
    cols = nseg * gs
    g = gs if gran == 2 else 0
    x = make_rows(seed, rows, cols, kinds, gs)
    xh = W.bf16_bits(x) if bf16 else x
    xg = to_gpu_bf16(xh) if bf16 else to_gpu(x)
    codes, s, z = gpu_lib.quantize(xg, bits, sym, gran, g)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize(xh, bits, sym, gran, g)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32)), "scales differ"
    if not sym:
        assert np.array_equal(z.cpu().numpy(), zo), "zero points differ"
    assert np.array_equal(codes.cpu().numpy().view(np.uint8), codes_bytes(q, bits, sym).view(np.uint8)), \
        "codes differ"
    y = gpu_lib.dequantize(codes, s, z, rows, cols, bits, sym, gran, g, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref32, _ = oracle.dequantize(q, so, zo, gran, g)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref32.view(np.uint32)), "dequantized values differ"


PRODUCT_KINDS = ("normal", "ties", "constant", "outliers", "zeros")


@PROPS
@given(seed=st.integers(0, 2 ** 32 - 1), m=st.integers(1, 40), n=st.integers(1, 160),
       ksteps=st.integers(1, 4), gs=st.sampled_from([32, 64, 128]), sym=st.booleans(),
       kinds=st.lists(st.sampled_from(PRODUCT_KINDS), min_size=1, max_size=3))
def test_w4a16_property(gpu_lib, seed, m, n, ksteps, gs, sym, kinds):
    k = 128 * ksteps
    w = make_rows(seed, n, k, kinds, gs)
    wh = W.bf16_bits(w)
    x = W.bf16_bits(make_rows(seed + 1, m, k, ("normal", "ties", "outliers"), gs))
    codes, s, z = gpu_lib.quantize(to_gpu_bf16(wh), 4, sym, 2, gs)
    y = gpu_lib.qlinear_w4a16(to_gpu_bf16(x), codes, s, z, gs, sym, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize(wh, 4, sym, 2, gs)
    y_ref = oracle.w4a16(x, q, so, zo, gs)
    yg = to_f64(y)
    if not np.any(y_ref):
        assert not np.any(yg), "all-zero product came out nonzero"
        return
    assert normwise(yg, y_ref) <= TOL_F32
    assert_per_element(yg, y_ref, abs_terms_w4(x, q, so, zo, gs), BOUND_W4A16_F32, "W4A16 property")


@PROPS
@given(seed=st.integers(0, 2 ** 32 - 1), m=st.integers(1, 300), n=st.integers(1, 300),
       kchunks=st.integers(1, 8), alpha=st.sampled_from([0.0, 0.5, 1.0]),
       kinds=st.lists(st.sampled_from(("normal", "ties", "outliers")), min_size=1, max_size=3))
def test_w8a8_property(gpu_lib, seed, m, n, kchunks, alpha, kinds):
    k = 32 * kchunks
    x = W.bf16_bits(make_rows(seed, m, k, kinds, 32))
    w = W.bf16_bits(make_rows(seed + 1, n, k, ("normal", "outliers"), 32) * np.float32(0.02))
    xg, wg = to_gpu_bf16(x), to_gpu_bf16(w)
    s = gpu_lib.smooth(xg, wg, alpha)
    w_q, s_w, _ = gpu_lib.quantize(wg, 8, True, 1, 0, s, 2)
    y, x_q, s_x = gpu_lib.qlinear_w8a8(xg, s, w_q, s_w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    r = oracle.w8a8(x, w, alpha)
    assert np.array_equal(x_q.cpu().numpy(), r["q_x"]), "activation codes differ"
    assert np.array_equal(w_q.cpu().numpy(), r["q_w"]), "weight codes differ"
    yg = to_f64(y)
    if not np.any(r["y"]):
        assert not np.any(yg), "all-zero product came out nonzero"
        return
    assert normwise(yg, r["y"]) <= TOL_F32
    assert_per_element(yg, r["y"], abs_terms_i8(r["q_x"], r["s_x"], r["q_w"], r["s_w"]), BOUND_W8A8_F32,
                       "W8A8 property")


@PROPS
@given(seed=st.integers(0, 2 ** 32 - 1), m=st.integers(1, 4), n=st.integers(1, 160), ksteps=st.integers(1, 4),
       gs=st.sampled_from([32, 64, 128]), sym=st.booleans(),
       kinds=st.lists(st.sampled_from(PRODUCT_KINDS), min_size=1, max_size=3))
def test_meta16_decode_property(gpu_lib, seed, m, n, ksteps, gs, sym, kinds):
    """Binary16 scales and packed zero points: quantize bit-exact, decode against the W4A16 reference on the
    stored (binary16) scales."""
    k = 128 * ksteps
    wh = W.bf16_bits(make_rows(seed, n, k, kinds, gs))
    x = W.bf16_bits(make_rows(seed + 1, m, k, ("normal", "ties", "outliers"), gs))
    codes, s16, z4 = gpu_lib.quantize_meta16(to_gpu_bf16(wh), sym, gs)
    y = gpu_lib.qlinear_w4a16_meta16(to_gpu_bf16(x), codes, s16, z4, gs, sym, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize_meta16(wh, sym, gs)
    assert np.array_equal(codes.cpu().numpy(), oracle.pack_int4(q)), "codes differ"
    assert np.array_equal(s16.cpu().numpy().view(np.uint16), so), "binary16 scales differ"
    if not sym:
        assert np.array_equal(z4.cpu().numpy(), oracle.pack_zeros4(zo)), "packed zero points differ"
    sf = oracle.f16_to_f32(so)
    y_ref = oracle.w4a16(x, q, sf, zo, gs)
    yg = to_f64(y)
    if not np.any(y_ref):
        assert not np.any(yg), "all-zero product came out nonzero"
        return
    assert normwise(yg, y_ref) <= TOL_F32
    assert_per_element(yg, y_ref, abs_terms_w4(x, q, sf, zo, gs), BOUND_W4A16_F32, "meta16 property")


ACT_KINDS = ("uniform", "zeros", "extreme", "small")


@PROPS
@given(seed=st.integers(0, 2 ** 32 - 1), m=st.integers(1, 200), n=st.integers(1, 300), ksteps=st.integers(1, 4),
       gs=st.sampled_from([32, 64, 128]), sym=st.booleans(),
       wkinds=st.lists(st.sampled_from(PRODUCT_KINDS), min_size=1, max_size=3),
       akinds=st.lists(st.sampled_from(ACT_KINDS), min_size=1, max_size=3))
def test_w4a8_property(gpu_lib, seed, m, n, ksteps, gs, sym, wkinds, akinds):
    """INT8 token codes (uniform, all-zero rows with a zero scale, rows at +-127, rows of small codes) times
    INT4 group weights of the value kinds above, fp32 out, against the oracle."""
    k = 128 * ksteps
    rng = np.random.default_rng(seed)
    qx = np.empty((m, k), np.int8)
    sx = np.empty(m, np.float32)
    for r in range(m):
        kind = akinds[r % len(akinds)]
        if kind == "uniform":
            qx[r] = rng.integers(-127, 128, k)
        elif kind == "zeros":
            qx[r] = 0
        elif kind == "extreme":
            qx[r] = rng.choice(np.array([-127, 127], np.int8), k)
        else:
            qx[r] = rng.integers(-2, 3, k)
        sx[r] = 0.0 if kind == "zeros" else np.float32(rng.uniform(1e-4, 0.05))
    w = make_rows(seed + 1, n, k, wkinds, gs)
    codes, s_w, z_w = gpu_lib.quantize(to_gpu(w), 4, sym, 2, gs)
    y = gpu_lib.qlinear_w4a8(to_gpu(qx), to_gpu(sx), codes, s_w, z_w, gs, sym, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q, so, zo = oracle.quantize(w, 4, sym, oracle.GROUP, gs)
    assert np.array_equal(codes.cpu().numpy(), oracle.pack_int4(q)), "weight codes differ"
    y_ref = oracle.w4a8(qx, sx, q, so, zo, gs)
    yg = to_f64(y)
    if not np.any(y_ref):
        assert not np.any(yg), "all-zero product came out nonzero"
        return
    assert normwise(yg, y_ref) <= TOL_F32
    assert_per_element(yg, y_ref, abs_terms_w4a8(qx, sx, q, so, zo, gs), BOUND_W4A8_F32, "W4A8 property")


@PROPS
@given(seed=st.integers(0, 2 ** 32 - 1), nblocks=st.integers(1, 3), bt=st.sampled_from([32, 64, 128, 256]),
       cblocks=st.integers(1, 4), sym=st.booleans(), bf16=st.booleans(),
       kinds=st.lists(st.sampled_from(KINDS), min_size=1, max_size=4))
def test_kv_keys_property(gpu_lib, seed, nblocks, bt, cblocks, sym, bf16, kinds):
    """Keys per channel over blocks of tokens: channel c follows kinds[c % len(kinds)] along the tokens. Codes,
    scales and zero points bit-exact."""
    tokens, channels = nblocks * bt, 64 * cblocks
    kt = np.ascontiguousarray(make_rows(seed, channels, tokens, kinds, bt).T)
    kh = W.bf16_bits(kt) if bf16 else kt
    q, s, z = gpu_lib.kv_quantize_keys(to_gpu_bf16(kh) if bf16 else to_gpu(kh), bt, sym)
    torch.cuda.synchronize()
    qo, so, zo = oracle.kv_quantize_keys(kh, bt, sym)
    assert np.array_equal(q.cpu().numpy().astype(np.int64), qo.astype(np.int64)), "key codes differ"
    assert np.array_equal(s.cpu().numpy().view(np.uint32).ravel(), so.view(np.uint32).ravel()), "key scales differ"
    if not sym:
        assert np.array_equal(z.cpu().numpy().ravel(), zo.ravel()), "key zero points differ"


@PROPS
@given(seed=st.integers(0, 2 ** 32 - 1), B=st.integers(1, 3), T=st.sampled_from([32, 64]), groups=st.integers(1, 2),
       cblocks=st.integers(1, 3), vg=st.sampled_from([0, 32, 64]), sym=st.booleans(), bf16=st.booleans(),
       kinds=st.lists(st.sampled_from(KINDS), min_size=1, max_size=4))
def test_kv_append_property(gpu_lib, seed, B, T, groups, cblocks, vg, sym, bf16, kinds):
    """Online appends, one token per sequence per step, sequences ending at different lengths (then pointed at
    -1 or past the cache): the key and value token vectors follow the value kinds above (token t of sequence b
    takes kinds[(b + t) % len(kinds)]). The whole cache -- codes, scales, zero points and the residual keys --
    bit-exact against the oracle's step-by-step simulation."""
    S, C = T * groups, 64 * cblocks
    rng = np.random.default_rng(seed)
    ks = make_rows(seed, B * S, C, kinds, 32).reshape(B, S, C)
    vs = make_rows(seed + 1, B * S, C, kinds[::-1], 32).reshape(B, S, C)
    if bf16:
        ks, vs = W.bf16_bits(ks), W.bf16_bits(vs)
    conv = to_gpu_bf16 if bf16 else to_gpu
    n_tok = [int(rng.integers(1, S + 1)) for _ in range(B)]
    nv = C // vg if vg else 1
    ref = {"k_res": np.zeros((B, T, C), ks.dtype), "k_q": np.zeros((B, S, C), np.int32),
           "k_s": np.zeros((B, S // T, C), np.float32), "v_q": np.zeros((B, S, C), np.int32),
           "v_s": np.zeros((B, S, nv), np.float32)}
    if not sym:
        ref["k_z"] = np.zeros((B, S // T, C), np.uint8)
        ref["v_z"] = np.zeros((B, S, nv), np.uint8)
    cache = gpu_lib.kv_cache_alloc(B, S, C, T, vg, sym, torch.bfloat16 if bf16 else torch.float32)
    for step in range(max(n_tok) + 1):
        pos = np.array([step if step < n_tok[b] else (S + 3 if b % 2 else -1) for b in range(B)], np.int64)
        kn = np.ascontiguousarray(ks[:, min(step, S - 1)])
        vn = np.ascontiguousarray(vs[:, min(step, S - 1)])
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
    res = cache["k_res"].view(torch.int16).cpu().numpy().view(np.uint16) if bf16 else cache["k_res"].cpu().numpy()
    assert np.array_equal(res, ref["k_res"]), "residual keys differ"
