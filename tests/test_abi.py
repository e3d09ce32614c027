"""The C ABI library on the host (no GPU): it loads, exports every entry point include/pqg.h declares, and
rejects bad arguments with a status and a message before anything is enqueued. No call here reaches a
kernel launch: every one fails validation or is an empty (zero-row) no-op."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pqg.h")

pqg = pytest.importorskip("post_quantization_group_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pqg.LIB_PATH):
        pytest.fail("libpqg.so is not built; run __graft_entry__.build()")
    return pqg.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(pqg_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(pqg.EXPORTS)


def test_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert lib.pqg_abi_version() == pqg.ABI_VERSION


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10001)


def q(lib, **kw):
    a = dict(x=FAKE, x_dtype=1, rows=4, cols=256, smooth=None, smooth_mode=0, bits=4, symmetric=1, gran=2, gs=128,
             codes=FAKE, scales=FAKE, zeros=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.pqg_quantize(a["x"], a["x_dtype"], a["rows"], a["cols"], a["smooth"], a["smooth_mode"], a["bits"],
                            a["symmetric"], a["gran"], a["gs"], a["codes"], a["scales"], a["zeros"], a["ws"],
                            a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,needle", [
    (dict(bits=5), "bits"), (dict(gs=48), "group_size"), (dict(cols=200, gran=1), "multiple of 32"),
    (dict(cols=288, gs=128), "multiple of group_size"), (dict(x_dtype=7), "x_dtype"), (dict(gran=9), "granularity"),
    (dict(symmetric=0), "zeros"), (dict(zeros=FAKE), "zeros must be NULL"), (dict(x=None), "required"),
    (dict(x=MISALIGNED), "misaligned"), (dict(smooth_mode=1), "smooth vector"), (dict(smooth_mode=4), "smooth_mode"),
    (dict(gran=0), "workspace"), (dict(rows=-1), "negative"), (dict(gran=1, cols=65568), "65536"),
])
def test_quantize_rejects(lib, kw, needle):
    rc = q(lib, **kw)
    assert rc in (pqg.EINVAL, pqg.EUNSUPPORTED)
    assert needle in lib.pqg_last_error().decode()


def test_quantize_empty_is_ok(lib):
    assert q(lib, rows=0, x=None, codes=None, scales=None) == pqg.OK
    assert lib.pqg_last_error().decode() == ""


def test_workspace_sizes(lib):
    assert lib.pqg_quantize_workspace_bytes(100, 256, pqg.GROUP) == 0
    assert lib.pqg_quantize_workspace_bytes(100, 256, pqg.ROW) == 0
    assert lib.pqg_quantize_workspace_bytes(100, 256, pqg.TENSOR) > 0
    assert lib.pqg_smooth_workspace_bytes(2048, 11008, 4096) >= 2 * 4096 * 4


@pytest.mark.parametrize("kw,needle", [
    (dict(bits=6), "bits"), (dict(scale=0.0), "scale"), (dict(scale=float("inf")), "scale"),
    (dict(scale=float("nan")), "scale"), (dict(zero=3), "zero must be 0"), (dict(symmetric=0, bits=4, zero=16), "outside"),
    (dict(symmetric=0, zero=-1), "outside"), (dict(cols=200), "multiple of 32"), (dict(x_dtype=5), "x_dtype"),
    (dict(x=None), "required"), (dict(codes=MISALIGNED), "misaligned"), (dict(rows=-2), "negative"),
])
def test_quantize_static_rejects(lib, kw, needle):
    a = dict(x=FAKE, x_dtype=1, rows=4, cols=256, bits=8, symmetric=1, scale=0.5, zero=0, codes=FAKE, row_scales=None)
    a.update(kw)
    rc = lib.pqg_quantize_static(a["x"], a["x_dtype"], a["rows"], a["cols"], a["bits"], a["symmetric"], a["scale"],
                                 a["zero"], a["codes"], a["row_scales"], None)
    assert rc == pqg.EINVAL
    assert needle in lib.pqg_last_error().decode()


def test_quantize_static_empty_is_ok(lib):
    assert lib.pqg_quantize_static(None, 1, 0, 256, 8, 1, 0.5, 0, None, None, None) == pqg.OK


def test_dequantize_rejects(lib):
    rc = lib.pqg_dequantize(FAKE, FAKE, None, 4, 256, 4, 0, 2, 128, FAKE, 0, None)
    assert rc == pqg.EINVAL and "zeros" in lib.pqg_last_error().decode()
    rc = lib.pqg_dequantize(FAKE, FAKE, None, 4, 256, 4, 1, 2, 128, FAKE, 3, None)
    assert rc == pqg.EINVAL and "out_dtype" in lib.pqg_last_error().decode()


def test_smooth_rejects(lib):
    rc = lib.pqg_smooth(FAKE, 1, 16, FAKE, 1, 16, 256, 1.5, FAKE, FAKE, 1 << 20, None)
    assert rc == pqg.EINVAL and "alpha" in lib.pqg_last_error().decode()
    rc = lib.pqg_smooth(FAKE, 1, 16, FAKE, 1, 16, 256, 0.5, FAKE, FAKE, 8, None)
    assert rc == pqg.EINVAL and "workspace" in lib.pqg_last_error().decode()
    rc = lib.pqg_smooth(FAKE, 1, 16, FAKE, 1, 16, 252, 0.5, FAKE, FAKE, 1 << 20, None)
    assert rc == pqg.EINVAL and "multiple of 8" in lib.pqg_last_error().decode()


def test_w4a16_rejects(lib):
    rc = lib.pqg_qlinear_w4a16(FAKE, 1, 64, 256, FAKE, FAKE, None, 96, 1, FAKE, 1, None)
    assert rc == pqg.EINVAL and "group_size" in lib.pqg_last_error().decode()
    rc = lib.pqg_qlinear_w4a16(FAKE, 1, 64, 200, FAKE, FAKE, None, 32, 1, FAKE, 1, None)
    assert rc == pqg.EINVAL and "multiple of group_size" in lib.pqg_last_error().decode()
    rc = lib.pqg_qlinear_w4a16(FAKE, 1, 64, 256, FAKE, FAKE, None, 32, 0, FAKE, 1, None)
    assert rc == pqg.EINVAL and "zeros" in lib.pqg_last_error().decode()
    assert lib.pqg_qlinear_w4a16(None, 0, 64, 256, None, None, None, 32, 1, None, 1, None) == pqg.OK


def test_w8a8_and_gemm_reject(lib):
    rc = lib.pqg_qlinear_w8a8(FAKE, None, FAKE, FAKE, 4, 64, 100, FAKE, 1, FAKE, FAKE, None)
    assert rc == pqg.EINVAL and "multiple of 32" in lib.pqg_last_error().decode()
    rc = lib.pqg_qlinear_w8a8(FAKE, None, FAKE, FAKE, 4, 64, 256, FAKE, 1, None, FAKE, None)
    assert rc == pqg.EINVAL and "required" in lib.pqg_last_error().decode()
    rc = lib.pqg_qlinear_w8a8(None, FAKE, FAKE, FAKE, 4, 64, 256, FAKE, 1, FAKE, FAKE, None)
    assert rc == pqg.EINVAL and "smooth must be NULL" in lib.pqg_last_error().decode()
    rc = lib.pqg_gemm_s8s8s32(FAKE, FAKE, 4, 4, 24, FAKE, None)
    assert rc == pqg.EINVAL and "multiple of 16" in lib.pqg_last_error().decode()
    rc = lib.pqg_gemm_s8s8s32(MISALIGNED, FAKE, 4, 4, 32, FAKE, None)
    assert rc == pqg.EINVAL and "misaligned" in lib.pqg_last_error().decode()


@pytest.mark.parametrize("K,needle", [(0, "K == 0"), (65536 + 16, "above 65536"), (1 << 24, "above 65536"),
                                      (11 << 20, "above 65536")])
def test_gemm_rejects_k_outside_the_exact_range(lib, K, needle):
    """K == 0 would give the kernels zero K steps (their first load address wraps below the operands) and K
    beyond 65536 overflows the 32-bit offsets within a tile or the int32 accumulators: both are rejected on
    the host before any launch, with every pointer a fake that must never be touched."""
    rc = lib.pqg_gemm_s8s8s32(FAKE, FAKE, 2048, 11008, K, FAKE, None)
    assert rc == pqg.EUNSUPPORTED and needle in lib.pqg_last_error().decode()
    rc = lib.pqg_qlinear_w8a8(FAKE, None, FAKE, FAKE, 2048, 11008, K, FAKE, 1, FAKE, FAKE, None)
    assert rc in (pqg.EUNSUPPORTED, pqg.EINVAL) and lib.pqg_last_error().decode()
    if K == 0:
        assert lib.pqg_gemm_s8s8s32(None, None, 0, 11008, 0, None, None) == pqg.OK  # empty: nothing to do


def test_w4a8_rejects_k_zero(lib):
    rc = lib.pqg_qlinear_w4a8(FAKE, FAKE, 4, 64, 0, FAKE, FAKE, None, 128, 1, FAKE, 1, None)
    assert rc == pqg.EUNSUPPORTED and "K == 0" in lib.pqg_last_error().decode()


def test_w4a8_rejects(lib):
    def call(**kw):
        a = dict(xq=FAKE, sx=FAKE, M=4, N=64, K=256, w=FAKE, sw=FAKE, zw=None, g=128, sym=1, y=FAKE, yd=1)
        a.update(kw)
        return lib.pqg_qlinear_w4a8(a["xq"], a["sx"], a["M"], a["N"], a["K"], a["w"], a["sw"], a["zw"], a["g"],
                                    a["sym"], a["y"], a["yd"], None)
    for kw, needle in [(dict(g=96), "group_size"), (dict(K=192), "multiple of 128"), (dict(K=(1 << 24) + 128), "2^24"),
                       (dict(sym=0), "w_zeros"),
                       (dict(zw=FAKE), "must be NULL"), (dict(yd=4), "y_dtype"), (dict(xq=None), "required"),
                       (dict(w=MISALIGNED), "misaligned"), (dict(M=-1), "negative")]:
        assert call(**kw) == pqg.EINVAL, kw
        assert needle in lib.pqg_last_error().decode(), kw
    assert call(M=0, xq=None, sx=None, w=None, sw=None, y=None) == pqg.OK


def test_kv_quantize_keys_rejects(lib):
    def call(**kw):
        a = dict(k=FAKE, kd=1, t=256, c=1024, T=128, sym=1, q=FAKE, s=FAKE, z=None)
        a.update(kw)
        return lib.pqg_kv_quantize_keys(a["k"], a["kd"], a["t"], a["c"], a["T"], a["sym"], a["q"], a["s"], a["z"],
                                        None)
    for kw, needle in [(dict(T=48), "block_tokens"), (dict(t=200), "multiple of block_tokens"),
                       (dict(c=1000), "multiple of 64"), (dict(sym=0), "zeros are required"),
                       (dict(z=FAKE), "must be NULL"), (dict(kd=4), "k_dtype"), (dict(q=None), "required"),
                       (dict(k=MISALIGNED), "misaligned")]:
        assert call(**kw) == pqg.EINVAL, kw
        assert needle in lib.pqg_last_error().decode(), kw
    assert call(t=0, k=None, q=None, s=None) == pqg.OK


def test_kv_dequantize_keys_rejects(lib):
    def call(**kw):
        a = dict(q=FAKE, s=FAKE, z=None, t=256, c=1024, T=128, sym=1, o=FAKE, od=1)
        a.update(kw)
        return lib.pqg_kv_dequantize_keys(a["q"], a["s"], a["z"], a["t"], a["c"], a["T"], a["sym"], a["o"], a["od"],
                                          None)
    for kw, needle in [(dict(T=100), "block_tokens"), (dict(t=130), "multiple of block_tokens"),
                       (dict(c=12), "multiple of 8"), (dict(sym=0), "zeros are required"),
                       (dict(od=3), "out_dtype"), (dict(o=None), "required"), (dict(o=MISALIGNED), "misaligned")]:
        assert call(**kw) == pqg.EINVAL, kw
        assert needle in lib.pqg_last_error().decode(), kw


def test_kv_append_rejects(lib):
    def call(**kw):
        a = dict(kn=FAKE, vn=FAKE, d=1, B=4, C=1024, pos=FAKE, S=4096, T=128, vg=0, sym=1, kr=FAKE, kq=FAKE, ks=FAKE,
                 kz=None, vq=FAKE, vs=FAKE, vz=None)
        a.update(kw)
        return lib.pqg_kv_append(a["kn"], a["vn"], a["d"], a["B"], a["C"], a["pos"], a["S"], a["T"], a["vg"],
                                 a["sym"], a["kr"], a["kq"], a["ks"], a["kz"], a["vq"], a["vs"], a["vz"], None)
    for kw, needle in [(dict(T=16), "block_tokens"), (dict(vg=48), "v_group_size"), (dict(C=1000), "multiple of 64"),
                       (dict(C=16384), "at most 8192"), (dict(C=192, vg=128), "multiple of 64"),
                       (dict(S=4000), "max_tokens"), (dict(sym=0), "required for asymmetric"),
                       (dict(kz=FAKE), "must be NULL"), (dict(pos=None), "required"),
                       (dict(kr=MISALIGNED), "misaligned"), (dict(B=-1), "negative"), (dict(d=5), "dtype")]:
        assert call(**kw) == pqg.EINVAL, kw
        assert needle in lib.pqg_last_error().decode(), kw
    assert call(B=0, kn=None, vn=None, pos=None) == pqg.OK


def test_meta16_rejects(lib):
    def quant(**kw):
        a = dict(x=FAKE, xd=1, r=64, c=1024, sym=1, g=128, q=FAKE, s=FAKE, z=None)
        a.update(kw)
        return lib.pqg_quantize_meta16(a["x"], a["xd"], a["r"], a["c"], a["sym"], a["g"], a["q"], a["s"], a["z"], None)
    for kw, needle in [(dict(g=96), "group_size"), (dict(c=1000), "multiple of group_size"),
                       (dict(sym=0), "zeros4 is required"), (dict(z=FAKE), "must be NULL"), (dict(xd=4), "x_dtype"),
                       (dict(q=None), "required"), (dict(x=MISALIGNED), "misaligned"), (dict(r=-1), "negative")]:
        assert quant(**kw) == pqg.EINVAL, kw
        assert needle in lib.pqg_last_error().decode(), kw

    def lin(**kw):
        a = dict(x=FAKE, M=1, N=64, K=1024, w=FAKE, s=FAKE, z=None, g=128, sym=1, y=FAKE, yd=1)
        a.update(kw)
        return lib.pqg_qlinear_w4a16_meta16(a["x"], a["M"], a["N"], a["K"], a["w"], a["s"], a["z"], a["g"], a["sym"],
                                            a["y"], a["yd"], None)
    assert lin(M=5) == pqg.EUNSUPPORTED
    assert "decode kernel only" in lib.pqg_last_error().decode()
    for kw, needle in [(dict(g=48), "group_size"), (dict(K=1000), "multiple of group_size"),
                       (dict(sym=0), "zeros4 is required"), (dict(s=None), "required"),
                       (dict(w=MISALIGNED), "misaligned"), (dict(yd=7), "y_dtype")]:
        assert lin(**kw) == pqg.EINVAL, kw
        assert needle in lib.pqg_last_error().decode(), kw
    assert lin(M=0, x=None, w=None, s=None, y=None) == pqg.OK


def test_w8a8_noalloc_rejects_before_touching_the_device(lib):
    """Shapes beyond the library's activation array and bad arguments are rejected on the host before the
    device is queried (no GPU here): M above 16384 tokens, M * K above 2^24 codes, x missing."""
    def call(**kw):
        a = dict(x=FAKE, sm=None, wq=FAKE, sw=FAKE, M=2048, N=11008, K=4096, y=FAKE, yd=1)
        a.update(kw)
        return lib.pqg_qlinear_w8a8_noalloc(a["x"], a["sm"], a["wq"], a["sw"], a["M"], a["N"], a["K"], a["y"],
                                            a["yd"], None)
    for kw, rc, needle in [(dict(M=16385, K=32), pqg.EUNSUPPORTED, "16384 tokens"),
                           (dict(M=4097, K=4096), pqg.EUNSUPPORTED, "activation codes"),
                           (dict(M=256, K=65536 + 32), pqg.EUNSUPPORTED, "above 65536"),
                           (dict(x=None), pqg.EINVAL, "x is required"), (dict(K=100), pqg.EINVAL, "multiple of 32"),
                           (dict(yd=9), pqg.EINVAL, "y_dtype"), (dict(wq=None), pqg.EINVAL, "required"),
                           (dict(x=MISALIGNED), pqg.EINVAL, "misaligned"), (dict(M=-1), pqg.EINVAL, "negative"),
                           (dict(K=0, M=4), pqg.EUNSUPPORTED, "K == 0")]:
        assert call(**kw) == rc, kw
        assert needle in lib.pqg_last_error().decode(), (kw, lib.pqg_last_error())
    assert call(M=0, x=None) == pqg.OK


def test_w4a16_grouped_rejects(lib):
    """Every problem is checked on the host before anything is enqueued."""
    P = pqg.W4A16Problem

    def call(n=2, M=1, g=128, sym=1, yd=1, **kw):
        probs = (P * max(n, 1))()
        for i in range(max(n, 1)):
            probs[i] = P(0x10000, 0x10000, 0x10000, None, 0x10000, 1024, 8192)
        for k, v in kw.items():
            i, field = k.split("_", 1)
            setattr(probs[int(i[1:])], field, v)
        return lib.pqg_qlinear_w4a16_grouped(probs, n, M, g, sym, yd, None)
    for kw, rc, needle in [(dict(n=0), pqg.EINVAL, "count"), (dict(n=9), pqg.EINVAL, "count"),
                           (dict(M=-1), pqg.EINVAL, "negative"), (dict(g=48), pqg.EINVAL, "group_size"),
                           (dict(yd=3), pqg.EINVAL, "y_dtype"), (dict(p1_K=8000), pqg.EINVAL, "problem 1"),
                           (dict(p0_x=None), pqg.EINVAL, "required"), (dict(sym=0), pqg.EINVAL, "zeros is required"),
                           (dict(p1_zeros=0x10000), pqg.EINVAL, "must be NULL"), (dict(p1_K=0), pqg.EUNSUPPORTED, "K == 0"),
                           (dict(p0_w_packed=0x10001), pqg.EINVAL, "misaligned"), (dict(p1_N=-1), pqg.EINVAL, "negative")]:
        assert call(**kw) == rc, kw
        assert needle in lib.pqg_last_error().decode(), (kw, lib.pqg_last_error())
    assert call(M=0) == pqg.OK
    assert call(p0_N=0, p1_N=0) == pqg.OK


def test_stream_read_probe_rejects_bad_arguments(lib):
    """The measurement probe validates on the host: bytes a non-negative multiple of 16, a sink, an aligned src."""
    misaligned = ctypes.c_void_p(FAKE.value + 4)
    assert lib.pqg_stream_read_probe(FAKE, 24, FAKE, None) == pqg.EINVAL
    assert lib.pqg_stream_read_probe(FAKE, -16, FAKE, None) == pqg.EINVAL
    assert lib.pqg_stream_read_probe(FAKE, 64, None, None) == pqg.EINVAL
    assert lib.pqg_stream_read_probe(None, 64, FAKE, None) == pqg.EINVAL
    assert lib.pqg_stream_read_probe(misaligned, 64, FAKE, None) == pqg.EINVAL
    assert lib.pqg_stream_read_probe(None, 0, FAKE, None) == pqg.OK


def test_mfma_probe_rejects_bad_arguments(lib):
    """The matrix-core probe validates on the host: blocks in [0, 65535], iters in [0, 2^20], a sink."""
    assert lib.pqg_mfma_i8_probe(-1, 4, FAKE, None) == pqg.EINVAL
    assert lib.pqg_mfma_i8_probe(65536, 4, FAKE, None) == pqg.EINVAL
    assert lib.pqg_mfma_i8_probe(8, -1, FAKE, None) == pqg.EINVAL
    assert lib.pqg_mfma_i8_probe(8, (1 << 20) + 1, FAKE, None) == pqg.EINVAL
    assert lib.pqg_mfma_i8_probe(8, 4, None, None) == pqg.EINVAL
    assert lib.pqg_mfma_i8_probe(0, 4, FAKE, None) == pqg.OK  # empty: nothing enqueued
