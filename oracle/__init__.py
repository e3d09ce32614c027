"""CPU oracle of the quantized linear layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow and independent of the HIP library: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path never does. The arithmetic lives in
``oracle.c`` (strict IEEE binary32, correctly rounded division and square root, round-half-to-even,
binary64/int64 accumulation for reference products); this module only marshals numpy arrays to it.

Sources, by page title and section:
  [P1] "量化、蒸馏与模型压缩" (LLM knowledge atlas, notes 03-05): core formula; error bound; §1.1 groups;
       §2.3 SmoothQuant.
  [P2] "模型压缩：量化、ZeroQuant、LLM.int8() 与 SmoothQuant": §3 basic formula; §4 granularity;
       §11 vector-wise scales; §12-13 SmoothQuant and alpha.
  [P3] "第11章 模型量化与压缩": §11.1.1-§11.1.6 affine quantization, granularity, worked INT4 example;
       §11.3.7 metadata share; §11.4.3-§11.4.5 smoothing factor and W8A8 pipeline; §11.6.2-§11.6.5 KV-cache
       quantization.
  [P5] "大模型压缩：从研究到生产的完整攻略（1）": symmetric / asymmetric worked examples; outliers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

TENSOR, ROW, GROUP = 0, 1, 2
SMOOTH_NONE, SMOOTH_DIV, SMOOTH_MUL = 0, 1, 2
F32, BF16 = 0, 1

# Strict IEEE build: no fast-math, no contraction into FMA, SSE2 scalar math on x86-64.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (when missing or older than its source, or when forced)."""
    with _lock:
        stale = not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
        if force or stale:
            tmp = _LIB + ".tmp%d" % os.getpid()
            subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
            os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.or_quantize.argtypes = [P, I32, I64, I64, P, I32, I32, I32, I32, I32, P, P, P]
        lib.or_quantize.restype = I32
        lib.or_dequantize.argtypes = [P, P, P, I64, I64, I32, I32, P, P]
        lib.or_quantize_static.argtypes = [P, I32, I64, I64, I32, I32, ctypes.c_float, I32, P]
        lib.or_quantize_static.restype = I32
        lib.or_fold_smoothing_bf16.argtypes = [P, I64, I64, P, P]
        lib.or_fold_smoothing_bf16.restype = None
        lib.or_w4a8.argtypes = [P, P, I64, I64, I64, P, P, P, I64, P]
        lib.or_w4a8.restype = I32
        lib.or_kv_keys.argtypes = [P, I32, I64, I64, I64, I32, P, P, P]
        lib.or_quantize_meta16.argtypes = [P, I32, I64, I64, I32, I32, P, P, P]
        lib.or_quantize_meta16.restype = I32
        lib.or_f32_to_f16.argtypes = [ctypes.c_float]
        lib.or_f32_to_f16.restype = ctypes.c_uint16
        lib.or_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.or_f16_to_f32.restype = ctypes.c_float
        lib.or_kv_keys.restype = I32
        lib.or_kv_dequant_keys.argtypes = [P, P, P, I64, I64, I64, P, P]
        lib.or_kv_dequant_keys.restype = I32
        lib.or_dequantize.restype = I32
        lib.or_pack_int4.argtypes = [P, I64, I64, P]
        lib.or_pack_int4.restype = I32
        lib.or_unpack_int4.argtypes = [P, I64, I64, I32, P]
        lib.or_unpack_int4.restype = I32
        lib.or_w4a16.argtypes = [P, I64, I64, I64, P, P, P, I32, P]
        lib.or_w4a16.restype = I32
        lib.or_smooth.argtypes = [P, I32, I64, P, I32, I64, I64, D, P]
        lib.or_smooth.restype = I32
        lib.or_gemm_s8.argtypes = [P, P, I64, I64, I64, P]
        lib.or_gemm_s8.restype = I32
        lib.or_w8a8_epilogue.argtypes = [P, P, P, I64, I64, P]
        lib.or_w8a8_epilogue.restype = None
        lib.or_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.or_f32_to_bf16.restype = ctypes.c_uint16
        lib.or_num_threads.restype = I32
        lib.or_set_num_threads.argtypes = [I32]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _float_input(x):
    """(contiguous array, dtype code): uint16 arrays are bf16 bit patterns, float32 arrays are fp32."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.float32:
        return x, F32
    raise TypeError("oracle inputs are bf16 bit patterns (uint16) or float32, got %s" % x.dtype)


def num_threads() -> int:
    return int(_load().or_num_threads())


def set_num_threads(n: int) -> None:
    _load().or_set_num_threads(int(n))


def n_segments(rows: int, cols: int, granularity: int, group_size: int) -> int:
    """Number of (scale, zero) pairs: 1, rows, or rows*cols/g [P1 §1.1: d_out*d_in/g for groups]."""
    if granularity == TENSOR:
        return 1
    if granularity == ROW:
        return rows
    return rows * cols // group_size


def quantize(x, bits: int, symmetric: bool, granularity: int, group_size: int = 0, smooth=None,
             smooth_mode: int = SMOOTH_NONE):
    """Affine quantization of a 2-D array. Returns (codes int32 [rows, cols], scales float32 [nseg],
    zeros uint8 [nseg] or None when symmetric)."""
    x, dt = _float_input(x)
    rows, cols = x.shape
    nseg = n_segments(rows, cols, granularity, group_size) if rows and cols else 0
    q = np.zeros((rows, cols), np.int32)
    s = np.zeros(max(nseg, 1), np.float32)[:nseg]
    z = None if symmetric else np.zeros(max(nseg, 1), np.uint8)[:nseg]
    sm = None
    if smooth_mode != SMOOTH_NONE:
        sm = np.ascontiguousarray(smooth, dtype=np.float32)
        assert sm.shape == (cols,)
    rc = _load().or_quantize(_ptr(x), dt, rows, cols, _ptr(sm), smooth_mode, bits, int(bool(symmetric)),
                             granularity, group_size, _ptr(q), _ptr(s), _ptr(z))
    if rc != 0:
        raise ValueError("or_quantize rejected its arguments")
    return q, s, z


def dequantize(q, scales, zeros, granularity: int, group_size: int = 0):
    """x_hat = s (q - z). Returns (fp32 values, their bf16 rounding as uint16)."""
    q = np.ascontiguousarray(q, dtype=np.int32)
    rows, cols = q.shape
    s = np.ascontiguousarray(scales, dtype=np.float32)
    z = None if zeros is None else np.ascontiguousarray(zeros, dtype=np.uint8)
    out32 = np.empty((rows, cols), np.float32)
    out16 = np.empty((rows, cols), np.uint16)
    rc = _load().or_dequantize(_ptr(q), _ptr(s), _ptr(z), rows, cols, granularity, group_size, _ptr(out32),
                               _ptr(out16))
    if rc != 0:
        raise ValueError("or_dequantize rejected its arguments")
    return out32, out16


def pack_int4(q):
    q = np.ascontiguousarray(q, dtype=np.int32)
    rows, cols = q.shape
    out = np.empty((rows, cols // 2), np.uint8)
    if _load().or_pack_int4(_ptr(q), rows, cols, _ptr(out)) != 0:
        raise ValueError("pack_int4 needs an even number of columns")
    return out


def unpack_int4(packed, cols: int, symmetric: bool):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    q = np.empty((rows, cols), np.int32)
    if _load().or_unpack_int4(_ptr(packed), rows, cols, int(bool(symmetric)), _ptr(q)) != 0:
        raise ValueError("unpack_int4 needs an even number of columns")
    return q


def w4a16(x_bf16, q, scales, zeros, group_size: int):
    """Reference y = x w_hat^T in binary64 (x bf16 [M, K] as uint16; q unpacked [N, K])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    if x.ndim == 1:
        x = x[None, :]
    q = np.ascontiguousarray(q, dtype=np.int32)
    M, K = x.shape
    N = q.shape[0]
    assert q.shape == (N, K)
    s = np.ascontiguousarray(scales, dtype=np.float32)
    z = None if zeros is None else np.ascontiguousarray(zeros, dtype=np.uint8)
    y = np.empty((M, N), np.float64)
    if _load().or_w4a16(_ptr(x), M, N, K, _ptr(q), _ptr(s), _ptr(z), group_size, _ptr(y)) != 0:
        raise ValueError("or_w4a16 rejected its arguments")
    return y


def w4a16_packed(x_bf16, packed, scales, zeros, group_size: int, symmetric: bool):
    K = packed.shape[1] * 2
    return w4a16(x_bf16, unpack_int4(packed, K, symmetric), scales, zeros, group_size)


def smooth(x, w, alpha: float):
    """SmoothQuant factor s[K] from activations x [T, K] and weights w [N, K]."""
    x, dx = _float_input(x)
    w, dw = _float_input(w)
    T, K = x.shape
    N, K2 = w.shape
    assert K == K2
    s = np.empty(K, np.float32)
    if _load().or_smooth(_ptr(x), dx, T, _ptr(w), dw, N, K, float(alpha), _ptr(s)) != 0:
        raise MemoryError("or_smooth")
    return s


def gemm_s8(a, b):
    """Exact integer product a [M, K] x b [N, K]^T -> int64 [M, N]; raises if a result leaves int32."""
    a = np.ascontiguousarray(a, dtype=np.int8)
    b = np.ascontiguousarray(b, dtype=np.int8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    c = np.empty((M, N), np.int64)
    if _load().or_gemm_s8(_ptr(a), _ptr(b), M, N, K, _ptr(c)) != 0:
        raise OverflowError("an INT32 accumulator would overflow")
    return c


def w8a8_epilogue(acc, s_x, s_w):
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    _load().or_w8a8_epilogue(_ptr(acc), _ptr(np.ascontiguousarray(s_x, np.float32)),
                             _ptr(np.ascontiguousarray(s_w, np.float32)), M, N, _ptr(y))
    return y


def f32_to_bf16(values):
    """Round fp32 values to bf16 (nearest, ties to even) with the oracle's own conversion."""
    f = _load().or_f32_to_bf16
    v = np.asarray(values, dtype=np.float32)
    return np.array([f(float(t)) for t in v.ravel()], np.uint16).reshape(v.shape)


def w8a8(x_bf16, w_bf16, alpha: float = 0.5):
    """The whole W8A8 path of the SmoothQuant pipeline [P3 §11.4.5], in the pages' order:
    smoothing factor; weight INT8 per output channel on diag(s) W; activation INT8 per token on
    X diag(s)^-1 (dynamic); exact integer GEMM; s_x * s_w epilogue. Returns a dict of every stage."""
    s = smooth(x_bf16, w_bf16, alpha)
    q_w, s_w, _ = quantize(w_bf16, 8, True, ROW, smooth=s, smooth_mode=SMOOTH_MUL)
    q_x, s_x, _ = quantize(x_bf16, 8, True, ROW, smooth=s, smooth_mode=SMOOTH_DIV)
    acc = gemm_s8(q_x.astype(np.int8), q_w.astype(np.int8))
    y = w8a8_epilogue(acc, s_x, s_w)
    return {"s": s, "q_w": q_w.astype(np.int8), "s_w": s_w, "q_x": q_x.astype(np.int8), "s_x": s_x,
            "acc": acc, "y": y}


def quantize_static(x, bits: int, symmetric: bool, scale: float, zero: int = 0):
    """Static per-tensor quantization with a given (scale, zero) [P3 §11.1.4; §11.4.5 step 5]: int32 codes
    (unpacked) of a float32 array or of bf16 bit patterns (uint16)."""
    xa, dt = _float_input(x)
    rows, cols = xa.shape
    q = np.empty((rows, cols), np.int32)
    if _load().or_quantize_static(_ptr(xa), dt, rows, cols, bits, int(symmetric), float(np.float32(scale)), int(zero),
                                  _ptr(q)) != 0:
        raise ValueError("bad static quantization parameters")
    return q


def fold_smoothing_bf16(x_bf16, s):
    """X diag(s)^-1 rounded to bf16, as a LayerNorm with s folded into its gain emits it [P3 §11.4.4]."""
    xa = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = xa.shape
    out = np.empty((rows, cols), np.uint16)
    _load().or_fold_smoothing_bf16(_ptr(xa), rows, cols, _ptr(np.ascontiguousarray(s, np.float32)), _ptr(out))
    return out


def w8a8_static(x_cal_bf16, x_bf16, w_bf16, alpha: float = 0.5):
    """The pages' own SmoothQuant pipeline [P3 §11.4.5], in their order: per-channel maxima of the calibration
    activations and of the weights give s (steps 1-2); diag(s) W to INT8 per output channel (steps 3a, 4); s
    folded into the previous LayerNorm, so activations arrive as bf16 X diag(s)^-1 (step 3b, §11.4.4); one
    per-tensor activation scale fixed from the calibration activations (step 5, static); at inference the
    static codes, the exact integer GEMM and the s_x * s_w epilogue (step 6). Returns a dict of every stage."""
    s = smooth(x_cal_bf16, w_bf16, alpha)
    q_w, s_w, _ = quantize(w_bf16, 8, True, ROW, smooth=s, smooth_mode=SMOOTH_MUL)
    xc_prime = fold_smoothing_bf16(x_cal_bf16, s)
    _, s_cal, _ = quantize(xc_prime, 8, True, TENSOR)
    s_x = np.float32(s_cal[0])
    x_prime = fold_smoothing_bf16(x_bf16, s)
    q_x = quantize_static(x_prime, 8, True, s_x)
    acc = gemm_s8(q_x.astype(np.int8), q_w.astype(np.int8))
    y = w8a8_epilogue(acc, np.full(x_prime.shape[0], s_x, np.float32), s_w)
    return {"s": s, "q_w": q_w.astype(np.int8), "s_w": s_w, "x_prime": x_prime, "s_x": s_x,
            "q_x": q_x.astype(np.int8), "acc": acc, "y": y}


def w4a8(q_x, s_x, q_w, s_w, z_w, group_size: int):
    """W4A8 product [P3 §11.4.5, §11.10.2]: q_x int8 [M, K] with per-token s_x [M]; q_w unpacked INT4 codes
    [N, K] with per-group s_w [N * K / g] and z_w (None for symmetric codes) -> binary64 y [M, N]."""
    xq = np.ascontiguousarray(q_x, dtype=np.int8)
    qw = np.ascontiguousarray(q_w, dtype=np.int32)
    M, K = xq.shape
    N = qw.shape[0]
    y = np.empty((M, N), np.float64)
    z = None if z_w is None else np.ascontiguousarray(z_w, dtype=np.uint8)
    if _load().or_w4a8(_ptr(xq), _ptr(np.ascontiguousarray(s_x, np.float32)), M, N, K, _ptr(qw),
                       _ptr(np.ascontiguousarray(s_w, np.float32)), _ptr(z), group_size, _ptr(y)) != 0:
        raise ValueError("group size must divide K")
    return y


def w4a8_pipeline(x_bf16, w_bf16, alpha: float, group_size: int, symmetric: bool):
    """W4A8 with SmoothQuant activations [P3 §11.4.5, §11.10.2]: the smoothing factor; diag(s) W to INT4 per
    group; X diag(s)^-1 to INT8 per token (dynamic); the W4A8 product. Returns a dict of every stage."""
    s = smooth(x_bf16, w_bf16, alpha)
    q_w, s_w, z_w = quantize(w_bf16, 4, symmetric, GROUP, group_size, smooth=s, smooth_mode=SMOOTH_MUL)
    q_x, s_x, _ = quantize(x_bf16, 8, True, ROW, smooth=s, smooth_mode=SMOOTH_DIV)
    y = w4a8(q_x.astype(np.int8), s_x, q_w, s_w, z_w, group_size)
    return {"s": s, "q_w": q_w, "s_w": s_w, "z_w": z_w, "q_x": q_x.astype(np.int8), "s_x": s_x, "y": y}


# ---------------------------------------------------------------- KV cache


def kv_quantize_keys(k, block_tokens: int, symmetric: bool):
    """Keys per channel over blocks of block_tokens consecutive tokens [P3 §11.6.3-§11.6.5]: k [tokens, channels]
    -> (codes int32 [tokens, channels], scales float32 [tokens / T, channels], zeros uint8 same shape or None)."""
    x, dt = _float_input(k)
    tokens, channels = x.shape
    nb = tokens // block_tokens if block_tokens > 0 else 0
    q = np.zeros((tokens, channels), np.int32)
    s = np.zeros((nb, channels), np.float32)
    z = None if symmetric else np.zeros((nb, channels), np.uint8)
    if _load().or_kv_keys(_ptr(x), dt, tokens, channels, block_tokens, int(bool(symmetric)), _ptr(q), _ptr(s),
                          _ptr(z)) != 0:
        raise ValueError("block_tokens must divide the token count")
    return q, s, z


def kv_dequantize_keys(q, scales, zeros, block_tokens: int):
    """x_hat[t, c] = s[t / T, c] (q[t, c] - z[t / T, c]). Returns (fp32 values, their bf16 rounding as uint16)."""
    q = np.ascontiguousarray(q, dtype=np.int32)
    tokens, channels = q.shape
    out32 = np.empty((tokens, channels), np.float32)
    out16 = np.empty((tokens, channels), np.uint16)
    z = None if zeros is None else np.ascontiguousarray(zeros, dtype=np.uint8)
    if _load().or_kv_dequant_keys(_ptr(q), _ptr(np.ascontiguousarray(scales, np.float32)), _ptr(z), tokens, channels,
                                  block_tokens, _ptr(out32), _ptr(out16)) != 0:
        raise ValueError("block_tokens must divide the token count")
    return out32, out16


def kv_append(cache, k_new, v_new, positions, block_tokens: int, v_group_size: int, symmetric: bool):
    """One online append step of a KV cache [P3 §11.6.2: the cache is quantized online, a few new tokens per
    step; §11.6.5: KIVI's grouped on-demand quantization keeps the most recent keys at full precision and
    quantizes a group of T keys per channel once it is complete, values per token on arrival].

    cache: dict of numpy arrays, updated in place, for B sequences of at most S tokens and C channels:
      k_res [B, T, C] (the keys of the incomplete group, as given), k_q [B, S, C], k_s / k_z [B, S / T, C],
      v_q [B, S, C], v_s / v_z [B, S, nv] (nv = 1 per token, or C / v_group_size per group).
    k_new, v_new: [B, C] (bf16 as uint16, or fp32); positions: [B], the token index each sequence appends at.
    A sequence whose position lies outside [0, S) is skipped.
    Values: quantize(v_new[b], per row or per group) -> v_q[b, p], v_s[b, p]. Keys: k_new[b] goes to slot
    p % T of k_res[b]; when p % T == T - 1 the group is complete and is quantized per channel into rows
    [p - T + 1, p] of k_q[b] and block p / T of k_s[b]."""
    B, C = k_new.shape
    S = cache["k_q"].shape[1]
    for b in range(B):
        p = int(positions[b])
        if p < 0 or p >= S:
            continue
        if v_group_size:
            vq, vs, vz = quantize(v_new[b:b + 1], 8, symmetric, GROUP, v_group_size)
        else:
            vq, vs, vz = quantize(v_new[b:b + 1], 8, symmetric, ROW)
        cache["v_q"][b, p] = vq[0]
        cache["v_s"][b, p] = vs
        if not symmetric:
            cache["v_z"][b, p] = vz
        cache["k_res"][b, p % block_tokens] = k_new[b]
        if p % block_tokens == block_tokens - 1:
            kq, ks, kz = kv_quantize_keys(cache["k_res"][b], block_tokens, symmetric)
            cache["k_q"][b, p - block_tokens + 1:p + 1] = kq
            cache["k_s"][b, p // block_tokens] = ks[0]
            if not symmetric:
                cache["k_z"][b, p // block_tokens] = kz[0]


# ---------------------------------------------------------------- 16-bit metadata


def f32_to_f16(v: float) -> int:
    """binary16 bits of a binary32 value, round to nearest even."""
    return int(_load().or_f32_to_f16(float(v)))


def f16_to_f32(h) -> np.ndarray:
    """binary16 bits (array) -> their exact binary32 values."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    f = _load().or_f16_to_f32
    return np.array([f(int(v)) for v in h.ravel()], np.float32).reshape(h.shape)


def quantize_meta16(x, symmetric: bool, group_size: int):
    """INT4 group quantization with binary16 scales [P1 §1.1; P3 §11.3.7]: returns (codes int32 [rows, cols],
    s16 uint16 binary16 bits [rows * cols / g], zeros uint8 [rows * cols / g] or None)."""
    x, dt = _float_input(x)
    rows, cols = x.shape
    nseg = rows * cols // group_size if group_size > 0 else 0
    q = np.zeros((rows, cols), np.int32)
    s16 = np.zeros(nseg, np.uint16)
    z = None if symmetric else np.zeros(nseg, np.uint8)
    if _load().or_quantize_meta16(_ptr(x), dt, rows, cols, int(bool(symmetric)), group_size, _ptr(q), _ptr(s16),
                                  _ptr(z)) != 0:
        raise ValueError("group_size must divide cols")
    return q, s16, z


def pack_zeros4(z) -> np.ndarray:
    """Zero points two per byte, the flattened group index 2i in the low nibble (an odd count ends with a
    high nibble of 0), using the INT4 pack."""
    z = np.ascontiguousarray(z, dtype=np.int32).ravel()
    if z.size % 2:
        z = np.concatenate([z, np.zeros(1, np.int32)])
    return pack_int4(z.reshape(1, -1)).ravel()
