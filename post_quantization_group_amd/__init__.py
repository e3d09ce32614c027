"""MI355X (gfx950) quantized linear layer: thin Python binding over the C ABI in include/pqg.h.

The functions below carry the names of the C entry points (without the ``pqg_`` prefix). They only
marshal arguments: check tensor dtypes/devices, allocate outputs with ``torch.empty`` on the input's
device, and pass raw device pointers plus the current HIP stream to libpqg.so. Every step of the
computation runs in the library's HIP kernels; there is no CPU or PyTorch fallback, and a missing
library is an error.

Tensor conventions: bf16 tensors are ``torch.bfloat16``; packed INT4 codes are ``torch.uint8``
[rows, cols/2]; INT8 codes are ``torch.int8`` (symmetric) or ``torch.uint8`` (asymmetric).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpqg.so")

# constants of include/pqg.h
OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
F32, BF16 = 0, 1
TENSOR, ROW, GROUP = 0, 1, 2
SMOOTH_NONE, SMOOTH_DIV, SMOOTH_MUL = 0, 1, 2
ABI_VERSION = 1

EXPORTS = [
    "pqg_abi_version", "pqg_last_error", "pqg_quantize_workspace_bytes", "pqg_quantize", "pqg_quantize_static",
    "pqg_dequantize",
    "pqg_smooth_workspace_bytes", "pqg_smooth", "pqg_qlinear_w4a16", "pqg_qlinear_w8a8", "pqg_gemm_s8s8s32",
    "pqg_qlinear_w4a8", "pqg_kv_quantize_keys", "pqg_kv_dequantize_keys", "pqg_kv_append",
    "pqg_quantize_meta16", "pqg_dequantize_meta16", "pqg_qlinear_w4a16_meta16", "pqg_qlinear_w8a8_noalloc",
    "pqg_qlinear_w4a16_grouped", "pqg_stream_read_probe", "pqg_mfma_i8_probe",
]

_lib = None


class W4A16Problem(ctypes.Structure):
    """pqg_w4a16_problem of include/pqg.h."""
    _fields_ = [("x", ctypes.c_void_p), ("w_packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class PqgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("pqg status %d: %s" % (status, message))
        self.status = status


def load(path: str = LIB_PATH):
    """Load libpqg.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libpqg.so is not built (%s); run __graft_entry__.build() or "
                          "python -m post_quantization_group_amd.build" % path)
    lib = ctypes.CDLL(path)
    P, I64, I32, SZ, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
    lib.pqg_abi_version.restype = I32
    lib.pqg_abi_version.argtypes = []
    lib.pqg_last_error.restype = ctypes.c_char_p
    lib.pqg_last_error.argtypes = []
    lib.pqg_quantize_workspace_bytes.restype = SZ
    lib.pqg_quantize_workspace_bytes.argtypes = [I64, I64, I32]
    lib.pqg_quantize.restype = I32
    lib.pqg_quantize.argtypes = [P, I32, I64, I64, P, I32, I32, I32, I32, I32, P, P, P, P, SZ, P]
    lib.pqg_quantize_static.restype = I32
    lib.pqg_quantize_static.argtypes = [P, I32, I64, I64, I32, I32, ctypes.c_float, I32, P, P, P]
    lib.pqg_dequantize.restype = I32
    lib.pqg_dequantize.argtypes = [P, P, P, I64, I64, I32, I32, I32, I32, P, I32, P]
    lib.pqg_smooth_workspace_bytes.restype = SZ
    lib.pqg_smooth_workspace_bytes.argtypes = [I64, I64, I64]
    lib.pqg_smooth.restype = I32
    lib.pqg_smooth.argtypes = [P, I32, I64, P, I32, I64, I64, D, P, P, SZ, P]
    lib.pqg_qlinear_w4a16.restype = I32
    lib.pqg_qlinear_w4a16.argtypes = [P, I64, I64, I64, P, P, P, I32, I32, P, I32, P]
    lib.pqg_qlinear_w8a8.restype = I32
    lib.pqg_qlinear_w8a8.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P, P, P]
    lib.pqg_gemm_s8s8s32.restype = I32
    lib.pqg_gemm_s8s8s32.argtypes = [P, P, I64, I64, I64, P, P]
    lib.pqg_qlinear_w4a8.restype = I32
    lib.pqg_qlinear_w4a8.argtypes = [P, P, I64, I64, I64, P, P, P, I32, I32, P, I32, P]
    lib.pqg_kv_quantize_keys.restype = I32
    lib.pqg_kv_quantize_keys.argtypes = [P, I32, I64, I64, I32, I32, P, P, P, P]
    lib.pqg_kv_dequantize_keys.restype = I32
    lib.pqg_kv_dequantize_keys.argtypes = [P, P, P, I64, I64, I32, I32, P, I32, P]
    lib.pqg_kv_append.restype = I32
    lib.pqg_quantize_meta16.restype = I32
    lib.pqg_quantize_meta16.argtypes = [P, I32, I64, I64, I32, I32, P, P, P, P]
    lib.pqg_dequantize_meta16.restype = I32
    lib.pqg_dequantize_meta16.argtypes = [P, P, P, I64, I64, I32, I32, P, I32, P]
    lib.pqg_qlinear_w4a16_meta16.restype = I32
    lib.pqg_qlinear_w4a16_meta16.argtypes = [P, I64, I64, I64, P, P, P, I32, I32, P, I32, P]
    lib.pqg_kv_append.argtypes = [P, P, I32, I64, I64, P, I64, I32, I32, I32, P, P, P, P, P, P, P, P]
    lib.pqg_qlinear_w4a16_grouped.restype = I32
    lib.pqg_qlinear_w4a16_grouped.argtypes = [ctypes.POINTER(W4A16Problem), I32, I64, I32, I32, I32, P]
    lib.pqg_qlinear_w8a8_noalloc.restype = I32
    lib.pqg_qlinear_w8a8_noalloc.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P]
    lib.pqg_stream_read_probe.restype = I32
    lib.pqg_stream_read_probe.argtypes = [P, I64, P, P]
    lib.pqg_mfma_i8_probe.restype = I32
    lib.pqg_mfma_i8_probe.argtypes = [I64, I32, P, P]
    if lib.pqg_abi_version() != ABI_VERSION:
        raise ImportError("libpqg.so ABI %d != binding ABI %d" % (lib.pqg_abi_version(), ABI_VERSION))
    _lib = lib
    return lib


def _check(status: int):
    if status != OK:
        raise PqgError(status, load().pqg_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _float_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("expected a bfloat16 or float32 tensor, got %s" % t.dtype)


def _dev(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.device


def n_segments(rows: int, cols: int, granularity: int, group_size: int) -> int:
    if granularity == TENSOR:
        return 1
    if granularity == ROW:
        return rows
    return rows * cols // group_size


# ----------------------------------------------------------------------------- entry points

def quantize(x: torch.Tensor, bits: int, symmetric: bool, granularity: int, group_size: int = 0,
             smooth: torch.Tensor | None = None, smooth_mode: int = SMOOTH_NONE, out=None):
    """pqg_quantize. Returns (codes, scales, zeros-or-None). `out` may pass preallocated (codes, scales, zeros)."""
    lib = load()
    dev = _dev(x)
    rows, cols = x.shape
    nseg = n_segments(rows, cols, granularity, group_size) if (granularity != GROUP or group_size > 0) else 0
    if out is None:
        if bits == 4:
            codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        else:
            codes = torch.empty((rows, cols), dtype=torch.int8 if symmetric else torch.uint8, device=dev)
        scales = torch.empty(max(nseg, 1), dtype=torch.float32, device=dev)[:nseg]
        zeros = None if symmetric else torch.empty(max(nseg, 1), dtype=torch.uint8, device=dev)[:nseg]
    else:
        codes, scales, zeros = out
    ws_bytes = lib.pqg_quantize_workspace_bytes(rows, cols, granularity)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    if smooth is not None:
        _dev(smooth)
    _check(lib.pqg_quantize(_ptr(x), _float_dtype(x), rows, cols, _ptr(smooth), smooth_mode, bits, int(symmetric),
                            granularity, group_size, _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(ws), ws_bytes,
                            _stream(dev)))
    return codes, scales, zeros


def quantize_static(x: torch.Tensor, bits: int, symmetric: bool, scale: float, zero: int = 0, out=None,
                    row_scales: bool | torch.Tensor = False):
    """pqg_quantize_static: codes of x with a fixed, calibrated per-tensor (scale, zero). Returns (codes,
    row_scales-or-None); row_scales=True allocates the [rows] per-token copy of the scale that qlinear_w8a8
    takes with x=None (or pass a preallocated fp32 tensor)."""
    lib = load()
    dev = _dev(x)
    rows, cols = x.shape
    if out is None:
        if bits == 4:
            codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        else:
            codes = torch.empty((rows, cols), dtype=torch.int8 if symmetric else torch.uint8, device=dev)
    else:
        codes = out
    if row_scales is True:
        row_scales = torch.empty(rows, dtype=torch.float32, device=dev)
    elif row_scales is False:
        row_scales = None
    _check(lib.pqg_quantize_static(_ptr(x), _float_dtype(x), rows, cols, bits, int(symmetric), float(scale), int(zero),
                                   _ptr(codes), _ptr(row_scales), _stream(dev)))
    return codes, row_scales


def dequantize(codes: torch.Tensor, scales: torch.Tensor, zeros, rows: int, cols: int, bits: int, symmetric: bool,
               granularity: int, group_size: int = 0, out_dtype=torch.float32, out=None):
    """pqg_dequantize -> [rows, cols] tensor of out_dtype (float32 or bfloat16); `out` may be preallocated."""
    lib = load()
    dev = _dev(codes)
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=dev)
    _check(lib.pqg_dequantize(_ptr(codes), _ptr(scales), _ptr(zeros), rows, cols, bits, int(symmetric), granularity,
                              group_size, _ptr(out), _float_dtype(out), _stream(dev)))
    return out


def smooth(x: torch.Tensor, w: torch.Tensor, alpha: float = 0.5):
    """pqg_smooth -> float32 [in_features] smoothing factor."""
    lib = load()
    dev = _dev(x)
    _dev(w)
    tokens, k = x.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("x and w disagree on in_features")
    s = torch.empty(k, dtype=torch.float32, device=dev)
    ws_bytes = lib.pqg_smooth_workspace_bytes(tokens, n, k)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    _check(lib.pqg_smooth(_ptr(x), _float_dtype(x), tokens, _ptr(w), _float_dtype(w), n, k, float(alpha), _ptr(s),
                          _ptr(ws), ws_bytes, _stream(dev)))
    return s


def qlinear_w4a16(x: torch.Tensor, w_packed: torch.Tensor, scales: torch.Tensor, zeros, group_size: int,
                  symmetric: bool, out_dtype=torch.bfloat16, out=None):
    """pqg_qlinear_w4a16: y = x @ dequant(w)^T for bf16 x [M, K] and packed INT4 w [N, K/2]."""
    lib = load()
    dev = _dev(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    M, K = x.shape
    N = w_packed.shape[0]
    if w_packed.shape[1] * 2 != K:
        raise ValueError("w_packed must be [N, K/2]")
    y = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _check(lib.pqg_qlinear_w4a16(_ptr(x), M, N, K, _ptr(w_packed), _ptr(scales), _ptr(zeros), group_size,
                                 int(symmetric), _ptr(y), _float_dtype(y), _stream(dev)))
    return y


def qlinear_w4a16_grouped(xs, ws, scales, zeros, group_size: int, symmetric: bool, out_dtype=torch.bfloat16,
                          outs=None):
    """pqg_qlinear_w4a16_grouped: several products y_i = x_i @ dequant(w_i)^T, in one launch up to 32 tokens.
    xs: bf16 [M, K_i] (M common); ws: packed [N_i, K_i / 2]; scales / zeros: per problem (zeros None when
    symmetric). Returns the list of y_i ([M, N_i] of out_dtype, or the tensors of `outs`)."""
    lib = load()
    n = len(xs)
    if not (len(ws) == len(scales) == n and (zeros is None or len(zeros) == n)):
        raise ValueError("one weight, scale (and zero) tensor per activation tensor")
    dev = _dev(xs[0])
    M = xs[0].shape[0]
    ys = []
    table = (W4A16Problem * n)()
    for i in range(n):
        x, w = xs[i], ws[i]
        _dev(x)
        _dev(w)
        if x.dtype != torch.bfloat16 or x.shape[0] != M:
            raise ValueError("every x must be bfloat16 with the same number of rows")
        N, K = w.shape[0], x.shape[1]
        if w.shape[1] * 2 != K:
            raise ValueError("w_packed must be [N, K/2]")
        y = torch.empty((M, N), dtype=out_dtype, device=dev) if outs is None else outs[i]
        ys.append(y)
        z = None if zeros is None else zeros[i]
        table[i] = W4A16Problem(x.data_ptr(), w.data_ptr(), scales[i].data_ptr(), None if z is None else z.data_ptr(),
                                y.data_ptr(), N, K)
    _check(lib.pqg_qlinear_w4a16_grouped(table, n, M, group_size, int(symmetric), _float_dtype(ys[0]), _stream(dev)))
    return ys


def qlinear_w8a8(x, smooth_s, w_q: torch.Tensor, w_scales: torch.Tensor, out_dtype=torch.bfloat16, out=None,
                 x_q=None, x_scales=None):
    """pqg_qlinear_w8a8: dynamic per-token INT8 activations (after X diag(s)^-1), INT8 GEMM, s_x*s_w epilogue.
    With x None the activations are already quantized: x_q [M, K] int8 and x_scales [M] are inputs and only
    the GEMM + epilogue runs. Returns (y, x_q, x_scales)."""
    lib = load()
    dev = _dev(w_q)
    N, K = w_q.shape
    if x is not None:
        _dev(x)
        if x.dtype != torch.bfloat16:
            raise TypeError("x must be bfloat16")
        M = x.shape[0]
        x_q = torch.empty((M, K), dtype=torch.int8, device=dev) if x_q is None else x_q
        x_scales = torch.empty(M, dtype=torch.float32, device=dev) if x_scales is None else x_scales
    else:
        if x_q is None or x_scales is None:
            raise ValueError("x_q and x_scales are required when x is None")
        M = x_q.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _check(lib.pqg_qlinear_w8a8(_ptr(x), _ptr(smooth_s), _ptr(w_q), _ptr(w_scales), M, N, K, _ptr(y),
                                _float_dtype(y), _ptr(x_q), _ptr(x_scales), _stream(dev)))
    return y, x_q, x_scales


def qlinear_w8a8_noalloc(x: torch.Tensor, smooth_s, w_q: torch.Tensor, w_scales: torch.Tensor,
                         out_dtype=torch.bfloat16, out=None):
    """pqg_qlinear_w8a8_noalloc: as qlinear_w8a8 with x given, the activation codes and scales kept in the
    library's own device array (nothing is allocated by the call; `out` may pass a preallocated y). Returns y."""
    lib = load()
    dev = _dev(w_q)
    _dev(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    N, K = w_q.shape
    M = x.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _check(lib.pqg_qlinear_w8a8_noalloc(_ptr(x), _ptr(smooth_s), _ptr(w_q), _ptr(w_scales), M, N, K, _ptr(y),
                                        _float_dtype(y), _stream(dev)))
    return y


def gemm_s8s8s32(a: torch.Tensor, b: torch.Tensor, out=None):
    """pqg_gemm_s8s8s32: exact int32 [M, N] = a [M, K] (int8) x b [N, K]^T (int8)."""
    lib = load()
    dev = _dev(a)
    M, K = a.shape
    N = b.shape[0]
    c = torch.empty((M, N), dtype=torch.int32, device=dev) if out is None else out
    _check(lib.pqg_gemm_s8s8s32(_ptr(a), _ptr(b), M, N, K, _ptr(c), _stream(dev)))
    return c


def qlinear_w4a8(x_q: torch.Tensor, x_scales: torch.Tensor, w_packed: torch.Tensor, w_scales: torch.Tensor, w_zeros,
                 group_size: int, symmetric: bool, out_dtype=torch.bfloat16, out=None):
    """pqg_qlinear_w4a8: per-token INT8 activation codes x [M, K] (scales [M]) times packed INT4 group codes
    [N, K/2] (scales / zero points [N * K / group_size]) -> y [M, N]."""
    lib = load()
    dev = _dev(x_q)
    if x_q.dtype != torch.int8:
        raise TypeError("x_q must be int8")
    M, K = x_q.shape
    N = w_packed.shape[0]
    if w_packed.shape[1] * 2 != K:
        raise ValueError("w_packed must be [N, K/2]")
    y = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _check(lib.pqg_qlinear_w4a8(_ptr(x_q), _ptr(x_scales), M, N, K, _ptr(w_packed), _ptr(w_scales), _ptr(w_zeros),
                                group_size, int(symmetric), _ptr(y), _float_dtype(y), _stream(dev)))
    return y


def kv_quantize_keys(k: torch.Tensor, block_tokens: int, symmetric: bool, out=None):
    """pqg_kv_quantize_keys: keys [tokens, channels] per channel over groups of block_tokens tokens. Returns
    (codes [tokens, channels] int8 / uint8, scales [tokens / T, channels], zeros or None); `out` may hold
    preallocated (codes, scales, zeros)."""
    lib = load()
    dev = _dev(k)
    tokens, channels = k.shape
    if out is None:
        codes = torch.empty((tokens, channels), dtype=torch.int8 if symmetric else torch.uint8, device=dev)
        scales = torch.empty((tokens // block_tokens, channels), dtype=torch.float32, device=dev)
        zeros = None if symmetric else torch.empty((tokens // block_tokens, channels), dtype=torch.uint8, device=dev)
    else:
        codes, scales, zeros = out
    _check(lib.pqg_kv_quantize_keys(_ptr(k), _float_dtype(k), tokens, channels, block_tokens, int(symmetric),
                                    _ptr(codes), _ptr(scales), _ptr(zeros), _stream(dev)))
    return codes, scales, zeros


def kv_dequantize_keys(codes: torch.Tensor, scales: torch.Tensor, zeros, block_tokens: int, symmetric: bool,
                       out_dtype=torch.bfloat16, out=None):
    """pqg_kv_dequantize_keys -> [tokens, channels] of out_dtype."""
    lib = load()
    dev = _dev(codes)
    tokens, channels = codes.shape
    if out is None:
        out = torch.empty((tokens, channels), dtype=out_dtype, device=dev)
    _check(lib.pqg_kv_dequantize_keys(_ptr(codes), _ptr(scales), _ptr(zeros), tokens, channels, block_tokens,
                                      int(symmetric), _ptr(out), _float_dtype(out), _stream(dev)))
    return out


def kv_cache_alloc(batch: int, max_tokens: int, channels: int, block_tokens: int, v_group_size: int,
                   symmetric: bool, dtype=torch.bfloat16, device="cuda"):
    """Zero-filled cache tensors for kv_append: k_res [B, T, C] of dtype; k_q, v_q [B, S, C] int8 / uint8;
    k_s [B, S / T, C]; v_s [B, S, nv] (nv = 1 per token, else C / v_group_size); k_z / v_z or None."""
    cd = torch.int8 if symmetric else torch.uint8
    nv = channels // v_group_size if v_group_size else 1
    c = {"k_res": torch.zeros((batch, block_tokens, channels), dtype=dtype, device=device),
         "k_q": torch.zeros((batch, max_tokens, channels), dtype=cd, device=device),
         "k_s": torch.zeros((batch, max_tokens // block_tokens, channels), dtype=torch.float32, device=device),
         "v_q": torch.zeros((batch, max_tokens, channels), dtype=cd, device=device),
         "v_s": torch.zeros((batch, max_tokens, nv), dtype=torch.float32, device=device),
         "k_z": None, "v_z": None}
    if not symmetric:
        c["k_z"] = torch.zeros((batch, max_tokens // block_tokens, channels), dtype=torch.uint8, device=device)
        c["v_z"] = torch.zeros((batch, max_tokens, nv), dtype=torch.uint8, device=device)
    return c


def kv_append(cache: dict, k_new: torch.Tensor, v_new: torch.Tensor, positions: torch.Tensor, block_tokens: int,
              v_group_size: int, symmetric: bool):
    """pqg_kv_append: one online step; k_new / v_new [B, C], positions int64 [B] on the device; `cache` as
    kv_cache_alloc returns it (updated in place)."""
    lib = load()
    dev = _dev(k_new)
    if positions.dtype != torch.int64 or positions.device != k_new.device:
        raise TypeError("positions must be an int64 tensor on the same device")
    B, C = k_new.shape
    S = cache["k_q"].shape[1]
    _check(lib.pqg_kv_append(_ptr(k_new), _ptr(v_new), _float_dtype(k_new), B, C, _ptr(positions), S, block_tokens,
                             v_group_size, int(symmetric), _ptr(cache["k_res"]), _ptr(cache["k_q"]),
                             _ptr(cache["k_s"]), _ptr(cache["k_z"]), _ptr(cache["v_q"]), _ptr(cache["v_s"]),
                             _ptr(cache["v_z"]), _stream(dev)))


def quantize_meta16(x: torch.Tensor, symmetric: bool, group_size: int, out=None):
    """pqg_quantize_meta16: INT4 groups with binary16 scales. Returns (codes uint8 [rows, cols / 2], scales16 int16
    tensor of binary16 bits [rows * cols / g] (view it as torch.float16 for values), zeros4 uint8 or None)."""
    lib = load()
    dev = _dev(x)
    rows, cols = x.shape
    ng = rows * cols // group_size
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales16 = torch.empty(ng, dtype=torch.float16, device=dev)
        zeros4 = None if symmetric else torch.empty((ng + 1) // 2, dtype=torch.uint8, device=dev)
    else:
        codes, scales16, zeros4 = out
    _check(lib.pqg_quantize_meta16(_ptr(x), _float_dtype(x), rows, cols, int(symmetric), group_size, _ptr(codes),
                                   _ptr(scales16), _ptr(zeros4), _stream(dev)))
    return codes, scales16, zeros4


def dequantize_meta16(codes: torch.Tensor, scales16: torch.Tensor, zeros4, rows: int, cols: int, symmetric: bool,
                      group_size: int, out_dtype=torch.float32, out=None):
    """pqg_dequantize_meta16 -> [rows, cols] of out_dtype."""
    lib = load()
    dev = _dev(codes)
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=dev)
    _check(lib.pqg_dequantize_meta16(_ptr(codes), _ptr(scales16), _ptr(zeros4), rows, cols, int(symmetric),
                                     group_size, _ptr(out), _float_dtype(out), _stream(dev)))
    return out


def qlinear_w4a16_meta16(x: torch.Tensor, w_packed: torch.Tensor, scales16: torch.Tensor, zeros4, group_size: int,
                         symmetric: bool, out_dtype=torch.bfloat16, out=None):
    """pqg_qlinear_w4a16_meta16: decode (M <= 4) with binary16 scales and packed zero points."""
    lib = load()
    dev = _dev(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    M, K = x.shape
    N = w_packed.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _check(lib.pqg_qlinear_w4a16_meta16(_ptr(x), M, N, K, _ptr(w_packed), _ptr(scales16), _ptr(zeros4), group_size,
                                        int(symmetric), _ptr(y), _float_dtype(y), _stream(dev)))
    return y


def stream_read_probe(buf: torch.Tensor, sink: torch.Tensor = None) -> torch.Tensor:
    """pqg_stream_read_probe: one streaming read of `buf` (a contiguous device tensor whose byte size is a
    multiple of 16), for measuring the device's read rate. Returns the 1-element int32 sink (its value is
    meaningless)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    dev = _dev(buf)
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(load().pqg_stream_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(dev)))
    return sink


def mfma_i8_probe(blocks: int, iters: int, sink: torch.Tensor) -> torch.Tensor:
    """pqg_mfma_i8_probe: `blocks` blocks of 8 waves, each wave issuing 12 * iters int8 32x32x32 matrix
    instructions from registers (blocks * 8 * 12 * iters * 65536 ops), for measuring the int8 matrix-core rate
    the device sustains. `sink` is a 1-element int32 device tensor (its value is meaningless)."""
    if not sink.is_cuda:
        raise ValueError("sink must be a device tensor")
    dev = _dev(sink)
    _check(load().pqg_mfma_i8_probe(int(blocks), int(iters), _ptr(sink), _stream(dev)))
    return sink
