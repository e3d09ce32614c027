"""Small shared helpers for the GPU tests (array conversions and error norms; no method arithmetic)."""
import numpy as np
import torch


def to_gpu_bf16(a_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).cuda()


def to_gpu(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_tensor_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(y: np.ndarray, ref: np.ndarray) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def announce(msg: str) -> None:
    print("[gpu-case] " + msg, flush=True)


# Per-element bounds on float outputs, relative to sum_k |x_k| |w_k| for each output (the size of its terms):
# bf16 outputs 2^-8 (half an ulp of bf16 is 2^-9 of |y|, plus the fp32 accumulation), fp32 outputs of the
# W4A16 products 2^-10 (the 128 + u operands cancel about 45 x in fp32 before the group scale), of the W8A8
# epilogue 2^-20 (three binary32 roundings of an exact integer) and of W4A8 2^-14 (one fp32 sum per group).
# A single wrong element anywhere -- which a normwise error can hide -- breaks them.
REL_BF16 = 2.0 ** -8
REL_W4A16_F32 = 2.0 ** -10
REL_W8A8_F32 = 2.0 ** -20
REL_W4A8_F32 = 2.0 ** -14


def bf16_values(u16: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def abs_terms_w4(x_u16: np.ndarray, q: np.ndarray, s: np.ndarray, z, gs: int) -> np.ndarray:
    """[M, N] sum_k |x[m, k]| |s[n, k/g] (q[n, k] - z[n, k/g])| in binary64 (the dequantized weight is exact)."""
    n, k = q.shape
    sc = np.repeat(np.asarray(s, np.float64).reshape(n, k // gs), gs, axis=1)
    zz = 0 if z is None else np.repeat(np.asarray(z, np.int64).reshape(n, k // gs), gs, axis=1)
    w_hat = np.abs(sc * (q.astype(np.int64) - zz))
    return np.abs(bf16_values(x_u16)) @ w_hat.T


def abs_terms_i8(qx: np.ndarray, sx, qw: np.ndarray, sw) -> np.ndarray:
    """[M, N] s_x[m] s_w[n] sum_k |q_x[m, k]| |q_w[n, k]| in binary64."""
    a = np.abs(qx.astype(np.float64)) @ np.abs(qw.astype(np.float64)).T
    return a * np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]


def abs_terms_w4a8(qx: np.ndarray, sx, q: np.ndarray, s: np.ndarray, z, gs: int) -> np.ndarray:
    """[M, N] s_x[m] sum_k |q_x[m, k]| |s_w[n, k/g] (q[n, k] - z[n, k/g])| in binary64."""
    n, k = q.shape
    sc = np.repeat(np.asarray(s, np.float64).reshape(n, k // gs), gs, axis=1)
    zz = 0 if z is None else np.repeat(np.asarray(z, np.int64).reshape(n, k // gs), gs, axis=1)
    w_hat = np.abs(sc * (q.astype(np.int64) - zz))
    return (np.abs(qx.astype(np.float64)) @ w_hat.T) * np.asarray(sx, np.float64)[:, None]


def assert_per_element(y: np.ndarray, y_ref: np.ndarray, terms: np.ndarray, rel: float, what: str = "") -> None:
    """|y - y_ref| <= rel * terms element by element (an exactly zero reference must come out zero)."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    err = np.abs(y - y_ref)
    bad = np.flatnonzero((err > rel * terms).ravel())
    assert bad.size == 0, "%s: %d of %d outputs outside the per-element bound, worst at %d (|err| %g, bound %g)" % (
        what, bad.size, err.size, bad[0], err.ravel()[bad[0]], rel * terms.ravel()[bad[0]])
