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


# Per-element bounds on float outputs: |y - y_ref| <= a |y_ref| + b sum_k |x_k| |w_k|, the second sum being the
# size of the output's terms. a covers the rounding of the output itself (bf16: half an ulp is 2^-9 of |y|),
# b the fp32 accumulation, which is relative to the terms (the W4A16 kernels sum x (16 + u) and subtract
# (16 + off) sum x, so their fp32 sums run about 8 x larger than the result; W4A8 adds one fp32 term per
# group; the W8A8 sum is an exact integer, rounded three times). A single output element off by a few percent
# -- which a normwise error over a whole row hides -- breaks them.
BOUND_BF16 = (2.0 ** -8, 2.0 ** -11)
BOUND_W4A16_F32 = (2.0 ** -20, 2.0 ** -12)
BOUND_W8A8_F32 = (2.0 ** -20, 2.0 ** -40)
BOUND_W8A8_BF16 = (2.0 ** -8, 2.0 ** -40)
BOUND_W4A8_F32 = (2.0 ** -20, 2.0 ** -15)


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


def assert_per_element(y: np.ndarray, y_ref: np.ndarray, terms: np.ndarray, bound, what: str = "") -> None:
    """|y - y_ref| <= bound[0] |y_ref| + bound[1] terms, element by element."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    err = np.abs(y - y_ref)
    lim = bound[0] * np.abs(y_ref) + bound[1] * terms
    bad = np.flatnonzero((err > lim).ravel())
    assert bad.size == 0, "%s: %d of %d outputs outside the per-element bound, worst at %d (|err| %g, bound %g)" % (
        what, bad.size, err.size, bad[0], err.ravel()[bad[0]], lim.ravel()[bad[0]])
