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
