"""Seeded synthetic inputs for the quantized linear layer.

This module only draws random tensors; it holds none of the quantization arithmetic. Both the CPU
oracle (in tests) and the HIP library (tests, smoke check, benchmark) consume its arrays, so the two sides
always see identical inputs.

The tensors stand in for the Llama-7B / Llama-70B layers the pages use as examples ("第11章 模型量化与压缩",
§11.1.6 numerical example and §11.10.1 bandwidth model): no trained weights or datasets are involved.

Recipe (every config, see ``describe()``):
  * one numpy PCG64 generator per tensor, seeded from (seed, config id, tensor id) so any tensor can be
    regenerated on its own (the 70B-layer weights use one generator per block of 512 rows);
  * N(0, sigma) = sigma * standard_normal(dtype=float32);
  * outliers are applied in fp32 before the single round-to-nearest-even cast to bf16;
  * outlier entry / column indices are drawn without replacement from their own generator;
  * activations for several batch sizes M are the first M rows of one [max M, K] draw.
Arrays are returned as numpy: float32, or uint16 holding bf16 bit patterns.
"""
from __future__ import annotations

import numpy as np

SEED = 0

# configuration ids (used only to separate generator streams)
TINY, ATTN7B, FFN7B, W8A8, L70B, KV = 1, 2, 3, 4, 5, 6

# Llama-70B-shaped decoder layer: (name, d_out, d_in) in draw order
L70B_PROJ = [
    ("q", 8192, 8192),
    ("k", 1024, 8192),
    ("v", 1024, 8192),
    ("o", 8192, 8192),
    ("gate", 28672, 8192),
    ("up", 28672, 8192),
    ("down", 8192, 28672),
]


def rng(config: int, tensor: int, seed: int = SEED) -> np.random.Generator:
    return np.random.default_rng([seed, config, tensor])


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(g: np.random.Generator, shape, sigma: float) -> np.ndarray:
    a = g.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def activations(config: int, tensor: int, m: int, k: int) -> np.ndarray:
    """bf16 activations [m, k] drawn from N(0, 1)."""
    return bf16_bits(normal(rng(config, tensor), (m, k), 1.0))


# ----------------------------------------------------------------------------- the five workloads

def tiny():
    """256x512 fp32 weight N(0, 0.02); 0.5 % of the entries (655, distinct) x20; x in R^512 N(0, 1) as bf16."""
    w = normal(rng(TINY, 0), (256, 512), 0.02)
    idx = rng(TINY, 1).choice(w.size, size=int(round(0.005 * w.size)), replace=False)
    w.reshape(-1)[idx] *= np.float32(20.0)
    x = activations(TINY, 2, 1, 512)
    return {"w": w, "x": x, "outlier_entries": np.sort(idx)}


def attn7b(ms=(1, 16)):
    """Llama-7B attention-shaped 4096x4096 bf16 N(0, 0.02); activations [max(ms), 4096]."""
    w = bf16_bits(normal(rng(ATTN7B, 0), (4096, 4096), 0.02))
    x = activations(ATTN7B, 1, max(ms), 4096)
    return {"w": w, "x": x}


def ffn7b(ms=(1, 8, 64)):
    """Llama-7B FFN-shaped 11008x4096 bf16 N(0, 0.02); 1 % of the input columns (41) x10."""
    w = normal(rng(FFN7B, 0), (11008, 4096), 0.02)
    cols = np.sort(rng(FFN7B, 1).choice(4096, size=int(round(0.01 * 4096)), replace=False))
    w[:, cols] *= np.float32(10.0)
    x = activations(FFN7B, 2, max(ms), 4096)
    return {"w": bf16_bits(w), "x": x, "outlier_cols": cols}


def w8a8(m: int = 2048, n: int = 11008, k: int = 4096):
    """W8A8 layer: X [m, k] N(0, 1) with 1 % of the channels (41 at k=4096) x50 as systematic outliers;
    W [n, k] N(0, 0.02). Both bf16."""
    x = normal(rng(W8A8, 0), (m, k), 1.0)
    chans = np.sort(rng(W8A8, 1).choice(k, size=int(round(0.01 * k)), replace=False))
    x[:, chans] *= np.float32(50.0)
    w = normal(rng(W8A8, 2), (n, k), 0.02)
    return {"x": bf16_bits(x), "w": bf16_bits(w), "outlier_chans": chans}


def w8a8_calibration(m: int = 512, k: int = 4096):
    """Calibration activations for the W8A8 layer: a second batch from the same distribution (N(0, 1), the
    same 1 % of channels x50), drawn from its own stream. bf16."""
    x = normal(rng(W8A8, 3), (m, k), 1.0)
    chans = np.sort(rng(W8A8, 1).choice(k, size=int(round(0.01 * k)), replace=False))
    x[:, chans] *= np.float32(50.0)
    return bf16_bits(x)


ROW_BLOCK = 512  # rows per generator stream for the large layer weights


def _block_rows(config: int, tensor: int, b: int, nrows: int, k: int, sigma: float) -> np.ndarray:
    return normal(rng(config, 1000 * tensor + b), (nrows, k), sigma)


def blocked_normal(config: int, tensor: int, n: int, k: int, sigma: float, rows=None) -> np.ndarray:
    """[n, k] N(0, sigma) fp32 drawn in blocks of ROW_BLOCK rows, each from its own generator, so the
    blocks are drawn in parallel and any subset of rows is regenerated without drawing the rest.
    `rows` (sorted indices) returns only those rows."""
    from concurrent.futures import ThreadPoolExecutor

    nblk = (n + ROW_BLOCK - 1) // ROW_BLOCK
    if rows is None:
        out = np.empty((n, k), np.float32)

        def fill(b):
            r0 = b * ROW_BLOCK
            r1 = min(n, r0 + ROW_BLOCK)
            out[r0:r1] = _block_rows(config, tensor, b, r1 - r0, k, sigma)

        with ThreadPoolExecutor(8) as ex:
            list(ex.map(fill, range(nblk)))
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, k), np.float32)
    for b in np.unique(rows // ROW_BLOCK):
        r0 = int(b) * ROW_BLOCK
        r1 = min(n, r0 + ROW_BLOCK)
        blk = _block_rows(config, tensor, int(b), r1 - r0, k, sigma)
        sel = (rows // ROW_BLOCK) == b
        out[sel] = blk[rows[sel] - r0]
    return out


def l70b_weight(i: int, rows=None) -> np.ndarray:
    """Projection i of the 70B layer (bf16 N(0, 0.02)); `rows` selects a subset of rows for samples."""
    name, n, k = L70B_PROJ[i]
    return bf16_bits(blocked_normal(L70B, 10 + i, n, k, 0.02, rows))


def l70b_x(i: int, m: int) -> np.ndarray:
    name, n, k = L70B_PROJ[i]
    return activations(L70B, 20 + i, m, k)


KV_CHANNELS = 1024  # one layer's keys (or values) per token: 8 KV heads x head_dim 128 (Llama-3-70B)


def kv_cache(tokens: int, channels: int = KV_CHANNELS, outlier_channels: int = 16):
    """One layer's keys and values for `tokens` cached tokens (all sequences' tokens stacked), token-major
    [tokens, channels], bf16: N(0, 1); the keys' outliers sit in `outlier_channels` channels (x10), the values
    have none. Drawn in blocks of ROW_BLOCK tokens, one generator each."""
    k = blocked_normal(KV, 1, tokens, channels, 1.0)
    chans = np.sort(rng(KV, 3).choice(channels, size=min(outlier_channels, channels), replace=False))
    k[:, chans] *= np.float32(10.0)
    v = blocked_normal(KV, 2, tokens, channels, 1.0)
    return {"k": bf16_bits(k), "v": bf16_bits(v), "outlier_chans": chans}


def describe() -> dict:
    return {
        "generator": "numpy PCG64, default_rng([0, config, tensor]), standard_normal(float32)",
        "bf16": "fp32 -> bf16 round-to-nearest-even after outliers are applied",
        "tiny": "W fp32 256x512 N(0,0.02), 655 entries x20; x bf16 [1,512] N(0,1)",
        "attn7b": "W bf16 4096x4096 N(0,0.02); x bf16 [M,4096] N(0,1), M in {1,16}",
        "ffn7b": "W bf16 11008x4096 N(0,0.02), 41 input columns x10; x bf16 [M,4096], M in {1,8,64}",
        "w8a8": "X bf16 2048x4096 N(0,1), 41 channels x50; W bf16 11008x4096 N(0,0.02)",
        "l70b": "q,k,v,o,gate,up,down bf16 N(0,0.02) (8192x8192, 1024x8192 x2, 8192x8192, 28672x8192 x2, "
                "8192x28672); x bf16 [M,d_in], M in {1,8,32}",
        "kv": "one layer's K and V bf16 [tokens, 1024] N(0,1); 16 key channels x10",
    }
