"""Adversarial inputs for the rounding step of affine quantization -- test infrastructure only.

The codes of the method are q = clamp(round(x / s) + z, qmin, qmax): the binary32 quotient x / s, correctly
rounded, then round half to even, then the zero point ("量化、蒸馏与模型压缩", core formula;
"大模型压缩：从研究到生产的完整攻略（1）", symmetric and asymmetric quantization). A fast implementation may form
x * (1 / s) instead of x / s. The two differ in the last bit, and that changes the code only when the
quotient lies at, or within a few ulps of, a half-integer. This module builds segments (groups, rows,
tensors, the token groups of one key channel) whose values sit exactly there:

  * near-ties: values whose quotient is within a few ulps of a half-integer, including those where the
    reciprocal product and the correctly rounded quotient round to different integers ("separating"
    values);
  * the special segments the definition singles out: exact ties at an exact scale, an odd zero point with
    ties (round, then add z), an all-zero range, a range whose scale underflows to 0, subnormal scales and
    values, constant segments, one-signed segments, and ranges near the top of binary32.

It only chooses inputs. Its own estimate of a segment's scale is used to aim values at half-integers; every
expected result in the tests comes from the oracle, never from this module.
"""
from __future__ import annotations

import numpy as np

import workloads as W

F32 = np.float32
_BF16_POS = None


def to_dtype_values(v: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values as the input dtype holds them (bf16: rounded to nearest even)."""
    v = np.ascontiguousarray(v, np.float32)
    return W.bf16_to_f32(W.bf16_bits(v)) if dtype == "bf16" else v


def as_input(v: np.ndarray, dtype: str) -> np.ndarray:
    """The array handed to both sides: uint16 bf16 bit patterns, or float32."""
    v = np.ascontiguousarray(v, np.float32)
    return W.bf16_bits(v) if dtype == "bf16" else v


def code_range(bits: int, sym: bool):
    return (-(2 ** (bits - 1) - 1), 2 ** (bits - 1) - 1) if sym else (0, 2 ** bits - 1)


def estimate_scale(lo, hi, bits: int, sym: bool, meta16: bool = False) -> np.float32:
    """The scale a segment with range [lo, hi] gets (used only to aim values at half-integers)."""
    lo, hi = F32(lo), F32(hi)
    if sym:
        s = F32(max(abs(lo), abs(hi))) / F32(2 ** (bits - 1) - 1)
    else:
        s = (F32(max(hi, 0)) - F32(min(lo, 0))) / F32(2 ** bits - 1)
    if not s > 0:
        s = F32(1)
    if meta16:
        h = np.float16(s)
        if h == 0:
            h = np.float16(2.0 ** -24)
        elif not np.isfinite(h):
            h = np.float16(65504.0)
        s = F32(h)
    return F32(s)


def _bf16_positive():
    global _BF16_POS
    if _BF16_POS is None:
        _BF16_POS = (np.arange(0x0001, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    return _BF16_POS


def candidates(lo, hi, s, dtype: str) -> np.ndarray:
    """Values in [lo, hi] whose quotient by s lies near a half-integer.

    bf16: every bf16 value in the range with |v| >= s / 4 (a few thousand; near-ties are then found by
    classification). fp32: for every half-integer h in range, fl(h s) and its neighbours up to 3 ulps away."""
    lo, hi, s = F32(lo), F32(hi), F32(s)
    if dtype == "bf16":
        p = _bf16_positive()
        p = p[p >= s / F32(4)]
        v = np.concatenate([p, -p])
    else:
        h = np.arange(np.floor(float(lo) / float(s)) - 1, np.ceil(float(hi) / float(s)) + 1) + 0.5
        x0 = (h * np.float64(s)).astype(np.float32)
        parts = [x0]
        up, dn = x0, x0
        for _ in range(3):
            up = np.nextafter(up, F32(np.inf))
            dn = np.nextafter(dn, F32(-np.inf))
            parts += [up, dn]
        v = np.concatenate(parts)
    v = v[np.isfinite(v) & (v >= lo) & (v <= hi)]
    return np.unique(v)


def classify(v: np.ndarray, s) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(separating, tie, distance): separating where round(fl(v * fl(1/s))) != round(fl(v / s)); tie where
    fl(v / s) is exactly a half-integer; distance of fl(v / s) from the nearest half-integer."""
    s = F32(s)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        t = (v / s).astype(np.float32)
        tr = (v * (F32(1) / s)).astype(np.float32)
        sep = np.rint(t) != np.rint(tr)
        frac = t - np.floor(t)
        tie = frac == F32(0.5)
        dist = np.abs(frac.astype(np.float64) - 0.5)
    return sep, tie, dist


def near_tie_segment(rng: np.random.Generator, L: int, bits: int, sym: bool, dtype: str, meta16: bool = False,
                     tries: int = 64):
    """One segment of L values: its range ends, then separating values, exact ties and the nearest near-ties.
    Returns (values float32 [L], number of separating values, number of exact ties)."""
    best = None
    for _ in range(tries):
        a = F32(np.exp(rng.uniform(np.log(1e-3), np.log(1e2))))
        if sym:
            lo, hi = -a, a
        else:
            u = rng.choice([0.0, 1.0, rng.uniform(0.05, 0.95)], p=[0.1, 0.1, 0.8])
            lo, hi = F32(-u * a), F32((1 - u) * a)
        lo, hi = to_dtype_values(np.array([lo, hi]), dtype)
        if not hi > lo:
            continue
        s = estimate_scale(lo, hi, bits, sym, meta16)
        v = candidates(lo, hi, s, dtype)
        if v.size == 0:
            continue
        sep, tie, dist = classify(v, s)
        if best is None or sep.sum() > best[-1].sum():
            best = (lo, hi, v, dist, tie, sep)
        if sep.any():
            break
    lo, hi, v, dist, tie, sep = best
    if sym:
        ends = [hi if rng.random() < 0.5 else -hi]
    else:
        ends = [lo, hi]
    order = np.concatenate([rng.permutation(np.flatnonzero(sep)), rng.permutation(np.flatnonzero(tie & ~sep)),
                            np.argsort(dist, kind="stable")])
    _, first = np.unique(order, return_index=True)
    order = order[np.sort(first)]  # separating first, then ties, then nearest, no repeats
    picks = v[order[: L - len(ends)]]
    vals = np.concatenate([np.array(ends, np.float32), picks])
    if vals.size < L:
        vals = np.concatenate([vals, rng.choice(picks if picks.size else vals, L - vals.size)])
    vals = vals.astype(np.float32)
    rng.shuffle(vals)
    sep_n = int(classify(vals, estimate_scale(lo, hi, bits, sym, meta16))[0].sum())
    tie_n = int(classify(vals, estimate_scale(lo, hi, bits, sym, meta16))[1].sum())
    return vals, sep_n, tie_n


def special_segments(L: int, bits: int, sym: bool, dtype: str) -> list:
    """The segments the definition singles out, each L values long, in the input dtype's values."""
    qmin, qmax = code_range(bits, sym)
    tiny = F32(2.0 ** -133) if dtype == "bf16" else F32(2.0 ** -149)  # smallest subnormal of the dtype
    segs = []

    def pad(vals, fill=0.0):
        vals = list(vals)[:L]
        return np.array(vals + [fill] * (L - len(vals)), np.float32)

    ties = [2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -3.5, 4.5, -5.5, 6.5, -1.5, 5.5]
    if sym:
        # absmax qmax: s = 1 exactly, so every x / s is exact and the ties are real ties
        segs.append(pad([qmax] + [t for t in ties if abs(t) < qmax]))
        # the same at s = 2^-3 and s = 2^4 (exact scalings)
        segs.append(pad([qmax * 0.125] + [t * 0.125 for t in ties if abs(t) < qmax]))
        segs.append(pad([-qmax * 16.0] + [t * 16.0 for t in ties if abs(t) < qmax]))
    else:
        if bits == 8:
            # s = (162 + 93) / 255 = 1 and z = 93 (odd): 0.5 rounds to 0 then adds 93; rounding x / s + z as
            # one number would give 94
            segs.append(pad([-93.0, 162.0, 0.5, 0.0, 1.5, -0.5, 2.5, -92.5, 160.5, -3.5]))
        # s = 1 and z = 7 (odd), ties on both sides of the zero point
        lo4 = -7.0 if bits == 4 else -101.0
        segs.append(pad([lo4, lo4 + qmax] + [t for t in ties if lo4 < t < lo4 + qmax]))
        segs.append(pad([lo4 * 0.25, (lo4 + qmax) * 0.25] + [t * 0.25 for t in ties if lo4 < t < lo4 + qmax]))
    segs.append(np.zeros(L, np.float32))                                    # zero range: s = 1, z = 0
    segs.append(pad([tiny]))                                                 # scale underflows to 0
    segs.append(pad([-tiny, tiny]))
    if dtype == "bf16":
        segs.append(pad([2.0 ** -126, 2.0 ** -127, -2.0 ** -128, 3 * 2.0 ** -130, 2.0 ** -133]))
    else:
        segs.append(pad([1e-40, 3e-41, -2e-41, 7e-42, 1.4e-45, -5e-40]))    # subnormal scale and values
        segs.append(pad([2.0 ** -126, 1e-39, -2.0 ** -127]))
    segs.append(np.full(L, 0.3, np.float32))                                 # constant segments
    segs.append(np.full(L, -1.7, np.float32))
    segs.append(np.full(L, 2.0 ** 20, np.float32))
    g = np.random.default_rng(L * 1000 + bits * 10 + int(sym))
    segs.append(g.uniform(0.5, 2.0, L).astype(np.float32))                  # one-signed segments
    segs.append(-g.uniform(0.01, 3.0, L).astype(np.float32))
    segs.append(pad([1e38, -0.7e38, 3e37, -1e36, 0.5e38]))                   # near the top of binary32
    return [to_dtype_values(s, dtype) for s in segs]


def segments(n: int, L: int, bits: int, sym: bool, dtype: str, seed: int, meta16: bool = False,
             specials: bool = True):
    """n segments of L values (specials first when asked, then near-tie segments), as float32 [n, L] in the
    dtype's values, and the count of separating values among them."""
    rng = np.random.default_rng(seed)
    rows = special_segments(L, bits, sym, dtype) if specials else []
    rows = rows[:n]
    nsep = 0
    while len(rows) < n:
        v, k, _ = near_tie_segment(rng, L, bits, sym, dtype, meta16)
        rows.append(v)
        nsep += k
    return np.stack(rows).astype(np.float32), nsep


def smoothing_powers_of_two(cols: int, seed: int) -> np.ndarray:
    """Per-column smoothing factors 2^k, k in [-2, 2]: dividing or multiplying by them is exact, so a
    near-tie of the smoothed value is a near-tie of the input scaled back."""
    k = np.random.default_rng(seed).integers(-2, 3, cols)
    return np.ldexp(np.ones(cols, np.float32), k).astype(np.float32)


# ----------------------------------------------------------------------------- layouts used by the tests

def quant_layout(bits: int, sym: bool, gran: int, gs: int, dtype: str, seed: int):
    """Input matrices for pqg_quantize whose segments (groups of gs, rows of 512, or the whole tensor) are
    adversarial segments, and the count of separating values they hold. GROUP and ROW give one matrix;
    TENSOR gives several small tensors, each one segment (near-tie tensors, then the special segments)."""
    cols = 512
    if gran == 2:
        segs, nsep = segments(96 * cols // gs, gs, bits, sym, dtype, seed)
        return [segs.reshape(-1, cols)], nsep
    if gran == 1:
        segs, nsep = segments(96, cols, bits, sym, dtype, seed)
        return [segs], nsep
    mats, nsep = [], 0
    for i in range(6):
        segs, k = segments(1, 16 * 256, bits, sym, dtype, seed + i, specials=False)
        mats.append(segs.reshape(16, 256))
        nsep += k
    for s in special_segments(256, bits, sym, dtype):
        mats.append(np.tile(s, (2, 1)))
    return mats, nsep


def static_cases(bits: int, sym: bool, dtype: str, seed: int):
    """(zero point, [(scale, values [rows, 512])], separating count) for static quantization: values at and next
    to every half-integer multiple of each scale, beyond the code range too, for s = 1 (exact ties), a
    subnormal scale and 10 (8-bit) or 64 (4-bit) scales absmax / qmax of random ranges."""
    qmin, qmax = code_range(bits, sym)
    zero = 0 if sym else (7 if bits == 4 else 93)
    rng = np.random.default_rng(seed)
    scales = [F32(1.0), F32(1e-40) if dtype == "f32" else F32(2.0 ** -130)]
    for _ in range(10 if bits == 8 else 64):
        a = F32(np.exp(rng.uniform(np.log(1e-3), np.log(1e2))))
        scales.append(F32(to_dtype_values(np.array([a]), dtype)[0] / F32(qmax)))
    out, nsep = [], 0
    for s in scales:
        lo = F32((qmin - zero - 3) * float(s))
        hi = F32((qmax - zero + 3) * float(s))
        v = candidates(lo, hi, s, dtype)
        if s == 1.0:
            v = np.concatenate([v, (np.arange(qmin - zero - 3, qmax - zero + 3) + 0.5).astype(np.float32)])
        sep, tie, dist = classify(v, s)
        nsep += int(sep.sum())
        pick = np.concatenate([v[sep], v[tie], v[np.argsort(dist, kind="stable")][:2048]])
        n = (pick.size + 511) // 512 * 512
        out.append((s, to_dtype_values(np.resize(pick, n).reshape(-1, 512), dtype)))
    return zero, out, nsep


def key_blocks(T: int, C: int, nb: int, sym: bool, dtype: str, seed: int):
    """Keys [nb * T, C] whose per-channel token groups are adversarial segments of length T (INT8)."""
    segs, nsep = segments(nb * C, T, 8, sym, dtype, seed)
    k = segs.reshape(nb, C, T).transpose(0, 2, 1).reshape(nb * T, C)
    return np.ascontiguousarray(k), nsep
