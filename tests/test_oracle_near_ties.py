"""The oracle on thousands of rounding edge cases, against exact rational arithmetic (CPU).

The code of x is clamp(round(x / s) + z) with x / s the correctly rounded binary32 quotient and round half to
even ("量化、蒸馏与模型压缩", core formula; "大模型压缩：从研究到生产的完整攻略（1）", symmetric and asymmetric
quantization). For every value of the adversarial inputs whose reciprocal product fl(x * fl(1/s)) rounds to a
different integer than fl(x / s) -- the values the GPU parity tests on edge cases are built around -- this
recomputes the code from the oracle's own scale and zero point with Python's exact fractions: the exact
quotient rounded once to binary32 (nearest, ties to even), then to an integer (half to even), then the zero
point and the clamp. It also checks that each input set really holds such values, so the GPU tests that use
the same sets cannot pass by missing them.
"""
from fractions import Fraction

import numpy as np
import pytest

import adversarial as A
import oracle


def _f32_of(r: Fraction) -> np.float32:
    """Round an exact rational to binary32, nearest, ties to even (three candidates around it)."""
    c = np.float32(float(r))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - r)
        key = (d, int(np.float32(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def _half_even(t: np.float32) -> int:
    f = Fraction(float(t))
    n = f.numerator // f.denominator
    rem = f - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def _check_against_fractions(x, q, s_el, z_el, bits, sym, limit=1500):
    qmin, qmax = A.code_range(bits, sym)
    s_el = np.where(s_el == 0, np.float32(1), s_el).astype(np.float32)  # a stored 0: codes took the unit step
    with np.errstate(all="ignore"):
        t = (x / s_el).astype(np.float32)
        tr = (x * (np.float32(1) / s_el)).astype(np.float32)
    sep = np.flatnonzero((np.rint(t) != np.rint(tr)).ravel())
    for i in sep[:limit]:
        xi, si = Fraction(float(x.ravel()[i])), Fraction(float(s_el.ravel()[i]))
        code = _half_even(_f32_of(xi / si)) + int(z_el.ravel()[i])
        code = min(max(code, qmin), qmax)
        assert q.ravel()[i] == code, (i, float(x.ravel()[i]), float(s_el.ravel()[i]))
    return sep.size


MIN_SEP = {"bf16": 50, "f32": 500}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", [(4, True, 2, 32), (4, False, 2, 128), (8, True, 1, 0), (8, False, 2, 64),
                                  (4, True, 0, 0)])
def test_oracle_codes_on_near_ties(case, dtype):
    bits, sym, gran, gs = case
    mats, nsep = A.quant_layout(bits, sym, gran, gs, dtype, seed=11 + 7 * bits + gs + 3 * gran + int(sym))
    assert nsep >= (MIN_SEP[dtype] if gran != 0 else MIN_SEP[dtype] // 10)
    checked = 0
    for x in mats:
        x_in = A.as_input(x, dtype)
        q, s, z = oracle.quantize(x_in, bits, sym, gran, gs)
        rows, cols = x.shape
        seg = np.zeros(x.shape, np.int64)
        if gran == 1:
            seg = np.repeat(np.arange(rows), cols).reshape(rows, cols)
        elif gran == 2:
            seg = np.arange(x.size).reshape(x.shape) // gs
        zz = np.zeros(x.shape, np.int64) if z is None else z[seg].astype(np.int64)
        checked += _check_against_fractions(A.to_dtype_values(x, dtype), q, s[seg], zz, bits, sym)
    assert checked >= (MIN_SEP[dtype] if gran != 0 else MIN_SEP[dtype] // 10)


@pytest.mark.parametrize("bits,sym", [(8, True), (4, False)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_oracle_static_codes_on_near_ties(bits, sym, dtype):
    zero, cases, nsep = A.static_cases(bits, sym, dtype, seed=31 + bits + int(sym))
    assert nsep >= MIN_SEP[dtype]
    for s, x in cases:
        q = oracle.quantize_static(A.as_input(x, dtype), bits, sym, s, zero)
        _check_against_fractions(x, q, np.full(x.shape, s, np.float32), np.full(x.shape, zero), bits, sym, 300)


def test_oracle_key_codes_on_near_ties():
    k, nsep = A.key_blocks(32, 128, 4, False, "f32", seed=93)
    assert nsep >= MIN_SEP["f32"]
    q, s, z = oracle.kv_quantize_keys(k, 32, False)
    blk = np.arange(k.shape[0])[:, None] // 32
    ch = np.arange(k.shape[1])[None, :]
    assert _check_against_fractions(k, q, s[blk, ch], z[blk, ch].astype(np.int64), 8, False) >= MIN_SEP["f32"]


def test_special_segments_cover_the_named_cases():
    """Each special segment is what its comment says: exact ties at s = 1, the odd zero point 93 of the
    round-then-add example, a zero range, an underflowing scale, a subnormal scale."""
    segs = A.special_segments(32, 8, False, "f32")
    q, s, z = oracle.quantize(np.stack(segs), 8, False, oracle.ROW)
    assert s[0] == 1.0 and z[0] == 93 and q[0, 2] == 93  # 0.5 -> 0 + 93, not 94
    segs = A.special_segments(32, 4, True, "f32")
    q, s, _ = oracle.quantize(np.stack(segs), 4, True, oracle.ROW)
    assert s[0] == 1.0 and q[0, 1:8].tolist() == [2, 4, -2, 0, 0, 2, -4]
    zero_row = [i for i, g in enumerate(segs) if not g.any()][0]
    assert s[zero_row] == 0.0 and not q[zero_row].any()
    assert s[zero_row + 1] == 0.0 and not q[zero_row + 1].any()  # the smallest subnormal alone: step 0
    assert 0 < s[zero_row + 3] < np.float32(2.0 ** -126)  # a subnormal scale
