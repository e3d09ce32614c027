"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test names the passage or the mathematical fact it checks. None of them re-derives a result by
re-typing the oracle's own formula: they use values printed on the pages, closed forms, invariants,
special cases that reduce to a library routine, exact rational arithmetic or brute force on tiny inputs.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def f32(v):
    return np.asarray(v, dtype=np.float32)


# --------------------------------------------------------------------------- printed worked examples

def test_worked_example_symmetric_int8():
    """Symmetric INT8 worked example ("大模型压缩：从研究到生产的完整攻略（1）", symmetric quantization)."""
    g = gold("worked_example_symmetric_int8.json")
    x = f32([g["x"]])
    q, s, z = oracle.quantize(x, 8, True, oracle.TENSOR)
    assert z is None
    assert abs(float(s[0]) - g["printed_scale_approx"]) < 5e-5
    printed = g["printed_codes"]
    # four of the five printed codes are reproduced exactly, including 127 for the absmax element
    for i in (0, 2, 3, 4):
        assert q[0, i] == printed[i]
    assert q[0].tolist() == g["expected_codes"]
    xhat, _ = oracle.dequantize(q, s, None, oracle.TENSOR)
    for i in (0, 2, 3):
        assert abs(float(xhat[0, i]) - g["printed_dequant"][i]) < 6e-4
    assert abs(float(xhat[0, 4]) - g["printed_dequant"][4]) < 5e-3


def test_worked_example_printed_minus72_is_a_slip():
    """No standard rounding of x/s gives the printed vector, so the printed -72 cannot be the method's."""
    g = gold("worked_example_symmetric_int8.json")
    x = np.array(g["x"], np.float64)
    s = 2.1 / 127.0
    t = x / s
    printed = np.array(g["printed_codes"])
    candidates = {
        "half-even": np.round(t),
        "half-away": np.sign(t) * np.floor(np.abs(t) + 0.5),
        "floor": np.floor(t),
        "ceil": np.ceil(t),
        "trunc": np.trunc(t),
    }
    for name, r in candidates.items():
        assert not np.array_equal(r.astype(int), printed), name
    # the exact real quotient for -1.2 is nowhere near a rounding tie
    assert abs(t[1] - (-72.5)) > 0.05


def test_outlier_example():
    """Outlier example: one value of 100 sets s ~ 0.79 and squeezes [-2, 2] into codes [-3, 3]."""
    g = gold("outlier_example.json")
    normal_vals = np.linspace(-2.0, 2.0, 401, dtype=np.float32)
    x = np.concatenate([normal_vals, f32([g["outlier"]])])[None, :]
    q, s, _ = oracle.quantize(x, 8, True, oracle.TENSOR)
    assert abs(float(s[0]) - g["printed_scale_approx"]) < 0.005
    assert q[0, -1] == 127
    lo, hi = g["printed_normal_code_range"]
    assert q[0, :-1].min() == lo and q[0, :-1].max() == hi


def test_int4_group_bookkeeping_llama7b():
    """§11.1.6 of "第11章 模型量化与压缩": 4096x4096, g=128 -> 32 groups per row, 131,072 groups, codes in [-7, 7],
    s = group absmax / 7 (checked with numpy's max on a few groups)."""
    g = gold("int4_group_example.json")
    n, k = g["shape"]
    w = workloads.attn7b(ms=(1,))["w"]
    q, s, z = oracle.quantize(w, 4, True, oracle.GROUP, g["group_size"])
    assert s.size == g["groups_total"] == n * k // g["group_size"]
    assert s.reshape(n, -1).shape[1] == g["groups_per_row"]
    assert q.min() >= g["code_range"][0] and q.max() <= g["code_range"][1]
    wf = workloads.bf16_to_f32(w)
    for row, grp in [(0, 0), (17, 31), (4095, 5)]:
        seg = wf[row, grp * 128:(grp + 1) * 128]
        assert s[row * 32 + grp] == np.float32(np.abs(seg).max()) / np.float32(7)
        assert np.abs(q[row, grp * 128:(grp + 1) * 128]).max() == 7


def test_metadata_overhead_accounting():
    """§1.1 of "量化、蒸馏与模型压缩" and §11.3.7 of "第11章 模型量化与压缩": metadata share for g=128 and g=32
    under 16-bit scales; the count of extra parameters is d_out*d_in/g."""
    g = gold("metadata_overhead.json")
    for gs in (128, 32):
        share = 16.0 / (4.0 * gs)
        lo, hi = g["ranges"][str(gs)]
        assert lo <= share <= hi
        assert abs(share - g["approx"][str(gs)]) < 0.006
        assert oracle.n_segments(11008, 4096, oracle.GROUP, gs) == 11008 * 4096 // gs


# --------------------------------------------------------------------------- rounding and division

def test_round_half_to_even_at_exact_ties():
    """A group with absmax 7 has s = 1 exactly, so x/s is exact and the ties are real ties."""
    x = f32([[7.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -3.5] + [0.0] * 24])
    q, s, _ = oracle.quantize(x, 4, True, oracle.GROUP, 32)
    assert s[0] == 1.0
    assert q[0, :8].tolist() == [7, 2, 4, -2, 0, 0, 2, -4]


def test_hand_computed_group():
    """absmax 3.5 -> s = 0.5 (exact); -3.5/0.5 = -7 ... and -1.75/0.5 = -3.5 ties to -4."""
    x = f32([[3.5, -1.75, 0.5, 0.0, -3.5, 1.25, 0.75, 0.2] + [0.0] * 24])
    q, s, _ = oracle.quantize(x, 4, True, oracle.GROUP, 32)
    assert s[0] == 0.5
    assert q[0, :8].tolist() == [7, -4, 1, 0, -7, 2, 2, 0]


def test_asymmetric_round_then_add_zero_point():
    """The core formula rounds x/s and then adds z. With s = 1 and z = 93, x = 0.5 gives 93; rounding
    x/s + z as one number (the blog's variant) would give 94. Pins the order of the two operations."""
    x = f32([[-93.0, 162.0, 0.5, 0.0, 1.5]])
    q, s, z = oracle.quantize(x, 8, False, oracle.ROW)
    assert s[0] == 1.0 and z[0] == 93
    assert q[0].tolist() == [0, 255, 93, 93, 95]


def _exact_f32_quotient(x, s):
    """Correctly rounded binary32 quotient via exact rationals (nearest, ties to even)."""
    r = Fraction(float(x)) / Fraction(float(s))
    lo = np.float32(float(r))  # float(r) is the correctly rounded binary64; refine to binary32 below
    cands = sorted({lo, np.nextafter(lo, np.float32(np.inf)), np.nextafter(lo, np.float32(-np.inf))},
                   key=lambda c: (abs(Fraction(float(c)) - r), int(np.float32(c).view(np.uint32)) & 1))
    return cands[0]


def test_division_not_reciprocal_multiply():
    """The code of x is taken from the correctly rounded quotient x/s. Find a value where x*(1/s) rounds
    across a half-integer while x/s does not, and check the oracle follows exact division."""
    s = np.float32(0.3)  # the group absmax is 7*s' below; pick s from a group directly
    rng = np.random.default_rng(7)
    found = None
    for _ in range(200000):
        a = np.float32(rng.uniform(0.5, 7.0))
        s = a / np.float32(7)
        h = np.float32(rng.integers(-6, 6)) + np.float32(0.5)
        xv = np.float32(h * s)
        for cand in (xv, np.nextafter(xv, np.float32(9)), np.nextafter(xv, np.float32(-9))):
            qd = np.rint(_exact_f32_quotient(cand, s))
            qr = np.rint(np.float32(cand * (np.float32(1) / s)))
            if qd != qr and abs(cand) < a:
                found = (a, cand, int(qd))
                break
        if found:
            break
    assert found is not None
    a, xv, qd = found
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = a
    x[0, 1] = xv
    q, s_out, _ = oracle.quantize(x, 4, True, oracle.GROUP, 32)
    assert s_out[0] == np.float32(a) / np.float32(7)
    assert q[0, 1] == qd


# --------------------------------------------------------------------------- error bound and zero point

@pytest.mark.parametrize("bits,sym,gran,gs", [
    (4, True, oracle.GROUP, 128), (4, True, oracle.GROUP, 32), (4, False, oracle.GROUP, 64),
    (8, True, oracle.ROW, 0), (8, False, oracle.ROW, 0), (8, True, oracle.TENSOR, 0),
    (4, False, oracle.TENSOR, 0), (8, False, oracle.GROUP, 128)])
def test_error_bound_half_step(bits, sym, gran, gs):
    """|x - x_hat| <= s/2 for every element that is not clipped ("量化、蒸馏与模型压缩", error bound under
    nearest rounding), up to the rounding of the fp32 quotient: s/2 + |x| 2^-24, in exact arithmetic."""
    rng = np.random.default_rng(bits * 100 + gs + int(sym))
    x = (rng.standard_normal((16, 256)) * rng.uniform(0.01, 3.0, size=(16, 1))).astype(np.float32)
    x[3, :64] += 2.0  # a shifted block (all positive) for the asymmetric cases
    q, s, z = oracle.quantize(x, bits, sym, gran, gs)
    seg = np.zeros(x.shape, np.int64)
    if gran == oracle.ROW:
        seg = np.repeat(np.arange(16), 256).reshape(16, 256)
    elif gran == oracle.GROUP:
        seg = np.arange(x.size).reshape(x.shape) // gs
    ss = s[seg].astype(np.float64)
    zz = 0 if z is None else z[seg].astype(np.int64)
    xhat = ss * (q - zz)  # exact in binary64 (24-bit scale times a small integer)
    err = np.abs(x.astype(np.float64) - xhat)
    bound = ss / 2 + np.abs(x) * 2.0 ** -24
    qmin, qmax = (-(2 ** (bits - 1) - 1), 2 ** (bits - 1) - 1) if sym else (0, 2 ** bits - 1)
    inside = (q > qmin) & (q < qmax)
    assert np.all(err[inside] <= bound[inside])
    # ends of the range: still within the bound except for (rare) clipping
    frac_bad = np.mean(err > bound)
    assert frac_bad < 1e-3
    assert q.min() >= qmin and q.max() <= qmax


def test_asymmetric_zero_is_exact():
    """With a zero point a real 0 maps to q = z and back to exactly 0 (blog, asymmetric quantization)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 256)).astype(np.float32) + 0.3
    x[:, ::7] = 0.0
    for bits, gran, gs in [(4, oracle.GROUP, 32), (4, oracle.GROUP, 128), (8, oracle.ROW, 0)]:
        q, s, z = oracle.quantize(x, bits, False, gran, gs)
        xhat, xhat16 = oracle.dequantize(q, s, z, gran, gs)
        assert np.all(xhat[x == 0] == 0.0)
        assert np.all(xhat16[x == 0] == 0)


def test_asymmetric_range_ends_and_all_positive_group():
    """min -> 0 and max -> 2^b - 1; a group with only positive values has lo widened to 0, so z = 0."""
    x = f32([[-1.0, 2.0, 0.25, 1.0] + [0.5] * 28, [0.5, 1.5, 3.0, 0.75] + [1.0] * 28])
    q, s, z = oracle.quantize(x, 4, False, oracle.GROUP, 32)
    assert s[0] == np.float32(3.0) / np.float32(15) and z[0] == 5
    assert q[0, 0] == 0 and q[0, 1] == 15
    assert s[1] == np.float32(3.0) / np.float32(15) and z[1] == 0
    assert q[1, 2] == 15


def test_zero_range_and_underflowing_groups():
    """An all-zero group, and a group whose fp32 scale underflows to 0, store s = 0 (and z = 0); their codes
    are all 0, so s (q - z) is exactly 0."""
    tiny = np.float32(1.4e-45)  # smallest positive subnormal
    x = np.zeros((3, 32), np.float32)
    x[1, 5] = tiny
    x[2, 5] = np.float32(1e-40)  # subnormal but large enough for a nonzero subnormal scale
    for sym in (True, False):
        q, s, z = oracle.quantize(x, 4, sym, oracle.GROUP, 32)
        assert s.view(np.uint32)[0] == 0 and s.view(np.uint32)[1] == 0  # +0, not -0
        assert np.all(q[0] == (0 if sym else 0)) and np.all(q[1] == 0)
        assert 0 < s[2] < 1e-40
        assert (q[2, 5] == 7) if sym else (q[2, 5] == 15)
        if not sym:
            assert z[0] == 0 and z[1] == 0


# --------------------------------------------------------------------------- granularity special cases

def test_granularity_reductions():
    """GROUP with g = cols is ROW; ROW of a one-row tensor is TENSOR; TENSOR of a one-group tensor is GROUP."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    for sym in (True, False):
        a = oracle.quantize(x, 4, sym, oracle.GROUP, 128)
        b = oracle.quantize(x, 4, sym, oracle.ROW)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        r1 = oracle.quantize(x[2:3], 8, sym, oracle.ROW)
        t1 = oracle.quantize(x[2:3], 8, sym, oracle.TENSOR)
        assert np.array_equal(r1[0], t1[0]) and np.array_equal(r1[1], t1[1])
        g1 = oracle.quantize(x[4:5, :32], 8, sym, oracle.GROUP, 32)
        t2 = oracle.quantize(x[4:5, :32], 8, sym, oracle.TENSOR)
        assert np.array_equal(g1[0], t2[0]) and np.array_equal(g1[1], t2[1])


def test_group_segments_are_independent():
    """Changing one group's values changes only that group's scale and codes (no index bleed)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    q0, s0, _ = oracle.quantize(x, 4, True, oracle.GROUP, 64)
    x2 = x.copy()
    x2[2, 100] = 9.0  # a new absmax inside group 1 of row 2
    q1, s1, _ = oracle.quantize(x2, 4, True, oracle.GROUP, 64)
    changed = np.nonzero(s0 != s1)[0].tolist()
    assert changed == [2 * 4 + 1]
    diff_rows, diff_cols = np.nonzero(q0 != q1)
    assert diff_rows.size > 0
    assert set(diff_rows.tolist()) <= {2} and diff_cols.min() >= 64 and diff_cols.max() < 128


# --------------------------------------------------------------------------- packing and dequantization

def test_pack_nibble_order():
    q = np.zeros((1, 8), np.int32)
    cases = [((0, 1), 0x01, 0), ((1, 1), 0x10, 0), ((0, -1), 0x0F, 0), ((1, -7), 0x90, 0), ((2, 7), 0x07, 1),
             ((3, -8), 0x80, 1)]
    for (pos, val), byte, idx in cases:
        qq = q.copy()
        qq[0, pos] = val
        p = oracle.pack_int4(qq)
        assert p[0, idx] == byte, (pos, val)
        assert np.count_nonzero(p) == 1


def test_pack_roundtrip():
    rng = np.random.default_rng(2)
    qs = rng.integers(-7, 8, size=(5, 64)).astype(np.int32)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(qs), 64, True), qs)
    qu = rng.integers(0, 16, size=(5, 64)).astype(np.int32)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(qu), 64, False), qu)


def test_dequantize_values_and_bf16_rounding():
    q = np.array([[-4, 3, 0, 7]], np.int32)
    s = f32([0.5])
    out, out16 = oracle.dequantize(q, s, None, oracle.TENSOR)
    assert out[0].tolist() == [-2.0, 1.5, 0.0, 3.5]
    # bf16 rounding, nearest-even: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> 1; 1 + 3*2^-8 -> 1 + 2^-6
    t = oracle.f32_to_bf16(f32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -1.0 - 2 ** -8]))
    assert t.tolist() == [0x3F80, 0x3F82, 0x3F81, 0xBF80]
    qa = np.array([[0, 15, 5, 6]], np.int32)
    out, _ = oracle.dequantize(qa, f32([0.25]), np.array([5], np.uint8), oracle.ROW)
    assert out[0].tolist() == [-1.25, 2.5, 0.0, 0.25]


# --------------------------------------------------------------------------- W4A16 reference

def test_w4a16_unit_scales_is_integer_matvec():
    """With s = 1 and z = 0 the layer is an integer matrix times a bf16 vector: numpy float64 matmul."""
    rng = np.random.default_rng(9)
    q = rng.integers(-7, 8, size=(48, 256)).astype(np.int32)
    x = workloads.bf16_bits(rng.standard_normal((3, 256)).astype(np.float32))
    s = np.ones(48 * 2, np.float32)
    y = oracle.w4a16(x, q, s, None, 128)
    ref = workloads.bf16_to_f32(x).astype(np.float64) @ q.T.astype(np.float64)
    assert np.allclose(y, ref, rtol=0, atol=1e-9)


def test_w4a16_brute_force_exact():
    """Tiny asymmetric case against exact rational arithmetic."""
    rng = np.random.default_rng(4)
    N, K, gsz = 3, 64, 32
    q = rng.integers(0, 16, size=(N, K)).astype(np.int32)
    s = rng.uniform(0.01, 0.2, size=N * K // gsz).astype(np.float32)
    z = rng.integers(0, 16, size=N * K // gsz).astype(np.uint8)
    x = workloads.bf16_bits(rng.standard_normal((2, K)).astype(np.float32))
    xf = workloads.bf16_to_f32(x)
    y = oracle.w4a16(x, q, s, z, gsz)
    for m in range(2):
        for n in range(N):
            exact = sum(Fraction(float(xf[m, k])) * Fraction(float(s[n * 2 + k // gsz])) *
                        (int(q[n, k]) - int(z[n * 2 + k // gsz])) for k in range(K))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 60)


# --------------------------------------------------------------------------- SmoothQuant factor

def test_smooth_alpha_special_cases():
    """§11.4.3 of "第11章 模型量化与压缩": alpha = 1 -> s_j = max|X_j|; alpha = 0 -> s_j = 1/max|W_j|."""
    d = workloads.w8a8(m=64, n=96, k=256)
    xf = workloads.bf16_to_f32(d["x"])
    wf = workloads.bf16_to_f32(d["w"])
    s1 = oracle.smooth(d["x"], d["w"], 1.0)
    assert np.array_equal(s1, np.abs(xf).max(axis=0))
    s0 = oracle.smooth(d["x"], d["w"], 0.0)
    assert np.array_equal(s0, np.float32(1) / np.abs(wf).max(axis=0))


def test_smooth_alpha_half_balances_columns():
    """alpha = 0.5 is the balance point ("量化、蒸馏与模型压缩" §2.3 eq. (2)): after smoothing, max|X'_j| equals
    max|W'_j| (here within a few ulps, from fp32 rounding)."""
    d = workloads.w8a8(m=64, n=96, k=256)
    xf = workloads.bf16_to_f32(d["x"]).astype(np.float64)
    wf = workloads.bf16_to_f32(d["w"]).astype(np.float64)
    s = oracle.smooth(d["x"], d["w"], 0.5).astype(np.float64)
    ax = np.abs(xf / s).max(axis=0)
    aw = np.abs(wf * s).max(axis=0)
    assert np.all(np.abs(ax - aw) <= 4 * 2.0 ** -23 * ax)
    # generic alpha agrees with the closed form to ~1 ulp
    s3 = oracle.smooth(d["x"], d["w"], 0.3).astype(np.float64)
    ref = np.abs(xf).max(axis=0) ** 0.3 / np.abs(wf).max(axis=0) ** 0.7
    assert np.all(np.abs(s3 - ref) <= 2.0 ** -23 * ref)


def test_smooth_zero_channel_and_equivalence():
    """A zero channel gets s_j = 1; and X diag(s)^-1 . diag(s) W^T equals X W^T (§11.4.2 identity)."""
    d = workloads.w8a8(m=32, n=48, k=128)
    x = d["x"].copy()
    x[:, 7] = 0
    s = oracle.smooth(x, d["w"], 0.5)
    assert s[7] == 1.0
    xf = workloads.bf16_to_f32(x).astype(np.float64)
    wf = workloads.bf16_to_f32(d["w"]).astype(np.float64)
    sd = s.astype(np.float64)
    assert np.allclose((xf / sd) @ (wf * sd).T, xf @ wf.T, rtol=1e-12, atol=1e-12)


def test_outliers_starve_per_tensor_int8():
    """"量化、蒸馏与模型压缩" §2.3: per-tensor INT8 on activations with outlier channels leaves the ordinary
    channels only a few levels (2-3 bits). With x50 outlier channels they stay within |q| <= 7 here."""
    d = workloads.w8a8(m=256, n=16, k=4096)
    q, s, _ = oracle.quantize(d["x"], 8, True, oracle.TENSOR)
    normal_cols = np.setdiff1d(np.arange(4096), d["outlier_chans"])
    lvl = np.abs(q[:, normal_cols])
    assert np.quantile(lvl, 0.999) <= 4 and lvl.max() <= 7
    assert np.abs(q).max() == 127


# --------------------------------------------------------------------------- INT8 GEMM and epilogue

def test_gemm_brute_force_extremes():
    a = np.array([[127, -127, 0, 5, -1], [1, 2, 3, 4, 5], [-127, -127, -127, -127, -127]], np.int8)
    b = np.array([[127, 127, 127, 127, 127], [-127, 127, -127, 127, -127], [0, 0, 1, 0, 0],
                  [1, -1, 1, -1, 1], [3, 1, 4, 1, 5], [-2, 7, -1, 8, -2], [127, -127, 127, -127, 127]], np.int8)
    c = oracle.gemm_s8(a, b)
    for i in range(3):
        for j in range(7):
            assert c[i, j] == sum(int(a[i, k]) * int(b[j, k]) for k in range(5))


def test_gemm_matches_numpy_int64():
    rng = np.random.default_rng(1)
    a = rng.integers(-127, 128, size=(37, 300)).astype(np.int8)
    b = rng.integers(-127, 128, size=(53, 300)).astype(np.int8)
    assert np.array_equal(oracle.gemm_s8(a, b), a.astype(np.int64) @ b.astype(np.int64).T)


def test_gemm_int32_bound():
    """K * 127^2 stays inside int32 for K = 4096 (66,064,384 < 2^31)."""
    a = np.full((1, 4096), 127, np.int8)
    c = oracle.gemm_s8(a, a)
    assert c[0, 0] == 4096 * 127 * 127 < 2 ** 31


def test_w8a8_epilogue_and_pipeline():
    d = workloads.w8a8(m=16, n=24, k=256)
    r = oracle.w8a8(d["x"], d["w"], 0.5)
    ref = r["acc"].astype(np.float64) * r["s_x"].astype(np.float64)[:, None] * r["s_w"].astype(np.float64)[None, :]
    assert np.array_equal(r["y"], ref)
    # the quantized layer approximates the float product X W^T
    xf = workloads.bf16_to_f32(d["x"]).astype(np.float64)
    wf = workloads.bf16_to_f32(d["w"]).astype(np.float64)
    y_true = xf @ wf.T
    assert np.linalg.norm(r["y"] - y_true) / np.linalg.norm(y_true) < 0.05
    assert np.abs(r["q_x"]).max() <= 127 and np.abs(r["q_w"]).max() <= 127


# --------------------------------------------------------------------------- static per-tensor path

def test_static_worked_example():
    """Static per-tensor INT8 with the worked example's own scale 2.1 / 127 ("大模型压缩：从研究到生产的完整
    攻略（1）", symmetric example; "第11章 模型量化与压缩" §11.1.4 static parameters): the printed codes of elements
    0, 2, 3, 4 and the recorded reading for element 1."""
    g = gold("worked_example_symmetric_int8.json")
    x = f32([g["x"]])
    s = np.float32(2.1) / np.float32(127)
    q = oracle.quantize_static(x, 8, True, s)
    for i in (0, 2, 3, 4):
        assert q[0, i] == g["printed_codes"][i]
    assert q[0].tolist() == g["expected_codes"]


def test_static_clips_outside_calibrated_range():
    """Values beyond the calibrated range clip to the ends of the code range (§11.1.4: static parameters
    are fixed, so out-of-distribution inputs saturate): INT8 symmetric at scale 1/127 maps [-1, 1] onto
    [-127, 127]; 1.5, 1e30 and -3 saturate, 0.5 is 63.5 -> 64 (tie to even), -0.25 is -31.75 -> -32."""
    x = f32([[1.5, 1e30, -3.0, 0.5, -0.25, 1.0, -1.0, 0.0]])
    q = oracle.quantize_static(x, 8, True, np.float32(1.0) / np.float32(127))
    assert q[0].tolist() == [127, 127, -127, 64, -32, 127, -127, 0]
    # INT4 asymmetric, zero 8, scale 0.5: [-4, 3.5] -> [0, 15]
    x4 = f32([[-4.0, -4.5, 3.5, 100.0, 0.0, 0.25, 0.75, -1.0]])
    q4 = oracle.quantize_static(x4, 4, False, np.float32(0.5), zero=8)
    assert q4[0].tolist() == [0, 0, 15, 15, 8, 8, 10, 6]


def test_static_asymmetric_exact_rational():
    """Brute force in exact rational arithmetic: q = clamp(rne(x / s) + z) for random x, s, z (ties in the
    binary32 quotient are skipped: there the exact and the rounded quotient may legitimately differ)."""
    rng = np.random.default_rng(7)
    for trial in range(20):
        bits = 4 if trial % 2 else 8
        qmax = (1 << bits) - 1
        z = int(rng.integers(0, qmax + 1))
        s = np.float32(rng.uniform(0.01, 0.3))
        x = (rng.standard_normal((1, 64)) * 5).astype(np.float32)
        q = oracle.quantize_static(x, bits, False, s, zero=z)
        for j in range(64):
            t = Fraction(float(x[0, j])) / Fraction(float(s))
            fl = t - (t.numerator // t.denominator)
            if abs(fl - Fraction(1, 2)) < Fraction(1, 1 << 18):
                continue
            r = round(t)  # Python rounds Fractions half to even
            assert q[0, j] == min(max(r + z, 0), qmax)


def test_static_matches_dynamic_when_given_its_scale():
    """With the scale the dynamic per-tensor path measures (pinned above), the static codes are the dynamic
    ones: the two paths share the code step and differ only in where (s, z) come from."""
    d = workloads.w8a8(m=32, n=16, k=256)
    for bits, sym in ((8, True), (8, False), (4, True), (4, False)):
        q, s, z = oracle.quantize(d["x"], bits, sym, oracle.TENSOR)
        qs = oracle.quantize_static(d["x"], bits, sym, s[0], zero=0 if sym else int(z[0]))
        assert np.array_equal(q, qs), (bits, sym)


def test_fold_smoothing_exact_cases():
    """X diag(s)^-1 in bf16 ("第11章 模型量化与压缩" §11.4.4, the factor folded into LayerNorm): s = 1 returns X
    bit for bit, and powers of two only move the exponent (exact, no rounding, away from the subnormals)."""
    d = workloads.w8a8(m=8, n=8, k=128)
    x = d["x"]
    assert np.array_equal(oracle.fold_smoothing_bf16(x, np.ones(128, np.float32)), x)
    s = np.where(np.arange(128) % 2 == 0, 4.0, 0.125).astype(np.float32)
    xp = workloads.bf16_to_f32(oracle.fold_smoothing_bf16(x, s)).astype(np.float64)
    assert np.array_equal(xp, workloads.bf16_to_f32(x).astype(np.float64) / s.astype(np.float64))


def test_w8a8_static_pipeline():
    """The pages' pipeline (§11.4.5 steps 1-6) with a static per-tensor activation scale: the scale is the
    calibration batch's max |X'| / 127; the epilogue is acc * s_x * s_w; the result approximates X W^T; and
    when the inference batch is the calibration batch the codes equal the dynamic per-tensor ones."""
    d = workloads.w8a8(m=64, n=24, k=256)
    xc = workloads.w8a8_calibration(m=128, k=256)
    r = oracle.w8a8_static(xc, d["x"], d["w"], 0.5)
    xcp = workloads.bf16_to_f32(oracle.fold_smoothing_bf16(xc, r["s"]))
    assert r["s_x"] == np.float32(np.abs(xcp).max()) / np.float32(127)
    ref = r["acc"].astype(np.float64) * np.float64(r["s_x"]) * r["s_w"].astype(np.float64)[None, :]
    assert np.array_equal(r["y"], ref)
    xf = workloads.bf16_to_f32(d["x"]).astype(np.float64)
    wf = workloads.bf16_to_f32(d["w"]).astype(np.float64)
    y_true = xf @ wf.T
    assert np.linalg.norm(r["y"] - y_true) / np.linalg.norm(y_true) < 0.05
    same = oracle.w8a8_static(d["x"], d["x"], d["w"], 0.5)
    qd, _, _ = oracle.quantize(same["x_prime"], 8, True, oracle.TENSOR)
    assert np.array_equal(same["q_x"], qd.astype(np.int8))


# --------------------------------------------------------------------------- W4A8

def test_w4a8_one_group_is_w8a8():
    """With one group spanning K and no zero point, W4A8 is the W8A8 product with a per-channel weight scale
    ("第11章 模型量化与压缩" §11.4.5): the pinned integer GEMM and epilogue."""
    rng = np.random.default_rng(11)
    qx = rng.integers(-127, 128, size=(9, 256)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(13, 256)).astype(np.int32)
    sx = rng.uniform(0.001, 0.1, 9).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, 13).astype(np.float32)
    y = oracle.w4a8(qx, sx, qw, sw, None, 256)
    ref = oracle.w8a8_epilogue(oracle.gemm_s8(qx, qw.astype(np.int8)), sx, sw)
    assert np.allclose(y, ref, rtol=1e-15, atol=0)


def test_w4a8_unit_scales_is_integer_product():
    """All scales 1: the result is the exact integer product of q_x and (q_w - z) with z per group."""
    rng = np.random.default_rng(12)
    for g in (32, 64, 128):
        qx = rng.integers(-127, 128, size=(5, 384)).astype(np.int8)
        qw = rng.integers(0, 16, size=(7, 384)).astype(np.int32)
        z = rng.integers(0, 16, size=(7, 384 // g)).astype(np.uint8)
        y = oracle.w4a8(qx, np.ones(5, np.float32), qw, np.ones(7 * 384 // g, np.float32), z.ravel(), g)
        wz = qw.astype(np.int64) - np.repeat(z.astype(np.int64), g, axis=1)
        assert np.array_equal(y, (qx.astype(np.int64) @ wz.T).astype(np.float64))


def test_w4a8_brute_force_rational():
    """Tiny inputs against exact rational arithmetic (the binary64 result within 1e-12 relative)."""
    rng = np.random.default_rng(13)
    qx = rng.integers(-127, 128, size=(3, 96)).astype(np.int8)
    qw = rng.integers(0, 16, size=(4, 96)).astype(np.int32)
    z = rng.integers(0, 16, size=(4, 3)).astype(np.uint8)
    sx = rng.uniform(0.01, 1, 3).astype(np.float32)
    sw = rng.uniform(0.01, 1, 12).astype(np.float32)
    y = oracle.w4a8(qx, sx, qw, sw, z.ravel(), 32)
    for m in range(3):
        for n in range(4):
            t = Fraction(0)
            for gi in range(3):
                acc = sum(int(qx[m, k]) * (int(qw[n, k]) - int(z[n, gi])) for k in range(32 * gi, 32 * gi + 32))
                t += Fraction(float(sw[n * 3 + gi])) * acc
            exact = Fraction(float(sx[m])) * t
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 10 ** 12)


def test_w4a8_pipeline_approximates_float_product():
    """INT4 group weights (g = 128) with SmoothQuant INT8 activations approximate X W^T (coarser than W8A8:
    INT4 weights)."""
    d = workloads.w8a8(m=32, n=48, k=512)
    xf = workloads.bf16_to_f32(d["x"]).astype(np.float64)
    wf = workloads.bf16_to_f32(d["w"]).astype(np.float64)
    y_true = xf @ wf.T
    for sym in (True, False):
        r = oracle.w4a8_pipeline(d["x"], d["w"], 0.5, 128, sym)
        assert np.linalg.norm(r["y"] - y_true) / np.linalg.norm(y_true) < 0.2


# ---------------------------------------------------------------- KV cache (P3 §11.6)


@pytest.mark.parametrize("sym", [True, False])
def test_kv_keys_are_row_quantization_of_each_block_transposed(sym):
    """Per-channel over a block of T tokens is per-row quantization of the block's transpose (the pinned
    per-row quantizer), block by block: codes, scales and zeros identical."""
    d = workloads.kv_cache(96, 64, outlier_channels=4)
    q, s, z = oracle.kv_quantize_keys(d["k"], 32, sym)
    for b in range(3):
        blk = np.ascontiguousarray(d["k"][32 * b:32 * b + 32].T)
        qr, sr, zr = oracle.quantize(blk, 8, sym, oracle.ROW)
        assert np.array_equal(q[32 * b:32 * b + 32], qr.T)
        assert np.array_equal(s[b].view(np.uint32), sr.view(np.uint32))
        if not sym:
            assert np.array_equal(z[b], zr)


def test_kv_keys_channels_are_independent():
    """Scaling one channel by a power of two scales its block scales by the same power and leaves its codes
    and every other channel unchanged: an outlier channel does not widen the others' steps."""
    d = workloads.kv_cache(64, 32, outlier_channels=0)
    k = workloads.bf16_to_f32(d["k"])
    k2 = k.copy()
    k2[:, 5] *= np.float32(64.0)
    q1, s1, _ = oracle.kv_quantize_keys(k, 32, True)
    q2, s2, _ = oracle.kv_quantize_keys(k2, 32, True)
    assert np.array_equal(q1, q2)
    others = [c for c in range(32) if c != 5]
    assert np.array_equal(s1[:, others], s2[:, others])
    assert np.array_equal(s2[:, 5], s1[:, 5] * np.float32(64.0))


def test_kv_keys_range_and_error_bound():
    """Symmetric: each (block, channel)'s absolute maximum codes to +-127, every code lies in [-127, 127], and
    dequantization is within s/2 of the input (no clipping). Asymmetric: codes span [0, 255] per segment with
    the error bound on unclamped elements [P1 core formula; P3 §11.1.1]."""
    d = workloads.kv_cache(128, 48, outlier_channels=3)
    k = workloads.bf16_to_f32(d["k"])
    q, s, _ = oracle.kv_quantize_keys(d["k"], 64, True)
    assert q.min() >= -127 and q.max() <= 127
    for b in range(2):
        blk = q[64 * b:64 * b + 64]
        assert np.array_equal(np.abs(blk).max(axis=0), np.full(48, 127))
    xh, _ = oracle.kv_dequantize_keys(q, s, None, 64)
    bound = np.repeat(s, 64, axis=0).astype(np.float64) / 2
    slack = np.abs(k).astype(np.float64) * 2.0 ** -22  # fp32 rounding of x / s and of s q
    assert np.all(np.abs(xh.astype(np.float64) - k) <= bound + slack)
    qa, sa, za = oracle.kv_quantize_keys(d["k"], 64, False)
    assert qa.min() >= 0 and qa.max() <= 255
    xa, _ = oracle.kv_dequantize_keys(qa, sa, za, 64)
    inner = (qa > 0) & (qa < 255)
    ba = np.repeat(sa, 64, axis=0).astype(np.float64) / 2
    assert np.all((np.abs(xa.astype(np.float64) - k) <= ba + slack + ba * 2.0 ** -20)[inner])


def _empty_cache(B, S, C, T, nv, sym):
    c = {"k_res": np.zeros((B, T, C), np.uint16), "k_q": np.zeros((B, S, C), np.int32),
         "k_s": np.zeros((B, S // T, C), np.float32), "v_q": np.zeros((B, S, C), np.int32),
         "v_s": np.zeros((B, S, nv), np.float32)}
    if not sym:
        c["k_z"] = np.zeros((B, S // T, C), np.uint8)
        c["v_z"] = np.zeros((B, S, nv), np.uint8)
    return c


@pytest.mark.parametrize("sym,vg", [(True, 0), (False, 32)])
def test_kv_append_online_equals_bulk(sym, vg):
    """Appending tokens one step at a time [P3 §11.6.2, §11.6.5] gives the cache that bulk quantization of the
    same tokens gives: complete key groups per channel, values per token (or group); the incomplete group's
    keys wait at full precision in the residual slots; positions outside the cache are skipped."""
    B, S, C, T = 3, 96, 64, 32
    d = workloads.kv_cache(B * S, C, outlier_channels=4)
    ks, vs = d["k"].reshape(B, S, C), d["v"].reshape(B, S, C)
    n_tok = [S, 70, 33]  # tokens each sequence ends with
    nv = C // vg if vg else 1
    cache = _empty_cache(B, S, C, T, nv, sym)
    for step in range(S + 2):
        pos = np.array([step if step < n_tok[b] else (S + 5 if b == 0 else -1) for b in range(B)])
        kn = np.stack([ks[b, min(step, S - 1)] for b in range(B)])
        vn = np.stack([vs[b, min(step, S - 1)] for b in range(B)])
        oracle.kv_append(cache, kn, vn, pos, T, vg, sym)
    for b in range(B):
        n = n_tok[b]
        full = n // T * T
        if full:
            q, s, z = oracle.kv_quantize_keys(ks[b, :full], T, sym)
            assert np.array_equal(cache["k_q"][b, :full], q)
            assert np.array_equal(cache["k_s"][b, :full // T], s)
            if not sym:
                assert np.array_equal(cache["k_z"][b, :full // T], z)
        assert not cache["k_q"][b, full:].any()
        assert np.array_equal(cache["k_res"][b, :n - full], ks[b, full:n])
        gran = oracle.GROUP if vg else oracle.ROW
        qv, sv, zv = oracle.quantize(vs[b, :n], 8, sym, gran, vg)
        assert np.array_equal(cache["v_q"][b, :n], qv)
        assert np.array_equal(cache["v_s"][b, :n].ravel(), sv)
        if not sym:
            assert np.array_equal(cache["v_z"][b, :n].ravel(), zv)
        assert not cache["v_q"][b, n:].any()


# ---------------------------------------------------------------- 16-bit metadata (P1 §1.1; P3 §11.3.7)


def test_f16_conversion_matches_numpy():
    """The oracle's binary32 -> binary16 rounding (nearest even, subnormals, overflow) agrees with numpy's cast,
    and binary16 -> binary32 is exact, over normal, subnormal, tie and overflow inputs."""
    rng = np.random.default_rng(30)
    v = np.concatenate([
        (rng.standard_normal(4000) * np.exp2(rng.integers(-30, 17, 4000))).astype(np.float32),
        np.float32([2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -24, 65504.0, 65519.99, 65520.0, 1 + 2.0 ** -11,
                    1 + 3 * 2.0 ** -11, 6.1e-5, 0.0])])
    with np.errstate(over="ignore"):
        ref = np.abs(v).astype(np.float16).view(np.uint16)
    mine = np.array([oracle.f32_to_f16(abs(float(x))) for x in v], np.uint16)
    assert np.array_equal(mine, ref)
    h = np.arange(0, 0x7C00, 7, dtype=np.uint16)
    assert np.array_equal(oracle.f16_to_f32(h), h.view(np.float16).astype(np.float32))


@pytest.mark.parametrize("sym", [True, False])
def test_meta16_scale_is_the_rounded_fp32_scale(sym):
    """The stored scale is the binary16 rounding of the pinned fp32 group scale; a scale that rounds to 0
    is stored as the smallest subnormal."""
    d = workloads.ffn7b(ms=(1,))
    w = d["w"][:64, :512]
    _, s32, _ = oracle.quantize(w, 4, sym, oracle.GROUP, 128)
    _, s16, _ = oracle.quantize_meta16(w, sym, 128)
    assert np.array_equal(s16, s32.astype(np.float16).view(np.uint16))
    tiny = np.full((1, 32), 1e-9, np.float32)
    _, st, _ = oracle.quantize_meta16(tiny, True, 32)
    assert st[0] == 0x0001
    q0, s0, _ = oracle.quantize_meta16(np.zeros((1, 32), np.float32), sym, 32)  # a zero range stores 0
    assert s0[0] == 0 and not q0.any()


@pytest.mark.parametrize("sym", [True, False])
def test_meta16_codes_equal_fp32_path_when_the_scale_is_exact(sym):
    """Groups whose fp32 scale is exact in binary16 get the codes (and zero points) of the pinned fp32 path."""
    rng = np.random.default_rng(31)
    x = rng.uniform(-0.8, 0.8, (16, 256)).astype(np.float32)
    x.reshape(-1, 32)[:, 0] = 7 * 2.0 ** -3 if sym else -1.5  # symmetric: s = 2^-3 exactly
    x.reshape(-1, 32)[:, 1] = -7 * 2.0 ** -3 if sym else 2.25  # asymmetric: s = (2.25 + 1.5) / 15 = 0.25
    q32, s32, z32 = oracle.quantize(x, 4, sym, oracle.GROUP, 32)
    q16, s16, z16 = oracle.quantize_meta16(x, sym, 32)
    assert np.array_equal(oracle.f16_to_f32(s16), s32)
    assert np.array_equal(q16, q32)
    if not sym:
        assert np.array_equal(z16, z32)


@pytest.mark.parametrize("sym", [True, False])
def test_meta16_error_bound(sym):
    """s16 (q - z) is within s16 / 2 of every unclamped input [P1 core formula]."""
    d = workloads.ffn7b(ms=(1,))
    w = workloads.bf16_to_f32(d["w"][:32, :1024])
    q, s16, z = oracle.quantize_meta16(w, sym, 64)
    s = np.repeat(oracle.f16_to_f32(s16), 64).reshape(w.shape).astype(np.float64)
    zz = 0 if sym else np.repeat(z, 64).reshape(w.shape).astype(np.float64)
    err = np.abs(s * (q - zz) - w)
    inner = (q > (-7 if sym else 0)) & (q < (7 if sym else 15))
    assert np.all((err <= s / 2 * (1 + 2.0 ** -20) + np.abs(w) * 2.0 ** -22)[inner])


def test_metadata_share_matches_the_pages():
    """With binary16 scales the metadata of INT4 weights is 1/32 of the code bytes at g = 128 (the pages: about
    3 %) and 1/8 at g = 32 (about 13 %) [P3 §11.3.7; P1 §1.1: 3-5 % and 10-15 %]; fp32 scales double it."""
    w = np.zeros((64, 1024), np.float32)
    w[:, ::7] = 1.0
    codes_bytes = oracle.pack_int4(oracle.quantize_meta16(w, True, 128)[0]).nbytes
    for g, pages in ((128, 0.03), (32, 0.13)):
        _, s16, _ = oracle.quantize_meta16(w, True, g)
        _, s32, _ = oracle.quantize(w, 4, True, oracle.GROUP, g)
        share16 = s16.nbytes / codes_bytes
        assert abs(share16 - pages) < 0.006
        assert s32.nbytes / codes_bytes == 2 * share16


def test_pack_zeros4_round_trip():
    """Packed zero points (two per byte) unpack to the zero points, odd counts included."""
    rng = np.random.default_rng(32)
    for n in (6, 7, 129):
        z = rng.integers(0, 16, n).astype(np.uint8)
        p = oracle.pack_zeros4(z)
        assert p.size == (n + 1) // 2
        lo, hi = p & 0xF, p >> 4
        assert np.array_equal(np.stack([lo, hi], 1).ravel()[:n], z)


@pytest.mark.parametrize("sym", [True, False])
def test_meta16_saturated_scale_clamps_the_code(sym):
    """A group holding values of 1e14 and more: its fp32 scale exceeds binary16, the stored scale saturates at
    65504, and x / s16 lies far beyond the int range. The clamp of the core formula applies to the rounded
    quotient plus z ("量化、蒸馏与模型压缩", core formula), so the largest positive value codes to the top
    of the range and the most negative one to the bottom -- never to a wrapped integer."""
    x = np.zeros((1, 32), np.float32)
    x[0, :5] = [1e38, -7e37, 3e37, -1e36, 2e14]
    q, s16, z = oracle.quantize_meta16(x, sym, 32)
    assert s16[0] == 0x7BFF  # 65504
    top, bottom = (7, -7) if sym else (15, 0)
    assert q[0, 0] == top and q[0, 2] == top and q[0, 4] == top
    assert q[0, 1] == bottom and q[0, 3] == bottom
    if not sym:
        assert z[0] == 15  # -lo / 65504 is far above 15: the zero point clamps too
