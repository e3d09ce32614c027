"""The per-element bounds of the GPU parity tests catch what a normwise error hides (CPU, oracle only).

A single output element of a 28,672-wide bf16 row that is off by 5 % moves the normwise error by far less than
the 5e-3 tolerance, but breaks |y - y_ref| <= 2^-8 |y_ref| + 2^-11 sum_k |x_k| |w_k| at that element; the exact
oracle output, rounded to bf16, stays inside the bound everywhere.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import BOUND_BF16, abs_terms_w4, assert_per_element, normwise


def _case():
    rng = np.random.default_rng(12)
    n, k = 28672, 256
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = W.bf16_bits(rng.standard_normal((1, k)).astype(np.float32))
    q, s, _ = oracle.quantize(w, 4, True, oracle.GROUP, 128)
    y_ref = oracle.w4a16(x, q, s, None, 128)
    return y_ref, abs_terms_w4(x, q, s, None, 128)


def test_bf16_rounding_of_the_exact_output_is_inside_the_bound():
    y_ref, terms = _case()
    y16 = W.bf16_to_f32(W.bf16_bits(y_ref.astype(np.float32))).astype(np.float64)
    assert_per_element(y16, y_ref, terms, BOUND_BF16, "bf16 rounding")


def test_one_wrong_element_breaks_the_bound_but_not_the_norm():
    y_ref, terms = _case()
    y = y_ref.copy()
    i = int(np.argmax(np.abs(y_ref)))
    y[0, i] *= 1.05
    assert normwise(y, y_ref) < 5e-3
    with pytest.raises(AssertionError, match="outside the per-element bound"):
        assert_per_element(y, y_ref, terms, BOUND_BF16, "planted")
