"""The comparison rules the GPU parity tests apply, checked on constructed cases."""

import numpy as np

import oracle as O
from attn_check import attn_errors, key_err_stats


def test_key_bound_accepts_one_ulp_and_rejects_two():
    rng = np.random.default_rng(0)
    ref = O.f64_to_bf16(rng.standard_normal((4, 256)))
    ratio, nd, nb, _ = key_err_stats(ref, ref)
    assert ratio == 0.0 and nd == 0 and nb == 0
    one_up = ref.copy()
    one_up[1, 7] += 1  # one BF16 step away from zero (positive or negative alike)
    ratio, nd, nb, _ = key_err_stats(one_up, ref)
    assert nd == 1 and nb == 0 and ratio <= 1.0
    two_up = ref.copy()
    two_up[2, 100] += 2
    ratio, nd, nb, excess = key_err_stats(two_up, ref)
    # two steps exceed one ulp by a full ulp, far more than 16 units of 2^-24 of the row max
    assert nd == 1 and nb == 1 and ratio > 1.0 and excess > 16


def test_attention_errors_are_row_relative_and_treat_empty_rows():
    o_ref = np.array([[1.0, -2.0, 0.5], [0.0, 0.0, 0.0]])
    lse_ref = np.array([3.0, -np.inf])
    got = O.f64_to_bf16(np.array([[1.0, -2.03, 0.5], [0.0, 0.0, 0.0]]))
    rel, lerr = attn_errors(got, np.array([3.01, -np.inf]), o_ref, lse_ref)
    # largest deviation in the row over the row's largest reference magnitude (2.0)
    assert abs(rel[0] - abs(O.bf16_to_f64(got)[0, 1] + 2.0) / 2.0) < 1e-12
    assert rel[1] == 0.0 and lerr[1] == 0.0
    assert abs(lerr[0] - 0.01 / 3.0) < 1e-12


def test_key_bound_requires_untouched_non_finite_slots():
    ref = O.f64_to_bf16(np.ones((2, 256)))
    ref[1, :] = 0x7FC0  # a slot outside the valid records, holding NaN
    assert key_err_stats(ref.copy(), ref)[0] == 0.0
    bad = ref.copy()
    bad[1, 3] = 0x3F80
    assert key_err_stats(bad, ref)[0] == float("inf")
