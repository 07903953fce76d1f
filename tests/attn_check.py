"""Comparison rules for attention outputs and stored keys (NumPy only, so worker
processes can use them without torch)."""

from __future__ import annotations

import numpy as np

import oracle as O


def attn_errors(o_gpu_bits, lse_gpu, o_ref, lse_ref):
    """Per-row relative output error and per-row LSE error (arrays over all rows)."""
    og = O.bf16_to_f64(o_gpu_bits).reshape(-1, o_ref.shape[-1])
    orf = np.asarray(o_ref, np.float64).reshape(-1, o_ref.shape[-1])
    scale = np.abs(orf).max(axis=1)
    err = np.abs(og - orf).max(axis=1)
    rel = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)
    lg = np.asarray(lse_gpu, np.float64).reshape(-1)
    lr = np.asarray(lse_ref, np.float64).reshape(-1)
    both_inf = np.isneginf(lg) & np.isneginf(lr)
    with np.errstate(invalid="ignore"):
        lerr = np.where(both_inf, 0.0, np.abs(lg - lr) / np.maximum(1.0, np.abs(lr)))
    return rel, lerr


KEY_ROW_SLACK = 2.0**-20  # FP32 error allowance of a stored key, times the row's largest magnitude


def key_err_stats(got_bits, ref_bits):
    """Stored keys (normalised, rotated, rounded to BF16) against the oracle's.

    The GPU computes a key in FP32 and the oracle in float64; both round once to
    BF16.  The FP32 value is off the exact one by a few units of 2^-24 of the row's
    largest magnitude (the norm factor, gain, cos/sin and products each add one or
    two such units; a rotated component that nearly cancels keeps the error of its
    operands, not of itself).  Each side then rounds within half a BF16 ulp of its
    own value, so |got - ref| <= 1 ulp(ref) + (FP32 error).  The bound used is one
    BF16 ulp of the reference element plus 2^-20 (16 units of 2^-24) of the row's
    largest magnitude.

    Returns (ratio, n_diff, n_beyond_ulp, excess): the largest |got - ref| / bound,
    the number of elements whose bits differ, the number that differ by more than
    one ulp, and the largest such excess over one ulp in units of 2^-24 of the row
    maximum.
    """
    got_bits, ref_bits = np.asarray(got_bits), np.asarray(ref_bits)
    g = O.bf16_to_f64(got_bits)
    r = O.bf16_to_f64(ref_bits)
    if g.size == 0:
        return 0.0, 0, 0, 0.0
    # a NaN or infinite reference (never a stored key; it marks a slot that must be
    # left as it was) must be matched bit for bit
    nonfin = ~np.isfinite(r)
    if np.any(got_bits[nonfin] != ref_bits[nonfin]):
        return float("inf"), int((got_bits != ref_bits).sum()), 0, float("inf")
    r = np.where(nonfin, 0.0, r)
    g = np.where(nonfin, 0.0, g)
    _, e = np.frexp(r)
    ulp = np.where(r != 0, np.ldexp(1.0, e - 8), 0.0)
    row = np.abs(r).max(axis=-1, keepdims=True)
    err = np.abs(g - r)
    bound = ulp + KEY_ROW_SLACK * row
    ratio = float((err / np.maximum(bound, 1e-300)).max())
    n_diff = int((got_bits != ref_bits).sum())
    beyond = err > ulp
    excess = float(((err - ulp) / np.maximum(row, 1e-300) * 2.0**24)[beyond].max()) if beyond.any() else 0.0
    return ratio, n_diff, int(beyond.sum()), excess


def key_err_ratio(got_bits, ref_bits):
    """The largest |got - ref| / bound of key_err_stats."""
    return key_err_stats(got_bits, ref_bits)[0]
