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


def key_err_ratio(got_bits, ref_bits):
    """Largest |got - ref| / bound of stored keys (normalised, rotated, rounded to BF16).

    The GPU computes them in FP32 and the oracle in float64; both round once to
    BF16.  An FP32 result differs from the exact one by a few units of 2^-24 of
    the row's scale, which can move it across one BF16 rounding boundary: the
    bound is one BF16 ulp of the reference element plus 2^-20 of the row's
    largest magnitude (the FP32 error with margin, for components that nearly
    cancel in the rotation).
    """
    g = O.bf16_to_f64(got_bits)
    r = O.bf16_to_f64(ref_bits)
    _, e = np.frexp(r)
    ulp = np.where(r != 0, np.ldexp(1.0, e - 8), 0.0)
    row = np.abs(r).max(axis=-1, keepdims=True)
    err = np.abs(g - r)
    bound = ulp + 2.0**-20 * row
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
