"""Comparison rules for the GDN step (NumPy only, so worker processes can use them).

New matrices: the GPU forms a S + k u in FP32 and rounds once to the storage type;
the oracle forms it in float64 and rounds once.  The FP32 value is within a few
2^-24 of the head's largest magnitude of the exact one, which can move it across
one rounding boundary of the storage type: the bound is one unit in the last place
of the reference element plus 2^-18 of the head's largest magnitude.
Outputs: BF16, within 1e-2 of their row's largest magnitude.
"""

from __future__ import annotations

import numpy as np

O_TOL = 1e-2


def state_bound(ref, whole=False):
    """Per-element bound of one step for matrices ref [..., 128, 128]: the magnitude
    term is each head's largest element, or with whole=True the largest element of
    all of ref."""
    r = np.asarray(ref, np.float64)
    if ref.dtype == np.float16:
        _, e = np.frexp(np.maximum(np.abs(r), 2.0 ** -14))
        ulp = np.ldexp(1.0, e - 11)
    else:
        _, e = np.frexp(np.maximum(np.abs(r), 2.0 ** -126))
        ulp = np.ldexp(1.0, e - 24)
    if whole:
        return ulp + 2.0 ** -18 * np.abs(r).max()
    lead = r.reshape(-1, r.shape[-2] * r.shape[-1])
    scale = np.abs(lead).max(axis=1).reshape(r.shape[:-2] + (1, 1))
    return ulp + 2.0 ** -18 * scale


def state_err_ratio(got, ref):
    """Largest |got - ref| / bound over all elements."""
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float((err / state_bound(ref)).max())


def out_rel(got, ref):
    """Per-row max |got - ref| / max |ref| of outputs [..., 128] (got: float values)."""
    g = np.asarray(got, np.float64).reshape(-1, 128)
    r = np.asarray(ref, np.float64).reshape(-1, 128)
    scale = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return np.abs(g - r).max(axis=1) / scale
