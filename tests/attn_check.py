"""Comparison rule for attention outputs (NumPy only, so worker processes can use it
without torch)."""

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
