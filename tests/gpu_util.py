"""Helpers for the GPU parity tests: moving state between the oracle (NumPy) and the
library (torch device tensors), and the comparison rules."""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
import swa_memory_anchor_amd as R
from attn_check import attn_errors, key_err_stats  # noqa: F401  (attn_errors re-exported)

DEV = "cuda"
ATTN_TOL = 2e-2  # row-relative, BF16 I/O with FP32 accumulation
SCORE_TOL = 1e-5  # |s_gpu - s_ref| <= SCORE_TOL * max(1, |s_ref|)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to(DEV).view(torch.bfloat16)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_dev(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def i32_dev(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


KV = ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v")
META = ("bank_score", "bank_src", "pend_score", "pend_src", "n_bank", "n_pend", "pos")


def upload(st: O.LayerState) -> R.LayerState:
    d = {nm: bf16_dev(getattr(st, nm)) for nm in KV}
    for nm in META:
        a = getattr(st, nm)
        d[nm] = f32_dev(a) if a.dtype == np.float32 else i32_dev(a)
    return R.LayerState(**d)


def download(st: R.LayerState) -> O.LayerState:
    d = {nm: bits_host(getattr(st, nm)) for nm in KV}
    for nm in META:
        d[nm] = getattr(st, nm).cpu().numpy()
    return O.LayerState(**d)


def norm_dev(gains: dict, eps=1e-6, base=1e7) -> R.Norm:
    return R.Norm(f32_dev(gains["gq_win"]), f32_dev(gains["gk_win"]), f32_dev(gains["gq_rma"]),
                  f32_dev(gains["gk_rma"]), eps, base)


def decode_gpu(st: R.LayerState, q_win: torch.Tensor, q_rma: torch.Tensor, norm: R.Norm):
    B = st.batch
    o_w = torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV)
    o_r = torch.empty_like(o_w)
    l_w = torch.empty(B, 16, dtype=torch.float32, device=DEV)
    l_r = torch.empty_like(l_w)
    ws = R.decode_workspace(B)
    R.swa_rma_decode_attn(st, B, q_win, q_rma, norm, o_w, l_w, o_r, l_r, ws)
    return o_w, l_w, o_r, l_r


def assert_attn_close(o_gpu_bits, lse_gpu, o_ref, lse_ref, tol=ATTN_TOL, what=""):
    rel, lerr = attn_errors(o_gpu_bits, lse_gpu, o_ref, lse_ref)
    msg = (f"{what}: rows={rel.size} out max={rel.max():.3e} median={np.median(rel):.3e}; "
           f"lse max={lerr.max():.3e}")
    print(msg)
    assert np.all(np.isfinite(rel)) and rel.max() <= tol, msg
    assert np.all(np.isfinite(lerr)) and lerr.max() <= tol, msg
    return rel, lerr


def assert_scores_close(s_gpu, s_ref, tol=SCORE_TOL, what=""):
    s_gpu = np.asarray(s_gpu, np.float64)
    s_ref = np.asarray(s_ref, np.float64)
    bound = tol * np.maximum(1.0, np.abs(s_ref))
    err = np.abs(s_gpu - s_ref)
    print(f"{what}: scores n={err.size} max err={err.max():.3e} (bound {bound.min():.1e})")
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} scores out of tolerance"


def assert_keys_close(got_bits, ref_bits, what=""):
    """Stored keys against the oracle's within attn_check.key_err_stats's bound (one
    BF16 ulp of the reference element plus 2^-20 of the row's largest magnitude)."""
    ratio, ndiff, nbeyond, excess = key_err_stats(got_bits, ref_bits)
    print(f"{what}: {ndiff} of {np.asarray(got_bits).size} elements differ, {nbeyond} by more "
          f"than one BF16 ulp (largest excess {excess:.2f} x 2^-24 of the row maximum); "
          f"max err/bound {ratio:.3f}")
    assert ratio <= 1.0, f"{what}: out of bound ({ratio:.3f})"


# ---------------------------------------------------------------- FP8 state
KV_SCALES = tuple(nm + "s" for nm in KV)


def upload_fp8(st) -> R.LayerStateFP8:
    """oracle.fp8_ref.LayerStateFP8 (host) -> device state."""
    d = {nm: torch.from_numpy(np.ascontiguousarray(getattr(st, nm), dtype=np.uint8)).to(DEV)
         for nm in KV}
    for nm in KV_SCALES:
        d[nm] = f32_dev(getattr(st, nm))
    for nm in META:
        a = getattr(st, nm)
        d[nm] = f32_dev(a) if a.dtype == np.float32 else i32_dev(a)
    return R.LayerStateFP8(**d)


def download_fp8(st: R.LayerStateFP8):
    from oracle import fp8_ref as F

    d = {nm: getattr(st, nm).cpu().numpy() for nm in KV + KV_SCALES + META}
    return F.LayerStateFP8(**d)


def decode_gpu_fp8(st: R.LayerStateFP8, q_win, q_rma, norm: R.Norm):
    B = st.pos.shape[0]
    o_w = torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV)
    o_r = torch.empty_like(o_w)
    l_w = torch.empty(B, 16, dtype=torch.float32, device=DEV)
    l_r = torch.empty_like(l_w)
    R.swa_rma_decode_attn_fp8(st, B, q_win, q_rma, norm, o_w, l_w, o_r, l_r,
                              R.decode_workspace(B))
    return o_w, l_w, o_r, l_r


def decode_gpu_i8(st: R.LayerStateFP8, q_win, q_rma, norm: R.Norm):
    B = st.pos.shape[0]
    o_w = torch.empty(B, 16, 256, dtype=torch.bfloat16, device=DEV)
    o_r = torch.empty_like(o_w)
    l_w = torch.empty(B, 16, dtype=torch.float32, device=DEV)
    l_r = torch.empty_like(l_w)
    R.swa_rma_decode_attn_i8(st, B, q_win, q_rma, norm, o_w, l_w, o_r, l_r,
                             R.decode_workspace(B))
    return o_w, l_w, o_r, l_r


def assert_i8_keys_close(got_codes, got_scale, ref_codes, ref_scale, what=""):
    """Stored INT8 key rows against the oracle's.

    As for FP8, the GPU's FP32 normalised and rotated key differs from the oracle's
    (float64 rounded to FP32) by a few units of 2^-24 of the row's largest magnitude,
    and the scale with it; a scaled element near a half-integer can then take the
    neighbouring code.  Each dequantised element must lie within one step of the
    row's grid (its scale) of the reference, plus 2^-16 of the row's largest
    magnitude; the scales must agree to 2^-18 relative.
    """
    from oracle import int8_ref as I

    gs = np.asarray(got_scale, np.float64)
    rs = np.asarray(ref_scale, np.float64)
    assert np.all(np.abs(gs - rs) <= 2.0 ** -18 * rs), f"{what}: scales differ"
    g = I.dequantize(got_codes, got_scale)
    r = I.dequantize(ref_codes, ref_scale)
    row = np.abs(r).max(axis=-1, keepdims=True)
    err = np.abs(g - r)
    bound = rs[..., None] + 2.0 ** -16 * row
    ndiff = int((np.asarray(got_codes) != np.asarray(ref_codes)).sum())
    print(f"{what}: {ndiff} of {g.size} codes differ; max err/bound "
          f"{float((err / np.maximum(bound, 1e-300)).max()):.3f}")
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} elements out of bound"


def assert_fp8_keys_close(got_codes, got_scale, ref_codes, ref_scale, what=""):
    """Stored FP8 key rows against the oracle's.

    The GPU forms the normalised, rotated key in FP32 and the oracle in float64
    (then rounds to FP32), so the two FP32 rows differ by a few units of 2^-24 of
    the row's largest magnitude.  The row maximum, and with it the scale, can move
    by as much; a scaled element near a rounding midpoint of the E4M3 grid can
    then take the neighbouring code.  The bound on each dequantised element is one
    E4M3 step at the reference element plus 2^-16 of the row's largest dequantised
    magnitude (the scale change acting on a code up to 448, with margin); the
    scales must agree to 2^-18 relative.
    """
    from oracle import fp8_ref as F

    gs = np.asarray(got_scale, np.float64)
    rs = np.asarray(ref_scale, np.float64)
    assert np.all(np.abs(gs - rs) <= 2.0 ** -18 * rs), f"{what}: scales differ"
    g = F.dequantize(got_codes, got_scale)
    r = F.dequantize(ref_codes, ref_scale)
    step = F.e4m3_step(F.e4m3_decode(ref_codes)) * rs[..., None]
    row = np.abs(r).max(axis=-1, keepdims=True)
    err = np.abs(g - r)
    bound = step + 2.0 ** -16 * row
    ndiff = int((np.asarray(got_codes) != np.asarray(ref_codes)).sum())
    print(f"{what}: {ndiff} of {g.size} codes differ; max err/bound "
          f"{float((err / np.maximum(bound, 1e-300)).max()):.3f}")
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} elements out of bound"
