"""Float64 reference of the INT8 K/V state variant of the RMA hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path.

The pages list INT8 and FP8 releases of EdgeRock-4B (fluxbbs.com page, section
"架构：递归、局部窗口与记忆锚点三件套"; neodrop.ai repost of the QbitAI article, section
"开源到哪一步") but no format for the attention state, so, as for FP8, this variant
is a reading of this build:

  * every stored K and V row (256 values of one sequence, KV group and slot) is held
    as 256 signed 8-bit integer codes (two's complement) and one FP32 scale;
  * scale = amax / 127 with amax = max_i |x_i|, computed in FP32; a row whose amax
    is below 127 * 2^-126 (where 127 / amax would pass 2^126 and the scale would
    leave the normal FP32 range), the all-zero row included, has scale 0 and all
    codes 0;
  * code_i = round-half-even(fp32(x_i * inv)), inv = fp32(127 / amax), so
    |code_i| <= 127 (-128 is never written);
  * the stored row means code_i * scale.

The layout is that of the FP8 state (1-byte codes plus one FP32 scale per row), so
the state object, the append loop, the attention over dequantised rows and the
commit are those of ``oracle.fp8_ref`` with this codec in place of E4M3.
"""

from __future__ import annotations

import numpy as np

from . import fp8_ref as F

I8_MAX = 127.0
TINY_ROW = np.float32(I8_MAX * 2.0**-126)  # rows below this amax are stored as zero

LayerStateI8 = F.LayerStateFP8
new_layer_state_i8 = F.new_layer_state_fp8
commit = F.commit  # an admitted row moves with its codes and scales, whatever they mean
kv_bytes_per_unit = F.kv_bytes_per_unit


def quantize_rows(x_f32):
    """Rows [..., 256] of FP32 values -> (codes uint8 [..., 256] holding int8, scale f32 [...])."""
    x = np.asarray(x_f32, np.float32)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax < TINY_ROW
    safe = np.where(zero, np.float32(1.0), amax)
    inv = np.float32(I8_MAX) / safe  # FP32 division, correctly rounded
    scale = np.where(zero, np.float32(0.0), amax / np.float32(I8_MAX)).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)  # FP32 product
    q = np.rint(y.astype(np.float64)).astype(np.int64)  # exact on FP32 values; ties to even
    q = np.where(zero[..., None], 0, q)
    return q.astype(np.int8).view(np.uint8), scale


def dequantize(codes, scale) -> np.ndarray:
    """Exact float64 value of stored rows: the signed code times the row's scale."""
    c = np.asarray(codes, np.uint8).view(np.int8).astype(np.float64)
    return c * np.asarray(scale, np.float64)[..., None]


def append(st, k_win, v_win, k_rma, v_rma, gk_win, gk_rma, eps: float, base: float,
           score=None) -> None:
    """``rma_ref.append`` with each written row quantised to INT8 (keys from their FP32
    normalised and rotated value, values from their BF16 input)."""
    F.append(st, k_win, v_win, k_rma, v_rma, gk_win, gk_rma, eps, base, score, quant=quantize_rows)


def decode(st, q_win, q_rma, gq_win, gq_rma, eps: float, base: float):
    """Both branches for every sequence over the dequantised INT8 rows (float64)."""
    return F.decode(st, q_win, q_rma, gq_win, gq_rma, eps, base, deq=dequantize)
