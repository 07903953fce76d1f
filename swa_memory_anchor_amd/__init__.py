"""Python binding of ``librma.so``: the Rock Memory Anchors (RMA) hot path on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels behind
the C ABI declared in ``include/rma.h``; this module converts torch tensors (used
for device memory and streams) into pointers and calls the entry points of the
same names.  If the library has not been built, importing the entry points
raises: there is no fallback.

Entry points: ``swa_rma_append``, ``swa_rma_decode_attn``, ``rma_score``,
``rma_commit_topk``, ``swa_rma_prefill``, the FP8-state variants ``swa_rma_append_fp8``,
``swa_rma_decode_attn_fp8`` and ``rma_commit_topk_fp8`` (which also commits the INT8
state), the INT8-state variants ``swa_rma_append_i8`` and ``swa_rma_decode_attn_i8``,
plus the size helpers
``rma_layer_state_bytes``, ``rma_layer_state_fp8_bytes``, ``rma_layer_kv_bytes``,
``rma_decode_workspace_bytes``, ``rma_decode_splits``, ``rma_prefill_workspace_bytes`` and
``rma_status_str``.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, fields

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librma.so")

Q_HEADS, KV_GROUPS, HEAD_DIM, ROPE_DIM = 16, 4, 256, 64
WINDOW, BANK, BLOCK, HIDDEN, SCORER_MID = 1024, 1024, 256, 2560, 256

EXPORTS = (
    "rma_layer_state_bytes", "rma_layer_kv_bytes", "rma_decode_workspace_bytes",
    "rma_decode_splits", "swa_rma_append", "swa_rma_decode_attn", "rma_score",
    "rma_commit_topk", "rma_status_str", "rma_prefill_workspace_bytes", "swa_rma_prefill",
    "rma_layer_state_fp8_bytes", "swa_rma_append_fp8", "swa_rma_decode_attn_fp8",
    "rma_commit_topk_fp8", "gdn_layer_state_bytes", "gdn_decode_step",
    "rma_step_workspace_bytes", "swa_rma_step", "rma_score_multi", "rma_score_workspace_bytes",
    "rma_score_multi_ws", "rma_commit_topk_multi",
    "gdn_prefill", "swa_rma_decode_attn_noalloc", "swa_rma_append_i8", "swa_rma_decode_attn_i8",
)

_c_void_p = ctypes.c_void_p


class RmaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {rma_status_str(status)} (status {status})")
        self.status = status


class _StateC(ctypes.Structure):
    _fields_ = [(n, _c_void_p) for n in (
        "win_k", "win_v", "bank_k", "bank_v", "bank_score", "bank_src", "pend_k", "pend_v",
        "pend_score", "pend_src", "n_bank", "n_pend", "pos")]


class _StateFp8C(ctypes.Structure):
    _fields_ = [(n, _c_void_p) for n in (
        "win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v", "win_ks", "win_vs", "bank_ks",
        "bank_vs", "pend_ks", "pend_vs", "bank_score", "bank_src", "pend_score", "pend_src",
        "n_bank", "n_pend", "pos")]


class _NormC(ctypes.Structure):
    _fields_ = [("gq_win", _c_void_p), ("gk_win", _c_void_p), ("gq_rma", _c_void_p),
                ("gk_rma", _c_void_p), ("eps", ctypes.c_float), ("rope_base", ctypes.c_float)]


class _ScoreJobC(ctypes.Structure):
    _fields_ = [("hidden", _c_void_p), ("w1", _c_void_p), ("w2", _c_void_p),
                ("scores", _c_void_p)]


class _GdnStateC(ctypes.Structure):
    _fields_ = [("S", _c_void_p), ("conv", _c_void_p)]


class _GdnParamsC(ctypes.Structure):
    _fields_ = [("conv_w", _c_void_p), ("a_log", _c_void_p), ("dt_bias", _c_void_p)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it is missing)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m swa_memory_anchor_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, _c_void_p
        sp = ctypes.POINTER(_StateC)
        npp = ctypes.POINTER(_NormC)
        for nm in ("rma_layer_state_bytes", "rma_layer_kv_bytes", "rma_decode_workspace_bytes",
                   "rma_step_workspace_bytes"):
            getattr(L, nm).argtypes, getattr(L, nm).restype = [i32], sz
        L.rma_decode_splits.argtypes, L.rma_decode_splits.restype = [i32], i32
        L.swa_rma_append.argtypes = [sp, i32, vp, vp, vp, vp, vp, npp, vp]
        L.swa_rma_append.restype = ctypes.c_int
        L.swa_rma_decode_attn.argtypes = [sp, i32, vp, vp, npp, vp, vp, vp, vp, vp, sz, vp]
        L.swa_rma_decode_attn.restype = ctypes.c_int
        L.swa_rma_decode_attn_noalloc.argtypes = [sp, i32, vp, vp, npp, vp, vp, vp, vp, vp]
        L.swa_rma_decode_attn_noalloc.restype = ctypes.c_int
        L.swa_rma_step.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, npp, vp, vp, vp, vp, vp,
                                   sz, vp]
        L.swa_rma_step.restype = ctypes.c_int
        L.rma_score.argtypes = [vp, i64, i64, vp, vp, vp, i64, vp]
        L.rma_score.restype = ctypes.c_int
        L.rma_commit_topk.argtypes = [sp, i32, vp, vp]
        L.rma_score_multi.argtypes = [ctypes.POINTER(_ScoreJobC), i32, i64, i64, i64, vp]
        L.rma_score_multi.restype = ctypes.c_int
        L.rma_score_workspace_bytes.argtypes = [i32, i64]
        L.rma_score_workspace_bytes.restype = sz
        L.rma_score_multi_ws.argtypes = [ctypes.POINTER(_ScoreJobC), i32, i64, i64, i64, vp, sz,
                                         vp]
        L.rma_score_multi_ws.restype = ctypes.c_int
        L.rma_commit_topk_multi.argtypes = [sp, i32, i32, ctypes.POINTER(vp), vp]
        L.rma_commit_topk_multi.restype = ctypes.c_int
        L.rma_commit_topk.restype = ctypes.c_int
        L.rma_status_str.argtypes, L.rma_status_str.restype = [ctypes.c_int], ctypes.c_char_p
        L.rma_prefill_workspace_bytes.argtypes = [i32, i32]
        L.rma_prefill_workspace_bytes.restype = sz
        L.swa_rma_prefill.argtypes = [sp, i32, i32, vp, vp, vp, vp, vp, vp, vp, npp, vp, vp, vp,
                                      vp, vp, sz, vp]
        L.swa_rma_prefill.restype = ctypes.c_int
        s8 = ctypes.POINTER(_StateFp8C)
        L.rma_layer_state_fp8_bytes.argtypes, L.rma_layer_state_fp8_bytes.restype = [i32], sz
        L.swa_rma_append_fp8.argtypes = [s8, i32, vp, vp, vp, vp, vp, npp, vp]
        L.swa_rma_append_fp8.restype = ctypes.c_int
        L.swa_rma_decode_attn_fp8.argtypes = [s8, i32, vp, vp, npp, vp, vp, vp, vp, vp, sz, vp]
        L.swa_rma_decode_attn_fp8.restype = ctypes.c_int
        L.rma_commit_topk_fp8.argtypes = [s8, i32, vp, vp]
        L.rma_commit_topk_fp8.restype = ctypes.c_int
        L.swa_rma_append_i8.argtypes = [s8, i32, vp, vp, vp, vp, vp, npp, vp]
        L.swa_rma_append_i8.restype = ctypes.c_int
        L.swa_rma_decode_attn_i8.argtypes = [s8, i32, vp, vp, npp, vp, vp, vp, vp, vp, sz, vp]
        L.swa_rma_decode_attn_i8.restype = ctypes.c_int
        L.gdn_layer_state_bytes.argtypes, L.gdn_layer_state_bytes.restype = [i32, i32], sz
        L.gdn_decode_step.argtypes = [ctypes.POINTER(_GdnStateC), i32, i32, vp, vp, vp, vp,
                                      ctypes.POINTER(_GdnParamsC), vp, vp]
        L.gdn_decode_step.restype = ctypes.c_int
        L.gdn_prefill.argtypes = [ctypes.POINTER(_GdnStateC), i32, i32, i32, vp, vp, vp, vp,
                                  ctypes.POINTER(_GdnParamsC), vp, vp]
        L.gdn_prefill.restype = ctypes.c_int
        _LIB = L
    return _LIB


# ---------------------------------------------------------------- plumbing (torch memory)
@dataclass
class LayerState:
    """Device tensors of one layer's state; shapes as in ``include/rma.h``."""

    win_k: object
    win_v: object
    bank_k: object
    bank_v: object
    bank_score: object
    bank_src: object
    pend_k: object
    pend_v: object
    pend_score: object
    pend_src: object
    n_bank: object
    n_pend: object
    pos: object

    @property
    def batch(self) -> int:
        return int(self.n_bank.shape[0])


@dataclass
class LayerStateFP8:
    """Device tensors of one layer's FP8 state (E4M3 codes + one FP32 scale per row)."""

    win_k: object
    win_v: object
    bank_k: object
    bank_v: object
    pend_k: object
    pend_v: object
    win_ks: object
    win_vs: object
    bank_ks: object
    bank_vs: object
    pend_ks: object
    pend_vs: object
    bank_score: object
    bank_src: object
    pend_score: object
    pend_src: object
    n_bank: object
    n_pend: object
    pos: object

    @property
    def batch(self) -> int:
        return int(self.n_bank.shape[0])


@dataclass
class Norm:
    gq_win: object
    gk_win: object
    gq_rma: object
    gk_rma: object
    eps: float = 1e-6
    rope_base: float = 1e7


def alloc_layer_state(batch: int, device="cuda", zero_kv: bool = True) -> LayerState:
    """Allocate one layer's state with torch (empty: n_bank = n_pend = 0, pos = -1)."""
    import torch

    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    mk = torch.zeros if zero_kv else torch.empty
    return LayerState(
        win_k=mk(batch, KV_GROUPS, WINDOW, HEAD_DIM, dtype=bf, device=device),
        win_v=mk(batch, KV_GROUPS, WINDOW, HEAD_DIM, dtype=bf, device=device),
        bank_k=mk(batch, KV_GROUPS, BANK, HEAD_DIM, dtype=bf, device=device),
        bank_v=mk(batch, KV_GROUPS, BANK, HEAD_DIM, dtype=bf, device=device),
        bank_score=torch.zeros(batch, KV_GROUPS, BANK, dtype=f32, device=device),
        bank_src=torch.zeros(batch, KV_GROUPS, BANK, dtype=i32, device=device),
        pend_k=mk(batch, KV_GROUPS, BLOCK, HEAD_DIM, dtype=bf, device=device),
        pend_v=mk(batch, KV_GROUPS, BLOCK, HEAD_DIM, dtype=bf, device=device),
        pend_score=torch.zeros(batch, BLOCK, KV_GROUPS, dtype=f32, device=device),
        pend_src=torch.zeros(batch, BLOCK, dtype=i32, device=device),
        n_bank=torch.zeros(batch, dtype=i32, device=device),
        n_pend=torch.zeros(batch, dtype=i32, device=device),
        pos=torch.full((batch,), -1, dtype=i32, device=device),
    )


def alloc_layer_state_fp8(batch: int, device="cuda") -> LayerStateFP8:
    """Allocate one layer's FP8 state with torch (empty: n_bank = n_pend = 0, pos = -1)."""
    import torch

    u8, f32, i32 = torch.uint8, torch.float32, torch.int32
    c = lambda n: torch.zeros(batch, KV_GROUPS, n, HEAD_DIM, dtype=u8, device=device)  # noqa: E731
    s = lambda n: torch.zeros(batch, KV_GROUPS, n, dtype=f32, device=device)  # noqa: E731
    return LayerStateFP8(
        win_k=c(WINDOW), win_v=c(WINDOW), bank_k=c(BANK), bank_v=c(BANK), pend_k=c(BLOCK),
        pend_v=c(BLOCK), win_ks=s(WINDOW), win_vs=s(WINDOW), bank_ks=s(BANK), bank_vs=s(BANK),
        pend_ks=s(BLOCK), pend_vs=s(BLOCK),
        bank_score=torch.zeros(batch, KV_GROUPS, BANK, dtype=f32, device=device),
        bank_src=torch.zeros(batch, KV_GROUPS, BANK, dtype=i32, device=device),
        pend_score=torch.zeros(batch, BLOCK, KV_GROUPS, dtype=f32, device=device),
        pend_src=torch.zeros(batch, BLOCK, dtype=i32, device=device),
        n_bank=torch.zeros(batch, dtype=i32, device=device),
        n_pend=torch.zeros(batch, dtype=i32, device=device),
        pos=torch.full((batch,), -1, dtype=i32, device=device),
    )


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_contiguous(), "tensors passed to the library must be contiguous"
    return t.data_ptr()


def _state_c(st: LayerState) -> _StateC:
    return _StateC(*[_ptr(getattr(st, f.name)) for f in fields(LayerState)])


def _state_fp8_c(st: LayerStateFP8) -> _StateFp8C:
    return _StateFp8C(*[_ptr(getattr(st, f.name)) for f in fields(LayerStateFP8)])


def _norm_c(nm: Norm) -> _NormC:
    return _NormC(_ptr(nm.gq_win), _ptr(nm.gk_win), _ptr(nm.gq_rma), _ptr(nm.gk_rma),
                  float(nm.eps), float(nm.rope_base))


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != 0:
        raise RmaError(status, where)


# ---------------------------------------------------------------- entry points
def rma_status_str(status: int) -> str:
    return lib().rma_status_str(int(status)).decode()


def rma_layer_state_bytes(batch: int) -> int:
    return int(lib().rma_layer_state_bytes(int(batch)))


def rma_layer_kv_bytes(batch: int) -> int:
    return int(lib().rma_layer_kv_bytes(int(batch)))


def rma_decode_workspace_bytes(batch: int) -> int:
    return int(lib().rma_decode_workspace_bytes(int(batch)))


def rma_decode_splits(batch: int) -> int:
    return int(lib().rma_decode_splits(int(batch)))


def swa_rma_append(st: LayerState, batch: int, k_win, v_win, k_rma, v_rma, score, norm: Norm,
                   stream=None) -> None:
    s = lib().swa_rma_append(ctypes.byref(_state_c(st)), int(batch), _ptr(k_win), _ptr(v_win),
                             _ptr(k_rma), _ptr(v_rma), _ptr(score), ctypes.byref(_norm_c(norm)),
                             _stream(stream))
    _check(s, "swa_rma_append")


def swa_rma_decode_attn(st: LayerState, batch: int, q_win, q_rma, norm: Norm, o_win, lse_win,
                        o_rma, lse_rma, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = lib().swa_rma_decode_attn(ctypes.byref(_state_c(st)), int(batch), _ptr(q_win),
                                  _ptr(q_rma), ctypes.byref(_norm_c(norm)), _ptr(o_win),
                                  _ptr(lse_win), _ptr(o_rma), _ptr(lse_rma), _ptr(workspace),
                                  ws_bytes, _stream(stream))
    _check(s, "swa_rma_decode_attn")


def swa_rma_decode_attn_noalloc(st: LayerState, batch: int, q_win, q_rma, norm: Norm, o_win,
                                lse_win, o_rma, lse_rma, stream=None) -> None:
    s = lib().swa_rma_decode_attn_noalloc(ctypes.byref(_state_c(st)), int(batch), _ptr(q_win),
                                          _ptr(q_rma), ctypes.byref(_norm_c(norm)), _ptr(o_win),
                                          _ptr(lse_win), _ptr(o_rma), _ptr(lse_rma),
                                          _stream(stream))
    _check(s, "swa_rma_decode_attn_noalloc")


def rma_step_workspace_bytes(batch: int) -> int:
    return int(lib().rma_step_workspace_bytes(int(batch)))


def swa_rma_step(st: LayerState, batch: int, k_win, v_win, k_rma, v_rma, score, q_win, q_rma,
                 norm: Norm, o_win, lse_win, o_rma, lse_rma, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = lib().swa_rma_step(ctypes.byref(_state_c(st)), int(batch), _ptr(k_win), _ptr(v_win),
                           _ptr(k_rma), _ptr(v_rma), _ptr(score), _ptr(q_win), _ptr(q_rma),
                           ctypes.byref(_norm_c(norm)), _ptr(o_win), _ptr(lse_win), _ptr(o_rma),
                           _ptr(lse_rma), _ptr(workspace), ws_bytes, _stream(stream))
    _check(s, "swa_rma_step")


def rma_score(hidden, n_rows: int, ld_hidden: int, w1, w2, scores, ld_scores: int,
              stream=None) -> None:
    s = lib().rma_score(_ptr(hidden), int(n_rows), int(ld_hidden), _ptr(w1), _ptr(w2),
                        _ptr(scores), int(ld_scores), _stream(stream))
    _check(s, "rma_score")


def rma_commit_topk(st: LayerState, batch: int, keep_idx=None, stream=None) -> None:
    s = lib().rma_commit_topk(ctypes.byref(_state_c(st)), int(batch), _ptr(keep_idx),
                              _stream(stream))
    _check(s, "rma_commit_topk")


def rma_score_multi(jobs, n_rows: int, ld_hidden: int, ld_scores: int, stream=None) -> None:
    """jobs: a sequence of (hidden, w1, w2, scores) tensors, one rma_score call each."""
    arr = (_ScoreJobC * len(jobs))(*[_ScoreJobC(_ptr(h), _ptr(a), _ptr(b), _ptr(o))
                                     for h, a, b, o in jobs])
    s = lib().rma_score_multi(arr, len(jobs), int(n_rows), int(ld_hidden), int(ld_scores),
                              _stream(stream))
    _check(s, "rma_score_multi")


def rma_score_workspace_bytes(n_jobs: int, n_rows: int) -> int:
    return int(lib().rma_score_workspace_bytes(int(n_jobs), int(n_rows)))


def score_workspace(n_jobs: int, n_rows: int, device="cuda"):
    """A workspace of the size rma_score_multi_ws needs for these calls (or None)."""
    import torch

    n = rma_score_workspace_bytes(n_jobs, n_rows)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


def rma_score_multi_ws(jobs, n_rows: int, ld_hidden: int, ld_scores: int, workspace,
                       stream=None) -> None:
    """rma_score_multi with a workspace (``score_workspace``) for its small-call path."""
    arr = (_ScoreJobC * len(jobs))(*[_ScoreJobC(_ptr(h), _ptr(a), _ptr(b), _ptr(o))
                                     for h, a, b, o in jobs])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = lib().rma_score_multi_ws(arr, len(jobs), int(n_rows), int(ld_hidden), int(ld_scores),
                                 _ptr(workspace), ws_bytes, _stream(stream))
    _check(s, "rma_score_multi_ws")


def rma_commit_topk_multi(states, batch: int, keep_idx=None, stream=None) -> None:
    """states: a sequence of LayerState; keep_idx: None or one tensor (or None) per state."""
    arr = (_StateC * len(states))(*[_state_c(st) for st in states])
    keeps = None
    if keep_idx is not None:
        keeps = (_c_void_p * len(states))(*[_ptr(k) for k in keep_idx])
    s = lib().rma_commit_topk_multi(arr, len(states), int(batch), keeps, _stream(stream))
    _check(s, "rma_commit_topk_multi")


def decode_workspace(batch: int, device="cuda"):
    """A zero-filled workspace of the size swa_rma_decode_attn needs at this batch (or None)."""
    import torch

    n = rma_decode_workspace_bytes(batch)
    return None if n == 0 else torch.zeros(n, dtype=torch.uint8, device=device)


def step_workspace(batch: int, device="cuda"):
    """A zero-filled workspace for swa_rma_step at this batch; it stays valid across calls."""
    import torch

    return torch.zeros(rma_step_workspace_bytes(batch), dtype=torch.uint8, device=device)


def rma_prefill_workspace_bytes(batch: int, n_tokens: int) -> int:
    return int(lib().rma_prefill_workspace_bytes(int(batch), int(n_tokens)))


def prefill_workspace(batch: int, n_tokens: int, device="cuda"):
    """A workspace tensor of the size swa_rma_prefill needs."""
    import torch

    return torch.empty(rma_prefill_workspace_bytes(batch, n_tokens), dtype=torch.uint8,
                       device=device)


def swa_rma_prefill(st: LayerState, batch: int, n_tokens: int, k_win, v_win, k_rma, v_rma, score,
                    q_win, q_rma, norm: Norm, o_win, lse_win, o_rma, lse_rma, workspace,
                    stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size()
    s = lib().swa_rma_prefill(ctypes.byref(_state_c(st)), int(batch), int(n_tokens), _ptr(k_win),
                              _ptr(v_win), _ptr(k_rma), _ptr(v_rma), _ptr(score), _ptr(q_win),
                              _ptr(q_rma), ctypes.byref(_norm_c(norm)), _ptr(o_win),
                              _ptr(lse_win), _ptr(o_rma), _ptr(lse_rma), _ptr(workspace),
                              ws_bytes, _stream(stream))
    _check(s, "swa_rma_prefill")


# ---------------------------------------------------------------- FP8 state variant
def rma_layer_state_fp8_bytes(batch: int) -> int:
    return int(lib().rma_layer_state_fp8_bytes(int(batch)))


def swa_rma_append_fp8(st: LayerStateFP8, batch: int, k_win, v_win, k_rma, v_rma, score,
                       norm: Norm, stream=None) -> None:
    s = lib().swa_rma_append_fp8(ctypes.byref(_state_fp8_c(st)), int(batch), _ptr(k_win),
                                 _ptr(v_win), _ptr(k_rma), _ptr(v_rma), _ptr(score),
                                 ctypes.byref(_norm_c(norm)), _stream(stream))
    _check(s, "swa_rma_append_fp8")


def swa_rma_decode_attn_fp8(st: LayerStateFP8, batch: int, q_win, q_rma, norm: Norm, o_win,
                            lse_win, o_rma, lse_rma, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = lib().swa_rma_decode_attn_fp8(ctypes.byref(_state_fp8_c(st)), int(batch), _ptr(q_win),
                                      _ptr(q_rma), ctypes.byref(_norm_c(norm)), _ptr(o_win),
                                      _ptr(lse_win), _ptr(o_rma), _ptr(lse_rma), _ptr(workspace),
                                      ws_bytes, _stream(stream))
    _check(s, "swa_rma_decode_attn_fp8")


def rma_commit_topk_fp8(st: LayerStateFP8, batch: int, keep_idx=None, stream=None) -> None:
    s = lib().rma_commit_topk_fp8(ctypes.byref(_state_fp8_c(st)), int(batch), _ptr(keep_idx),
                                  _stream(stream))
    _check(s, "rma_commit_topk_fp8")


# ---------------------------------------------------------------- INT8 state variant
# The FP8 state's layout with signed 8-bit codes: LayerStateFP8 / alloc_layer_state_fp8
# hold it, rma_commit_topk_fp8 commits it.
def swa_rma_append_i8(st: LayerStateFP8, batch: int, k_win, v_win, k_rma, v_rma, score,
                      norm: Norm, stream=None) -> None:
    s = lib().swa_rma_append_i8(ctypes.byref(_state_fp8_c(st)), int(batch), _ptr(k_win),
                                _ptr(v_win), _ptr(k_rma), _ptr(v_rma), _ptr(score),
                                ctypes.byref(_norm_c(norm)), _stream(stream))
    _check(s, "swa_rma_append_i8")


def swa_rma_decode_attn_i8(st: LayerStateFP8, batch: int, q_win, q_rma, norm: Norm, o_win,
                           lse_win, o_rma, lse_rma, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = lib().swa_rma_decode_attn_i8(ctypes.byref(_state_fp8_c(st)), int(batch), _ptr(q_win),
                                     _ptr(q_rma), ctypes.byref(_norm_c(norm)), _ptr(o_win),
                                     _ptr(lse_win), _ptr(o_rma), _ptr(lse_rma), _ptr(workspace),
                                     ws_bytes, _stream(stream))
    _check(s, "swa_rma_decode_attn_i8")


# ---------------------------------------------------------------- GDN decode step (gdn.h)
GDN_K_HEADS, GDN_V_HEADS, GDN_HEAD_DIM, GDN_CONV, GDN_CONV_DIM = 16, 32, 128, 4, 8192
GDN_STATE_F16, GDN_STATE_F32 = 0, 1


@dataclass
class GdnState:
    """One GDN layer: S [B][32][128][128] (float16 or float32), conv bf16 [B][4][8192]."""

    S: object
    conv: object

    @property
    def dtype_code(self) -> int:
        import torch

        return GDN_STATE_F32 if self.S.dtype == torch.float32 else GDN_STATE_F16


@dataclass
class GdnParams:
    """conv_w f32 [8192][4], a_log f32 [32], dt_bias f32 [32] (device)."""

    conv_w: object
    a_log: object
    dt_bias: object


def alloc_gdn_state(batch: int, dtype: str = "f16", device="cuda") -> GdnState:
    """Zero state (the start of a stream)."""
    import torch

    dt = torch.float16 if dtype == "f16" else torch.float32
    return GdnState(torch.zeros(batch, GDN_V_HEADS, GDN_HEAD_DIM, GDN_HEAD_DIM, dtype=dt,
                                device=device),
                    torch.zeros(batch, GDN_CONV, GDN_CONV_DIM, dtype=torch.bfloat16, device=device))


def gdn_layer_state_bytes(batch: int, state_dtype: int) -> int:
    return int(lib().gdn_layer_state_bytes(int(batch), int(state_dtype)))


def gdn_decode_step(st: GdnState, batch: int, x, a, b, pos, prm: GdnParams, o,
                    stream=None) -> None:
    sc = _GdnStateC(_ptr(st.S), _ptr(st.conv))
    pc = _GdnParamsC(_ptr(prm.conv_w), _ptr(prm.a_log), _ptr(prm.dt_bias))
    s = lib().gdn_decode_step(ctypes.byref(sc), int(batch), st.dtype_code, _ptr(x), _ptr(a),
                              _ptr(b), _ptr(pos), ctypes.byref(pc), _ptr(o), _stream(stream))
    _check(s, "gdn_decode_step")


def gdn_prefill(st: GdnState, batch: int, n_tokens: int, x, a, b, pos, prm: GdnParams, o,
                stream=None) -> None:
    """n_tokens successive GDN decode steps per sequence in one call (see gdn.h)."""
    sc = _GdnStateC(_ptr(st.S), _ptr(st.conv))
    pc = _GdnParamsC(_ptr(prm.conv_w), _ptr(prm.a_log), _ptr(prm.dt_bias))
    s = lib().gdn_prefill(ctypes.byref(sc), int(batch), int(n_tokens), st.dtype_code, _ptr(x),
                          _ptr(a), _ptr(b), _ptr(pos), ctypes.byref(pc), _ptr(o), _stream(stream))
    _check(s, "gdn_prefill")
