"""HIP-graph capture of the per-token work of a decoding stream.

A decoding step of one SWA||RMA layer is append + decode (+ the split merge); every
256 tokens the block's candidates are scored and committed (neodrop.ai repost of the
QbitAI article on EdgeRock-4B, section "三段记忆，只记值得记的").  At batch 1 each of
these launches is short, so host-side launch cost matters as much as the kernels;
the pages' single-request decoding rates (fluxbbs.com page, section "吞吐：一张
80GB 卡跑 512 路长推理") come from a backend that replays captured graphs
(agentlenshq.com "rockmatrix-ai/EdgeRock", section "如何尝试").  ``StreamBlockGraph``
records one whole 256-token block for every layer (256 x L steps, then the
scores of every layer (one launch, or two for small blocks) and the commits of every
layer in one launch) into a
single HIP graph through torch's graph capture, and replays it per block.  A step is one ``swa_rma_step`` launch (append and
attention fused; the split merge follows where the key range is split) or, with
``fused=False``, the separate append and decode launches.

The graph reads its inputs from static buffers owned by this object (fill them
before each replay: ``rec``, ``q_win``, ``q_rma``, ``hidden``) and writes every
token's outputs into ``o_win``/``lse_win``/``o_rma``/``lse_rma``.  All state
(positions, counts, pending rows) lives on the device, so the same graph serves
every block.  The library's entry points allocate nothing, synchronise nothing
and record no memset, so they can be captured; run each entry point once on the
device (eagerly) before ``capture()``, so its code object is loaded.
"""

from __future__ import annotations

import ctypes

from . import (BLOCK, HEAD_DIM, HIDDEN, KV_GROUPS, Q_HEADS, LayerState, Norm, _norm_c, _ptr,
               _ScoreJobC, _state_c, _StateC, decode_workspace, lib, score_workspace,
               step_workspace)

RMA_MAX_JOBS = 16  # calls one *_multi entry point takes at most (rma.h)

RECORD_NAMES = ("k_win", "v_win", "k_rma", "v_rma")


class StreamBlockGraph:
    """One block of ``tokens`` decoding steps in all layers, captured as a HIP graph.

    states/norms: one LayerState / Norm per layer; scorer: one (w1, w2) pair per layer.
    Static inputs (device tensors, filled by the caller before ``replay``):
      rec[name]  [L][tokens][B][4][256] BF16 (raw window / candidate records)
      q_win, q_rma  [L][tokens][B][16][256] BF16
      hidden     [L][B][256][2560] BF16 (the block's scorer input; used when ``commit``)
    Outputs: o_win, o_rma [L][tokens][B][16][256] BF16; lse_win, lse_rma [L][tokens][B][16].
    With commit=True the last token must end a block (the pending block is full after
    it), as in a stream that starts on a block boundary: a whole block of 256 tokens,
    or fewer tokens that finish one (a single block-end token, say).
    """

    def __init__(self, states: list[LayerState], norms: list[Norm], scorer, batch: int,
                 tokens: int = BLOCK, commit: bool = True, fused: bool = True, device="cuda"):
        import torch

        if commit and not 1 <= tokens <= BLOCK:
            raise ValueError("a graph that commits ends one pending block: 1..256 tokens")
        L = len(states)
        self.L, self.B, self.T, self.commit = L, batch, tokens, commit
        bf = torch.bfloat16
        self.rec = {nm: torch.zeros(L, tokens, batch, KV_GROUPS, HEAD_DIM, dtype=bf, device=device)
                    for nm in RECORD_NAMES}
        self.q_win = torch.zeros(L, tokens, batch, Q_HEADS, HEAD_DIM, dtype=bf, device=device)
        self.q_rma = torch.zeros_like(self.q_win)
        self.hidden = (torch.zeros(L, batch, BLOCK, HIDDEN, dtype=bf, device=device)
                       if commit else None)
        self.o_win = torch.zeros(L, tokens, batch, Q_HEADS, HEAD_DIM, dtype=bf, device=device)
        self.o_rma = torch.zeros_like(self.o_win)
        self.lse_win = torch.zeros(L, tokens, batch, Q_HEADS, device=device)
        self.lse_rma = torch.zeros_like(self.lse_win)
        self.fused = fused
        # the fused step's workspace holds counters that start at zero and are back
        # at zero after every step, so one zero fill serves every replay
        self.workspace = step_workspace(batch, device) if fused else decode_workspace(batch, device)
        # stage-1 scorer results of every layer's block (small calls spread the 256
        # columns of a row tile over 8 CUs and sum them in a second launch)
        self.score_ws = (score_workspace(min(L, RMA_MAX_JOBS), batch * BLOCK, device)
                         if commit else None)
        self._states, self._norms, self._scorer = states, norms, scorer
        # the ctypes structs must outlive the graph: kernels read them at launch only,
        # but keep them with the object for the record
        self._st_c = [_state_c(s) for s in states]
        self._nm_c = [_norm_c(n) for n in norms]
        self.graph = None

    def _launch_all(self, stream: int) -> None:
        lb = lib()
        B, T, L = self.B, self.T, self.L
        rb = KV_GROUPS * HEAD_DIM * 2 * B  # bytes of one token's record, all sequences
        qb = Q_HEADS * HEAD_DIM * 2 * B
        lb_ = Q_HEADS * 4 * B
        ws = _ptr(self.workspace)
        wsn = 0 if self.workspace is None else self.workspace.numel()
        rp = {nm: self.rec[nm].data_ptr() for nm in RECORD_NAMES}
        for t in range(T):
            for l in range(L):
                off = (l * T + t)
                r = [rp[nm] + off * rb for nm in RECORD_NAMES]
                st = ctypes.byref(self._st_c[l])
                nm = ctypes.byref(self._nm_c[l])
                if self.fused:
                    s = lb.swa_rma_step(
                        st, B, r[0], r[1], r[2], r[3], None, self.q_win.data_ptr() + off * qb,
                        self.q_rma.data_ptr() + off * qb, nm, self.o_win.data_ptr() + off * qb,
                        self.lse_win.data_ptr() + off * lb_, self.o_rma.data_ptr() + off * qb,
                        self.lse_rma.data_ptr() + off * lb_, ws, wsn, stream)
                    if s != 0:
                        raise RuntimeError(f"swa_rma_step failed during capture (status {s})")
                    continue
                s = lb.swa_rma_append(st, B, r[0], r[1], r[2], r[3], None, nm, stream)
                if s != 0:
                    raise RuntimeError(f"swa_rma_append failed during capture (status {s})")
                s = lb.swa_rma_decode_attn(
                    st, B, self.q_win.data_ptr() + off * qb, self.q_rma.data_ptr() + off * qb,
                    nm, self.o_win.data_ptr() + off * qb, self.lse_win.data_ptr() + off * lb_,
                    self.o_rma.data_ptr() + off * qb, self.lse_rma.data_ptr() + off * lb_, ws,
                    wsn, stream)
                if s != 0:
                    raise RuntimeError(f"swa_rma_decode_attn failed during capture (status {s})")
        if self.commit:
            # every layer's scores in one launch, then every layer's commit in one
            hb = HIDDEN * 2 * B * BLOCK
            for l0 in range(0, L, RMA_MAX_JOBS):
                ls = range(l0, min(L, l0 + RMA_MAX_JOBS))
                jobs = (_ScoreJobC * len(ls))(*[
                    _ScoreJobC(self.hidden.data_ptr() + l * hb, _ptr(self._scorer[l][0]),
                               _ptr(self._scorer[l][1]), _ptr(self._states[l].pend_score))
                    for l in ls])
                sws = _ptr(self.score_ws)
                swn = 0 if self.score_ws is None else self.score_ws.numel()
                s = lb.rma_score_multi_ws(jobs, len(ls), B * BLOCK, HIDDEN, KV_GROUPS, sws,
                                          swn, stream)
                if s != 0:
                    raise RuntimeError(f"rma_score_multi_ws failed during capture (status {s})")
                sts = (_StateC * len(ls))(*[self._st_c[l] for l in ls])
                s = lb.rma_commit_topk_multi(sts, len(ls), B, None, stream)
                if s != 0:
                    raise RuntimeError(f"rma_commit_topk_multi failed during capture (status {s})")

    def capture(self) -> "StreamBlockGraph":
        """Record the block (nothing runs while recording)."""
        import torch

        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._launch_all(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        return self

    def replay(self) -> None:
        """Run the captured block on the current stream."""
        if self.graph is None:
            raise RuntimeError("capture() the block before replaying it")
        self.graph.replay()
