"""A captured 256-token block (append + decode in every layer, then score + commit)
replayed as a HIP graph gives exactly what the same calls give eagerly.

The eager calls are themselves checked against the oracle elsewhere (the long-stream
and workload tests); here every replay is compared bit for bit with the eager run,
several times, with eager device work and synchronisations between the replays.
"""

import numpy as np
import pytest
import torch

import swa_memory_anchor_amd as R
import synth
from swa_memory_anchor_amd.graph import RECORD_NAMES, StreamBlockGraph
from synth.core import normal_bf16_torch_

from gpu_util import DEV, bits_host

pytestmark = pytest.mark.gpu

T = R.BLOCK


def _fill_state(st: R.LayerState, tag, counts):
    for nm in ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        normal_bf16_torch_(getattr(st, nm), synth.stream_key(tag, nm))
    B = len(counts)
    for b, (nb, pos) in enumerate(counts):
        st.n_bank[b], st.n_pend[b], st.pos[b] = nb, 0, pos
        for g in range(R.KV_GROUPS):
            st.bank_src[b, g] = torch.from_numpy(synth.distinct_ints_np(
                synth.stream_key(tag, "src", b, g), R.BANK, 0, 10**6).astype(np.int32))
    score = synth.normal_f32_np(synth.stream_key(tag, "bank_score"), (B, R.KV_GROUPS, R.BANK))
    st.bank_score.copy_(torch.from_numpy(score))


def _clone(st: R.LayerState) -> R.LayerState:
    return R.LayerState(**{k: v.clone() for k, v in st.__dict__.items()})


def _assign(dst: R.LayerState, src: R.LayerState):
    for k, v in src.__dict__.items():
        getattr(dst, k).copy_(v)


def _eager(states, norms, scorer, g: StreamBlockGraph):
    """The same calls as the graph, one by one, into outputs of the same layout."""
    L, B = len(states), g.B
    outs = [torch.empty_like(x) for x in (g.o_win, g.lse_win, g.o_rma, g.lse_rma)]
    ws = R.decode_workspace(B)
    for t in range(T):
        for l in range(L):
            R.swa_rma_append(states[l], B, *[g.rec[nm][l, t] for nm in RECORD_NAMES], None,
                             norms[l])
            R.swa_rma_decode_attn(states[l], B, g.q_win[l, t], g.q_rma[l, t], norms[l],
                                  outs[0][l, t], outs[1][l, t], outs[2][l, t], outs[3][l, t], ws)
    for l in range(L):
        R.rma_score(g.hidden[l], B * T, R.HIDDEN, scorer[l][0], scorer[l][1],
                    states[l].pend_score, R.KV_GROUPS)
        R.rma_commit_topk(states[l], B)
    return outs


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("B", [1, 3])
def test_block_graph_replays_match_eager(B, fused):
    """The eager reference is always the separate append + decode; the fused step's
    graph must match it bit for bit too."""
    print(f"case: block graph B={B} fused={fused}", flush=True)
    tag = f"graph_b{B}"
    L = 2
    counts = [(1024, 65535), (300, 767), (0, -1)][:B]
    init = []
    for l in range(L):
        st = R.alloc_layer_state(B, DEV)
        _fill_state(st, (tag, l), counts)
        init.append(st)
    norms = []
    scorer = []
    for l in range(L):
        gs = [torch.from_numpy(synth.normal_f32_np(synth.stream_key(tag, l, nm), (256,), 1.0, 0.1))
              .to(DEV) for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma")]
        norms.append(R.Norm(*gs))
        w1 = synth.normal_f32_np(synth.stream_key(tag, l, "w1"), (R.HIDDEN, R.SCORER_MID), 0, 0.02)
        w2 = synth.normal_f32_np(synth.stream_key(tag, l, "w2"), (R.SCORER_MID, 4), 0, 0.02)
        scorer.append((torch.from_numpy(w1).to(DEV), torch.from_numpy(w2).to(DEV)))

    live = [_clone(s) for s in init]
    eager_states = [_clone(s) for s in init]
    g = StreamBlockGraph(live, norms, scorer, B, fused=fused)
    for nm in RECORD_NAMES:
        normal_bf16_torch_(g.rec[nm], synth.stream_key(tag, "rec", nm))
    normal_bf16_torch_(g.q_win, synth.stream_key(tag, "qw"))
    normal_bf16_torch_(g.q_rma, synth.stream_key(tag, "qr"))
    normal_bf16_torch_(g.hidden, synth.stream_key(tag, "hid"))
    ref = _eager(eager_states, norms, scorer, g)  # also loads every kernel before capture
    if fused:  # load the fused step's kernel too, on a throwaway copy of the state
        scratch = _clone(init[0])
        o = [torch.empty_like(x[0, 0]) for x in (g.o_win, g.lse_win, g.o_rma, g.lse_rma)]
        R.swa_rma_step(scratch, B, *[g.rec[nm][0, 0] for nm in RECORD_NAMES], None,
                       g.q_win[0, 0], g.q_rma[0, 0], norms[0], *o, R.step_workspace(B))
    torch.cuda.synchronize()
    g.capture()
    ref_bits = [bits_host(ref[0]), ref[1].cpu().numpy(), bits_host(ref[2]), ref[3].cpu().numpy()]
    ref_state = {k: v.cpu() for k, v in
                 ((f"{l}.{k}", v) for l in range(L) for k, v in eager_states[l].__dict__.items())}

    for rep in range(3):
        for l in range(L):
            _assign(live[l], init[l])  # eager device work between replays
        for x in (g.o_win, g.o_rma, g.lse_win, g.lse_rma):
            x.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bits_host(g.o_win), g.lse_win.cpu().numpy(), bits_host(g.o_rma),
               g.lse_rma.cpu().numpy()]
        for a, b_, nm in zip(got, ref_bits, ("o_win", "lse_win", "o_rma", "lse_rma")):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b_.view(np.uint32) if b_.dtype == np.float32 else b_), (rep, nm)
        for l in range(L):
            for k, v in live[l].__dict__.items():
                assert torch.equal(v.cpu().view(torch.int16) if v.dtype == torch.bfloat16 else
                                   v.cpu(),
                                   ref_state[f"{l}.{k}"].view(torch.int16)
                                   if v.dtype == torch.bfloat16 else ref_state[f"{l}.{k}"]), \
                    (rep, l, k)
        # the replay advanced every sequence by one block and committed it
        assert live[0].pos.cpu().tolist() == [p + T for _, p in counts]
        assert live[0].n_pend.cpu().tolist() == [0] * B


def test_block_end_token_graph_matches_eager():
    """A one-token graph that ends a block (step, then the block's scores from its 256
    hidden rows per sequence, then the commit) replays bit for bit as the same calls
    made eagerly with the one-launch scorer."""
    B, L = 2, 2
    tag = "graph_end"
    print(f"case: block-end token graph B={B}", flush=True)
    counts = [(1024, 65790), (300, 766)]  # 255 pending rows each: the next token ends a block
    init = []
    for l in range(L):
        st = R.alloc_layer_state(B, DEV)
        _fill_state(st, (tag, l), counts)
        for b, (_, pos) in enumerate(counts):
            st.n_pend[b] = T - 1
            st.pend_src[b] = torch.arange(pos - (T - 2), pos + 2, dtype=torch.int32)
        init.append(st)
    norms, scorer = [], []
    for l in range(L):
        gs = [torch.from_numpy(synth.normal_f32_np(synth.stream_key(tag, l, nm), (256,), 1.0, 0.1))
              .to(DEV) for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma")]
        norms.append(R.Norm(*gs))
        w1 = synth.normal_f32_np(synth.stream_key(tag, l, "w1"), (R.HIDDEN, R.SCORER_MID), 0, 0.02)
        w2 = synth.normal_f32_np(synth.stream_key(tag, l, "w2"), (R.SCORER_MID, 4), 0, 0.02)
        scorer.append((torch.from_numpy(w1).to(DEV), torch.from_numpy(w2).to(DEV)))
    live = [_clone(s) for s in init]
    eager_states = [_clone(s) for s in init]
    g = StreamBlockGraph(live, norms, scorer, B, tokens=1, commit=True)
    for nm in RECORD_NAMES:
        normal_bf16_torch_(g.rec[nm], synth.stream_key(tag, "rec", nm))
    normal_bf16_torch_(g.q_win, synth.stream_key(tag, "qw"))
    normal_bf16_torch_(g.q_rma, synth.stream_key(tag, "qr"))
    normal_bf16_torch_(g.hidden, synth.stream_key(tag, "hid"))

    ref = [torch.empty_like(x) for x in (g.o_win, g.lse_win, g.o_rma, g.lse_rma)]
    ws = R.step_workspace(B)
    for l in range(L):
        R.swa_rma_step(eager_states[l], B, *[g.rec[nm][l, 0] for nm in RECORD_NAMES], None,
                       g.q_win[l, 0], g.q_rma[l, 0], norms[l], ref[0][l, 0], ref[1][l, 0],
                       ref[2][l, 0], ref[3][l, 0], ws)
    for l in range(L):
        R.rma_score(g.hidden[l], B * T, R.HIDDEN, scorer[l][0], scorer[l][1],
                    eager_states[l].pend_score, R.KV_GROUPS)
        R.rma_commit_topk(eager_states[l], B)
    R.rma_score_multi_ws([(g.hidden[0], scorer[0][0], scorer[0][1], torch.empty(B * T, 4, device=DEV))],
                         B * T, R.HIDDEN, R.KV_GROUPS, R.score_workspace(1, B * T, DEV))
    torch.cuda.synchronize()
    g.capture()
    ref_bits = [bits_host(ref[0]), ref[1].cpu().numpy(), bits_host(ref[2]), ref[3].cpu().numpy()]
    for rep in range(3):
        for l in range(L):
            _assign(live[l], init[l])
        for x in (g.o_win, g.o_rma, g.lse_win, g.lse_rma):
            x.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bits_host(g.o_win), g.lse_win.cpu().numpy(), bits_host(g.o_rma),
               g.lse_rma.cpu().numpy()]
        for a, b_, nm in zip(got, ref_bits, ("o_win", "lse_win", "o_rma", "lse_rma")):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b_.view(np.uint32) if b_.dtype == np.float32 else b_), (rep, nm)
        for l in range(L):
            for k, v in live[l].__dict__.items():
                e = eager_states[l].__dict__[k]
                if v.dtype == torch.bfloat16:
                    v, e = v.view(torch.int16), e.view(torch.int16)
                elif v.dtype == torch.float32:
                    v, e = v.view(torch.int32), e.view(torch.int32)
                assert torch.equal(v, e), (rep, l, k)
        assert live[0].n_pend.cpu().tolist() == [0] * B
        assert live[0].pos.cpu().tolist() == [p + 1 for _, p in counts]
