"""swa_rma_decode_attn_noalloc through the C ABI: the same bits as swa_rma_decode_attn
with a caller workspace, on consecutive calls of shrinking size (the second call
finds the first one's partials in the library's array), and the oracle's results."""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import swa_memory_anchor_amd as R
import synth

from gpu_util import DEV, assert_attn_close, bf16_dev, bits_host, norm_dev, upload

pytestmark = pytest.mark.gpu


def _state(tag, B):
    st = O.new_layer_state(B)
    for nm in ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(synth.stream_key(tag, nm), a.size).reshape(a.shape)
    rng = synth.rng_np(synth.stream_key(tag, "counts"))
    st.n_bank[:] = rng.integers(0, 1025, B)
    st.n_pend[:] = rng.integers(0, 257, B)
    st.pos[:] = rng.integers(-1, 3000, B)
    st.n_bank[0], st.n_pend[0], st.pos[0] = 1024, 256, 70000
    return st


def _gains(tag):
    return {nm: synth.normal_f32_np(synth.stream_key(tag, nm), (256,), 1.0, 0.1)
            for nm in ("gq_win", "gk_win", "gq_rma", "gk_rma")}


def _outs(B, fill):
    return [torch.full((B, 16, 256), fill, dtype=torch.bfloat16, device=DEV),
            torch.full((B, 16), fill, device=DEV),
            torch.full((B, 16, 256), fill, dtype=torch.bfloat16, device=DEV),
            torch.full((B, 16), fill, device=DEV)]


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("batches", [(37, 3), (63, 8, 1), (64, 2)])
def test_noalloc_decode_matches_workspace_decode(batches):
    lib = R.lib()
    stream = torch.cuda.current_stream().cuda_stream
    for i, B in enumerate(batches):
        print(f"case: noalloc call {i} batch={B} splits={R.rma_decode_splits(B)}", flush=True)
        tag = f"noalloc_{B}_{i}"
        st = _state(tag, B)
        g = _gains(tag)
        q = synth.normal_bf16_np(synth.stream_key(tag, "q"), B * 4096).reshape(B, 16, 256)
        dst = upload(st)
        nm = norm_dev(g)
        qd = bf16_dev(q)
        ref_out = _outs(B, 5.0)
        R.swa_rma_decode_attn(dst, B, qd, qd, nm, *ref_out, R.decode_workspace(B))
        got = _outs(B, -3.0)
        rc = lib.swa_rma_decode_attn_noalloc(
            ctypes.byref(R._state_c(dst)), B, qd.data_ptr(), qd.data_ptr(),
            ctypes.byref(R._norm_c(nm)), got[0].data_ptr(), got[1].data_ptr(),
            got[2].data_ptr(), got[3].data_ptr(), stream)
        assert rc == 0, R.rma_status_str(rc)
        torch.cuda.synchronize()
        for x, y in zip(got, ref_out):
            assert _same(x, y), f"batch {B}: differs from the workspace call"
        ref = O.decode(st, q, q, g["gq_win"], g["gq_rma"], 1e-6, 1e7)
        assert_attn_close(bits_host(got[0]), got[1].cpu().numpy(), ref[0], ref[1],
                          what=f"noalloc B={B} window")
        assert_attn_close(bits_host(got[2]), got[3].cpu().numpy(), ref[2], ref[3],
                          what=f"noalloc B={B} anchor")


def test_noalloc_rejects_bad_arguments():
    lib = R.lib()
    assert lib.swa_rma_decode_attn_noalloc(None, 4, 16, 16, None, 16, 16, 16, 16, None) == 1
    st = R._StateC(*([16] * 13))
    nm = R._NormC(16, 16, 16, 16, 1e-6, 1e7)
    assert lib.swa_rma_decode_attn_noalloc(ctypes.byref(st), 0, 16, 16, ctypes.byref(nm), 16, 16,
                                           16, 16, None) == 1
    # a misaligned query is refused before anything is launched
    assert lib.swa_rma_decode_attn_noalloc(ctypes.byref(st), 4, 18, 16, ctypes.byref(nm), 16, 16,
                                           16, 16, None) == 2
