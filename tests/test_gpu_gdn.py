"""GPU parity of the GDN decode step (gdn_decode_step) against oracle.gdn_ref.

Bars (derived in the tests' helpers): the convolution ring is bit-exact (a copy of
the BF16 input); the new recurrent matrix is within one unit in the last place of
its storage precision plus the FP32 arithmetic's share; the BF16 output is
within 1e-2 of its row's largest magnitude.
"""

import numpy as np
import pytest
import torch

from oracle import gdn_ref as G
import swa_memory_anchor_amd as R
import synth
from synth import core as C
from synth import workloads as W

import oracle_pool
from gdn_check import O_TOL, out_rel, state_bound, state_err_ratio
from gpu_util import DEV, bits_host, f32_dev, i32_dev

pytestmark = pytest.mark.gpu



def _params(tag):
    rng = synth.rng_np(synth.stream_key(tag, "params"))
    return {"conv_w": (rng.standard_normal((8192, 4)) * 0.5).astype(np.float32),
            "a_log": np.log(rng.uniform(1, 16, 32)).astype(np.float32),
            "dt_bias": rng.standard_normal(32).astype(np.float32)}


def _params_dev(p):
    return R.GdnParams(f32_dev(p["conv_w"]), f32_dev(p["a_log"]), f32_dev(p["dt_bias"]))


def _state(tag, B, dtype, zero=False):
    st = G.new_state(B, dtype)
    if not zero:
        dt = np.float16 if dtype == "f16" else np.float32
        st.S[...] = C.scaled_normal_np(synth.stream_key(tag, "S"), st.S.size,
                                       dtype=dt).reshape(st.S.shape)
        st.conv[...] = synth.normal_bf16_np(synth.stream_key(tag, "conv"),
                                            st.conv.size).reshape(st.conv.shape)
    return st


def _upload(st: G.GdnState) -> R.GdnState:
    S = torch.from_numpy(st.S.copy()).to(DEV)
    conv = torch.from_numpy(st.conv.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return R.GdnState(S, conv)


def assert_state_close(got, ref, what=""):
    """New matrices against the oracle's (both stored in the same precision), within
    the one-step bound of gdn_check (one unit in the last place of the reference
    element plus 2^-18 of the head's largest magnitude)."""
    ratio = state_err_ratio(got, ref)
    print(f"{what}: {int((got != ref).sum())} of {got.size} entries differ; max err/bound "
          f"{ratio:.3f}")
    assert ratio <= 1.0, f"{what}: out of bound ({ratio:.3f})"


def assert_out_close(got_bits, ref, what=""):
    rel = out_rel(synth.bf16_bits_to_f32_np(got_bits), ref)
    print(f"{what}: rows={rel.size} out max={rel.max():.3e} median={np.median(rel):.3e}")
    assert np.all(np.isfinite(rel)) and rel.max() <= O_TOL, what


def _step(dev_state, B, x, a, b, pos, prm_dev):
    o = torch.full((B, 32, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    R.gdn_decode_step(dev_state, B, x, a, b, pos, prm_dev, o)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("B", [6, 20])  # a narrow (4 slices per head) and a wide launch
def test_gdn_step_matches_oracle(dtype, B):
    print(f"case: gdn step B={B} dtype={dtype}", flush=True)
    tag = f"gdn_step_{B}_{dtype}"
    st = _state(tag, B, dtype)
    prm = _params(tag)
    x = synth.normal_bf16_np(synth.stream_key(tag, "x"), B * 8192).reshape(B, 8192)
    rng = synth.rng_np(synth.stream_key(tag, "ab"))
    a = (rng.standard_normal((B, 32)) * 2).astype(np.float32)
    b = (rng.standard_normal((B, 32)) * 2).astype(np.float32)
    pos = np.array([0, 1, 2, 3, 4, 70001] * 4, np.int32)[:B]
    dev = _upload(st)
    o = _step(dev, B, torch.from_numpy(x.view(np.int16)).to(DEV), f32_dev(a), f32_dev(b),
              i32_dev(pos), _params_dev(prm))
    ref_o = G.decode_step(st, x, a, b, prm["conv_w"], prm["a_log"], prm["dt_bias"], pos)
    assert np.array_equal(bits_host(dev.conv), st.conv), "convolution ring"
    assert_state_close(dev.S.cpu().numpy(), st.S, what="S")
    assert_out_close(bits_host(o), ref_o, what="o")


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_gdn_stream_from_zero_state(dtype):
    """Two sequences stream 40 tokens from an empty state (positions 0..39 and 7..46).

    Every step is checked on its own: the oracle takes the GPU's state from before
    the step and must agree with the GPU's new state and output within the
    one-step bars.  The two independent trajectories are then compared per head in
    the Frobenius norm: a step's map S -> alpha (I - beta k k^T) S is non-expansive
    (0 < alpha <= 1, 0 <= beta <= 1, |k| = 1), so rounding differences can add up
    but not grow, and after T steps the distance is at most T times the norm of a
    step's bound."""
    B, T = 2, 40
    print(f"case: gdn stream B={B} T={T} dtype={dtype}", flush=True)
    tag = f"gdn_stream_{dtype}"
    ref = _state(tag, B, dtype, zero=True)
    prm = _params(tag)
    dev = _upload(ref)
    pd = _params_dev(prm)
    rng = synth.rng_np(synth.stream_key(tag, "ab"))
    for t in range(T):
        x = synth.normal_bf16_np(synth.stream_key(tag, "x", t), B * 8192).reshape(B, 8192)
        a = rng.standard_normal((B, 32)).astype(np.float32)
        b = rng.standard_normal((B, 32)).astype(np.float32)
        pos = np.array([t, t + 7], np.int32)
        before = G.GdnState(dev.S.cpu().numpy(), bits_host(dev.conv).copy())
        o = _step(dev, B, torch.from_numpy(x.view(np.int16)).to(DEV), f32_dev(a), f32_dev(b),
                  i32_dev(pos), pd)
        one_o = G.decode_step(before, x, a, b, prm["conv_w"], prm["a_log"], prm["dt_bias"], pos)
        G.decode_step(ref, x, a, b, prm["conv_w"], prm["a_log"], prm["dt_bias"], pos)
        assert np.array_equal(bits_host(dev.conv), before.conv), f"ring t={t}"
        got = dev.S.cpu().numpy()
        if t in (0, 1, 3, 20, T - 1):
            assert_state_close(got, before.S, what=f"S t={t}")
            assert_out_close(bits_host(o), one_o, what=f"o t={t}")
        else:
            err = np.abs(got.astype(np.float64) - before.S.astype(np.float64))
            assert np.all(err <= state_bound(before.S, whole=True)), f"S t={t}"
    got = dev.S.cpu().numpy().astype(np.float64)
    for s_ in range(B):
        for h in range(32):
            d = np.linalg.norm(got[s_, h] - ref.S[s_, h].astype(np.float64))
            lim = T * np.linalg.norm(np.broadcast_to(state_bound(ref.S[s_, h], whole=True), (128, 128)))
            assert d <= lim, (s_, h, d, lim)
    print(f"trajectories: max head distance / bound "
          f"{max(np.linalg.norm(got[s_, h] - ref.S[s_, h]) / (T * np.linalg.norm(np.broadcast_to(state_bound(ref.S[s_, h], whole=True), (128, 128)))) for s_ in range(B) for h in range(32)):.3f}")


def _full_size(wl, layers):
    """One step of `layers` layers at the workload's full size; every (sequence, layer)
    unit (all 32 heads: new matrices, outputs, ring) against the oracle, in worker
    processes that regenerate each unit's inputs from the seeds."""
    B = wl.batch
    print(f"case: {wl.name} B={B} layers={layers}", flush=True)
    dt = torch.float16 if wl.extra["state"] == "f16" else torch.float32
    outs, states = [], []
    for layer in range(layers):
        st = R.GdnState(torch.empty(B, 32, 128, 128, dtype=dt, device=DEV),
                        torch.empty(B, 4, 8192, dtype=torch.bfloat16, device=DEV))
        W.gdn_state_torch_(wl, layer, st.S)
        W.gdn_conv_torch_(wl, layer, st.conv)
        x = torch.empty(B, 8192, dtype=torch.bfloat16, device=DEV)
        W.gdn_x_torch_(wl, layer, x)
        a, b = W.gdn_gate_inputs(wl, layer)
        p = W.gdn_params(wl, layer)
        pos = torch.full((B,), wl.position, dtype=torch.int32, device=DEV)
        o = torch.empty(B, 32, 128, dtype=torch.bfloat16, device=DEV)
        R.gdn_decode_step(st, B, x, f32_dev(a), f32_dev(b), pos, _params_dev(p), o)
        states.append(st)
        outs.append(o)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.isfinite(o.float()).all()
    print("step done; checking every unit", flush=True)
    tasks = []
    for layer in range(layers):
        S = states[layer].S.cpu().numpy()
        o = bits_host(outs[layer])
        ring = bits_host(states[layer].conv)
        tasks += [(wl.name, layer, b_, S[b_], o[b_], ring[b_]) for b_ in range(B)]
    res = oracle_pool.all_gdn_unit_errors(tasks)
    worst_s = max(r[2] for r in res)
    worst_o = max(r[3] for r in res)
    print(f"{wl.name}: all {len(res)} units ({32 * len(res)} heads) against the oracle; "
          f"max state err/bound {worst_s:.3f}, worst output row error {worst_o:.3e}", flush=True)
    assert all(r[4] for r in res), "convolution ring differs"
    assert worst_s <= 1.0 and worst_o <= O_TOL


def test_gdn_decode_b512_every_unit():
    _full_size(W.GDN_DECODE_B512, 2)


def test_gdn_decode_b1_every_head():
    _full_size(W.GDN_DECODE_B1, 1)


def _same_bits(x, y, what):
    """Bit equality with a short message: count of differing elements and the first."""
    ne = (x != y).reshape(-1)
    n = int(ne.sum())
    if n:
        i = int(torch.nonzero(ne)[0])
        raise AssertionError(f"{what}: {n} of {ne.numel()} elements differ; first at flat index "
                             f"{i}: {int(x.reshape(-1)[i])} vs {int(y.reshape(-1)[i])}")


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("B", [6, 20])  # the narrow and the wide column slices
def test_gdn_prefill_equals_decode_steps(dtype, B):
    """gdn_prefill(T tokens) leaves the matrices, the ring and the outputs exactly as T
    gdn_decode_step calls do (chunks of 1, 3, 16 and 37 tokens; positions 0 (empty ring),
    1 and 70001); the first token's output also against the oracle."""
    tag = f"gdn_prefill_{B}_{dtype}"
    prm = _params(tag)
    pd = _params_dev(prm)
    for T in (1, 3, 16, 37):
        print(f"case: gdn prefill B={B} dtype={dtype} T={T}", flush=True)
        st = _state(f"{tag}_{T}", B, dtype)
        p0 = np.array([0, 1, 70001] * 8, np.int32)[:B]
        x = synth.normal_bf16_np(synth.stream_key(tag, "x", T), B * T * 8192).reshape(B, T, 8192)
        rng = synth.rng_np(synth.stream_key(tag, "ab", T))
        a = (rng.standard_normal((B, T, 32)) * 2).astype(np.float32)
        b = (rng.standard_normal((B, T, 32)) * 2).astype(np.float32)
        chunk, steps = _upload(st), _upload(st)
        o_chunk = torch.full((B, T, 32, 128), 7.0, dtype=torch.bfloat16, device=DEV)
        R.gdn_prefill(chunk, B, T, torch.from_numpy(x.view(np.int16)).to(DEV), f32_dev(a),
                      f32_dev(b), i32_dev(p0), pd, o_chunk)
        o_steps = []
        for i in range(T):
            xi = torch.from_numpy(np.ascontiguousarray(x[:, i]).view(np.int16)).to(DEV)
            o_steps.append(_step(steps, B, xi, f32_dev(np.ascontiguousarray(a[:, i])),
                                 f32_dev(np.ascontiguousarray(b[:, i])), i32_dev(p0 + i), pd))
        torch.cuda.synchronize()
        ib = torch.int16 if dtype == "f16" else torch.int32
        _same_bits(chunk.S.view(ib), steps.S.view(ib), "S")
        _same_bits(chunk.conv.view(torch.int16), steps.conv.view(torch.int16), "ring")
        for i in range(T):
            _same_bits(o_chunk[:, i].view(torch.int16), o_steps[i].view(torch.int16), f"o[{i}]")
        # the first token against the oracle (the state before it is known exactly)
        ref = G.GdnState(st.S.copy(), st.conv.copy())
        ref_o = G.decode_step(ref, x[:, 0], a[:, 0], b[:, 0], prm["conv_w"], prm["a_log"],
                              prm["dt_bias"], p0)
        assert_out_close(bits_host(o_chunk[:, 0]), ref_o, what=f"o T={T} token 0")


def test_gdn_prefill_b512_full_size():
    """gdn_prefill in the benchmark's call (gdn_prefill_b512, layer 0: 512 sequences x
    256 tokens, FP16 matrices, one 128-column slice per head): the matrices, the ring
    and all 512 x 256 outputs equal those of 256 gdn_decode_step calls bit for bit.
    Three sampled sequences are then checked against the oracle: one-step checks at
    tokens 0, 128 and 255 (the oracle starts from the GPU's state before the token),
    and the whole 256-token trajectory from the same initial state, whose distance
    per head is at most 256 times the norm of a step's bound (the step map is
    non-expansive; see test_gdn_stream_from_zero_state)."""
    wl = W.GDN_PREFILL_B512
    B, T, layer = wl.batch, wl.extra["chunk"], 0
    print(f"case: {wl.name} full size B={B} T={T}", flush=True)
    chunk = R.GdnState(torch.empty(B, 32, 128, 128, dtype=torch.float16, device=DEV),
                       torch.empty(B, 4, 8192, dtype=torch.bfloat16, device=DEV))
    W.gdn_state_torch_(wl, layer, chunk.S)
    W.gdn_conv_torch_(wl, layer, chunk.conv)
    steps = R.GdnState(chunk.S.clone(), chunk.conv.clone())
    x = torch.empty(B, T, 8192, dtype=torch.bfloat16, device=DEV)
    W.gdn_chunk_x_torch_(wl, layer, x)
    a_h, b_h = W.gdn_chunk_gates(wl, layer, T)
    a, b = f32_dev(a_h), f32_dev(b_h)
    prm = W.gdn_params(wl, layer)
    pd = _params_dev(prm)
    pos = torch.full((B,), wl.position, dtype=torch.int32, device=DEV)
    o_chunk = torch.full((B, T, 32, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    R.gdn_prefill(chunk, B, T, x, a, b, pos, pd, o_chunk)

    samples = [0, 257, 511]
    checks = (0, 128, T - 1)
    snap = {}
    o_i = torch.empty(B, 32, 128, dtype=torch.bfloat16, device=DEV)
    for i in range(T):
        if i in checks:
            snap[i] = (steps.S[samples].cpu().numpy(), bits_host(steps.conv[samples]).copy())
        R.gdn_decode_step(steps, B, x[:, i].contiguous(), a[:, i].contiguous(),
                          b[:, i].contiguous(), pos + i, pd, o_i)
        _same_bits(o_chunk[:, i].view(torch.int16), o_i.view(torch.int16), f"o[{i}]")
    _same_bits(chunk.S.view(torch.int16), steps.S.view(torch.int16), "S")
    _same_bits(chunk.conv.view(torch.int16), steps.conv.view(torch.int16), "ring")
    print("chunk equals 256 decode steps bit for bit; oracle on sampled sequences", flush=True)

    got_S = chunk.S[samples].cpu().numpy()
    for k, s in enumerate(samples):
        xs = W.gdn_chunk_x_np(wl, layer, s, T)
        for i in checks:
            S0, conv0 = snap[i]
            st = G.GdnState(S0[k:k + 1].copy(), conv0[k:k + 1].copy())
            ref_o = G.decode_step(st, xs[i][None], a_h[s:s + 1, i], b_h[s:s + 1, i],
                                  prm["conv_w"], prm["a_log"], prm["dt_bias"],
                                  np.array([wl.position + i], np.int32))
            assert_out_close(bits_host(o_chunk[s, i])[None], ref_o, what=f"seq {s} o[{i}]")
            if i == T - 1:
                assert_state_close(got_S[k:k + 1], st.S, what=f"seq {s} S after token {i}")
        # the trajectory from the initial state
        S0, conv0 = snap[0]
        ref = G.GdnState(S0[k:k + 1].copy(), conv0[k:k + 1].copy())
        for i in range(T):
            G.decode_step(ref, xs[i][None], a_h[s:s + 1, i], b_h[s:s + 1, i], prm["conv_w"],
                          prm["a_log"], prm["dt_bias"], np.array([wl.position + i], np.int32))
        worst = 0.0
        for h in range(32):
            r = ref.S[0, h]
            d = np.linalg.norm(got_S[k, h].astype(np.float64) - r.astype(np.float64))
            lim = T * np.linalg.norm(np.broadcast_to(state_bound(r, whole=True), (128, 128)))
            worst = max(worst, d / lim)
        print(f"seq {s}: 256-token trajectory, max head distance / bound {worst:.2e}", flush=True)
        assert worst <= 1.0, s


@pytest.mark.parametrize("B,dtype,T", [(1, "f32", 4096), (16, "f16", 1024)])
def test_gdn_prefill_long_chunks(B, dtype, T):
    """Long chunks (256 and 64 groups of 16 tokens) at the batch-1 configuration (FP32,
    32-column slices) and the smallest wide batch (FP16, one slice per head): matrices,
    ring and every output equal T gdn_decode_step calls bit for bit."""
    tag = f"gdn_prefill_long_{B}_{dtype}"
    print(f"case: gdn prefill long chunk B={B} dtype={dtype} T={T}", flush=True)
    prm = _params(tag)
    pd = _params_dev(prm)
    st = _state(tag, B, dtype)
    p0 = np.array([5, 70001, 0, 3] * 4, np.int32)[:B]
    x = torch.empty(B, T, 8192, dtype=torch.bfloat16, device=DEV)
    C.normal_bf16_torch_(x, synth.stream_key(tag, "x"))
    rng = synth.rng_np(synth.stream_key(tag, "ab"))
    a = f32_dev((rng.standard_normal((B, T, 32)) * 2).astype(np.float32))
    b = f32_dev((rng.standard_normal((B, T, 32)) * 2).astype(np.float32))
    pos = i32_dev(p0)
    chunk, steps = _upload(st), _upload(st)
    o_chunk = torch.full((B, T, 32, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    R.gdn_prefill(chunk, B, T, x, a, b, pos, pd, o_chunk)
    o_i = torch.empty(B, 32, 128, dtype=torch.bfloat16, device=DEV)
    for i in range(T):
        R.gdn_decode_step(steps, B, x[:, i].contiguous(), a[:, i].contiguous(),
                          b[:, i].contiguous(), pos + i, pd, o_i)
        _same_bits(o_chunk[:, i].view(torch.int16), o_i.view(torch.int16), f"o[{i}]")
    ib = torch.int16 if dtype == "f16" else torch.int32
    _same_bits(chunk.S.view(ib), steps.S.view(ib), "S")
    _same_bits(chunk.conv.view(torch.int16), steps.conv.view(torch.int16), "ring")
