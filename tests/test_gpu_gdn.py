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

from gpu_util import DEV, bits_host, f32_dev, i32_dev

pytestmark = pytest.mark.gpu

O_TOL = 1e-2


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
    """New matrices against the oracle's (both stored in the same precision).

    The GPU forms a S + k u in FP32 and rounds once to the storage type; the oracle
    forms it in float64 and rounds once.  The FP32 value is within a few 2^-24 of
    the head's largest magnitude of the exact one, which can move it across one
    rounding boundary of the storage type: the bound is one unit in the last place
    of the reference element plus 2^-18 of the head's largest magnitude.
    """
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if ref.dtype == np.float16:
        _, e = np.frexp(np.maximum(np.abs(r), 2.0 ** -14))
        ulp = np.ldexp(1.0, e - 11)
    else:
        _, e = np.frexp(np.maximum(np.abs(r), 2.0 ** -126))
        ulp = np.ldexp(1.0, e - 24)
    scale = np.abs(r).reshape(r.shape[0], -1).max(axis=1).reshape((-1,) + (1,) * (r.ndim - 1))
    bound = ulp + 2.0 ** -18 * scale
    err = np.abs(g - r)
    ndiff = int((got != ref).sum())
    print(f"{what}: {ndiff} of {g.size} entries differ; max err/bound "
          f"{float((err / bound).max()):.3f}")
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} entries out of bound"


def assert_out_close(got_bits, ref, what=""):
    g = synth.bf16_bits_to_f32_np(got_bits).astype(np.float64).reshape(-1, 128)
    r = np.asarray(ref, np.float64).reshape(-1, 128)
    scale = np.maximum(np.abs(r).max(axis=1), 1e-30)
    rel = np.abs(g - r).max(axis=1) / scale
    print(f"{what}: rows={rel.size} out max={rel.max():.3e} median={np.median(rel):.3e}")
    assert np.all(np.isfinite(g)) and rel.max() <= O_TOL, what


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


def _state_bound(ref):
    """Per-element bound of one step (see assert_state_close)."""
    r = np.asarray(ref, np.float64)
    if ref.dtype == np.float16:
        _, e = np.frexp(np.maximum(np.abs(r), 2.0 ** -14))
        ulp = np.ldexp(1.0, e - 11)
    else:
        _, e = np.frexp(np.maximum(np.abs(r), 2.0 ** -126))
        ulp = np.ldexp(1.0, e - 24)
    return ulp + 2.0 ** -18 * np.abs(r).max()


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
            assert np.all(err <= _state_bound(before.S)), f"S t={t}"
    got = dev.S.cpu().numpy().astype(np.float64)
    for s_ in range(B):
        for h in range(32):
            d = np.linalg.norm(got[s_, h] - ref.S[s_, h].astype(np.float64))
            lim = T * np.linalg.norm(np.broadcast_to(_state_bound(ref.S[s_, h]), (128, 128)))
            assert d <= lim, (s_, h, d, lim)
    print(f"trajectories: max head distance / bound "
          f"{max(np.linalg.norm(got[s_, h] - ref.S[s_, h]) / (T * np.linalg.norm(np.broadcast_to(_state_bound(ref.S[s_, h]), (128, 128)))) for s_ in range(B) for h in range(32)):.3f}")


def _full_size(wl, layers, samples):
    B = wl.batch
    print(f"case: {wl.name} B={B} layers={layers}", flush=True)
    dt = torch.float16 if wl.extra["state"] == "f16" else torch.float32
    outs, states, xs, gates, params = [], [], [], [], []
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
        gates.append((a, b))
        params.append(p)
    torch.cuda.synchronize()
    print("step done; checking samples", flush=True)
    for b_, layer, h in samples:
        sdt = np.float16 if wl.extra["state"] == "f16" else np.float32
        ref = G.GdnState(np.zeros((1, 32, 128, 128), sdt), W.gdn_conv_np(wl, layer, b_)[None].copy())
        ref.S[0, h] = W.gdn_state_np(wl, layer, b_, h)
        a, b = gates[layer]
        p = params[layer]
        ref_o = G.decode_step(ref, W.gdn_x_np(wl, layer, b_)[None], a[b_:b_ + 1], b[b_:b_ + 1],
                              p["conv_w"], p["a_log"], p["dt_bias"], [wl.position], heads=[h])
        assert_state_close(states[layer].S[b_, h].cpu().numpy()[None], ref.S[0, h][None],
                           what=f"S b={b_} layer={layer} h={h}")
        assert_out_close(bits_host(outs[layer][b_, h]), ref_o[0, h],
                         what=f"o b={b_} layer={layer} h={h}")
        got_ring = bits_host(states[layer].conv[b_])
        assert np.array_equal(got_ring, ref.conv[0]), "ring"
    for o in outs:
        assert torch.isfinite(o.float()).all()


def test_gdn_decode_b512_sampled():
    wl = W.GDN_DECODE_B512
    rng = np.random.default_rng(5120)
    samples = [(int(b), int(l), int(h)) for b, l, h in zip(rng.integers(0, 512, 16),
                                                            rng.integers(0, 2, 16),
                                                            rng.integers(0, 32, 16))]
    samples += [(0, 0, 0), (511, 1, 31)]
    _full_size(wl, 2, samples)


def test_gdn_decode_b1_every_head():
    wl = W.GDN_DECODE_B1
    _full_size(wl, 1, [(0, 0, h) for h in range(32)])
