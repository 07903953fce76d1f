"""Pins of the GDN decode-step oracle (oracle/gdn_ref.py): the delta rule's own
algebra (what a write stores, what a reset leaves, retrieval through orthonormal
keys, the matrix form of the update), the base model's public implementation
of the recurrence and of the convolution update (transformers), torch's
softplus/sigmoid/SiLU, and the state sizes the pages print."""

import math

import numpy as np
import pytest
import torch

from oracle import gdn_ref as G
from oracle import rma_ref as O
import synth


def _rng(tag):
    return synth.rng_np(synth.stream_key("gdn_oracle", tag))


def _unit(x):
    return x / np.linalg.norm(x)


def test_full_strength_write_stores_the_value_under_its_key():
    # alpha = beta = 1 and a unit key: afterwards S^T k returns exactly v (delta rule)
    rng = _rng("memorise")
    S = rng.standard_normal((128, 128))
    k = _unit(rng.standard_normal(128))
    v = rng.standard_normal(128)
    S1, _ = G.delta_rule_step(S, np.zeros(128), k, v, 1.0, 1.0)
    assert np.allclose(S1.T @ k, v, atol=1e-12)
    # directions orthogonal to k are untouched
    w = rng.standard_normal(128)
    w -= (w @ k) * k
    assert np.allclose(S1.T @ w, S.T @ w, atol=1e-10)


def test_zero_decay_resets_the_state():
    rng = _rng("reset")
    S = rng.standard_normal((128, 128))
    q, k, v = (rng.standard_normal(128) for _ in range(3))
    S1, o = G.delta_rule_step(S, q, k, v, 0.0, 0.3)
    assert np.allclose(S1, 0.3 * np.outer(k, v), atol=1e-14)
    assert np.allclose(o, 0.3 * v * (k @ q), atol=1e-12)


def test_orthonormal_keys_retrieve_their_values():
    rng = _rng("retrieve")
    Q, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    keys = Q[:, :10].T
    vals = rng.standard_normal((10, 128))
    S = np.zeros((128, 128))
    for k, v in zip(keys, vals):
        S, _ = G.delta_rule_step(S, np.zeros(128), k, v, 1.0, 1.0)
    for j in range(10):
        _, o = G.delta_rule_step(S, keys[j], keys[j], np.zeros(128), 1.0, 0.0)
        assert np.allclose(o, vals[j], atol=1e-11)


def test_update_equals_the_matrix_form():
    # S' = alpha (I - beta k k^T) S + beta k v^T, o = S'^T q
    rng = _rng("matrix")
    for _ in range(5):
        S = rng.standard_normal((128, 128))
        q, k, v = (rng.standard_normal(128) for _ in range(3))
        alpha, beta = rng.uniform(0.1, 1.0), rng.uniform(0.0, 1.0)
        S1, o = G.delta_rule_step(S, q, k, v, alpha, beta)
        M = alpha * (np.eye(128) - beta * np.outer(k, k)) @ S + beta * np.outer(k, v)
        assert np.allclose(S1, M, atol=1e-10)
        assert np.allclose(o, M.T @ q, atol=1e-9)


def test_scalar_maps_match_torch():
    x = np.concatenate([np.linspace(-40, 40, 801), [0.0, 1e-8, -1e-8, 700.0, -700.0]])
    t = torch.from_numpy(x)
    assert np.allclose(G.softplus(x), torch.nn.functional.softplus(t, threshold=1e9).numpy(),
                       rtol=1e-14, atol=1e-300)
    assert np.allclose(G.sigmoid(x), torch.sigmoid(t).numpy(), rtol=1e-14, atol=1e-300)
    assert np.allclose(G.silu(x[np.abs(x) < 600]), torch.nn.functional.silu(t[np.abs(t) < 600]).numpy(),
                       rtol=1e-14, atol=1e-300)
    assert G.softplus(0.0) == pytest.approx(math.log(2.0), abs=1e-16)
    assert G.sigmoid(0.0) == 0.5 and G.silu(0.0) == 0.0


def test_gates_in_range():
    rng = _rng("gates")
    a, b = rng.standard_normal((4, 32)) * 3, rng.standard_normal((4, 32)) * 3
    alpha, beta = G.gates(a, b, np.log(rng.uniform(1, 16, 32)), rng.standard_normal(32))
    assert np.all((alpha > 0) & (alpha <= 1)) and np.all((beta > 0) & (beta < 1))
    # A_log = -inf (A = 0) means no decay at all
    alpha0, _ = G.gates(a, b, np.full(32, -np.inf), np.zeros(32))
    assert np.all(alpha0 == 1.0)
    # closed forms: A = 1, a + dt_bias = 0 -> alpha = exp(-ln 2) = 1/2;
    # A = 3, softplus(a + dt_bias) = 1 -> alpha = e^-3; b = ln 3 -> beta = 3/4
    one = np.ones((1, 32))
    al, be = G.gates(0.7 * one, np.log(3.0) * one, np.zeros(32), np.full(32, -0.7))
    assert np.allclose(al, 0.5, rtol=1e-15) and np.allclose(be, 0.75, rtol=1e-15)
    al, _ = G.gates(np.log(np.e - 1.0) * one, one, np.full(32, np.log(3.0)), np.zeros(32))
    assert np.allclose(al, np.exp(-3.0), rtol=1e-14)


def test_convolution_with_a_unit_tap_is_a_time_shift():
    rng = _rng("conv")
    C = 8
    xs = rng.standard_normal((10, C))
    for lag in range(4):
        w = np.zeros((C, 4))
        w[:, 3 - lag] = 1.0  # tap 3 - lag multiplies the input of position p - lag
        ring = np.zeros((4, C))
        for p in range(10):
            y, ring = G.conv_step(ring, xs[p], w, p)
            pre = xs[p - lag] if p - lag >= 0 else np.zeros(C)
            assert np.allclose(y, G.silu(pre), atol=1e-15)


def _hf():
    return pytest.importorskip("transformers.models.qwen3_5.modeling_qwen3_5")


def test_convolution_matches_the_base_models_update():
    hf = _hf()
    rng = _rng("conv_hf")
    C, T = 64, 9
    w = rng.standard_normal((C, 4))
    xs = rng.standard_normal((T, C))
    state = torch.zeros(1, C, 4, dtype=torch.float64)
    ring = np.zeros((4, C))
    for p in range(T):
        ref = hf.causal_conv1d_update(torch.from_numpy(xs[p]).reshape(1, C, 1), state,
                                      torch.from_numpy(w), None, "silu")
        y, ring = G.conv_step(ring, xs[p], w, p)
        assert np.allclose(y, ref.reshape(C).numpy(), rtol=1e-13, atol=1e-14)


def test_recurrence_matches_the_base_models_implementation():
    """The whole step after the convolution (L2 norms, q scale, key head per value
    head, decay, delta rule, output) against transformers' recurrent gated delta
    rule over several tokens.  That routine computes in FP32 whatever its inputs
    are, so the bar is FP32-sized; a wrong sign, index or transposition anywhere
    would show as an O(1) relative difference."""
    hf = _hf()
    rng = _rng("rec_hf")
    B, T = 2, 5
    q = rng.standard_normal((B, T, 16, 128))
    k = rng.standard_normal((B, T, 16, 128))
    v = rng.standard_normal((B, T, 32, 128))
    g = -rng.uniform(0.0, 2.0, (B, T, 32))
    beta = rng.uniform(0.0, 1.0, (B, T, 32))
    S0 = rng.standard_normal((B, 32, 128, 128)) * 0.1
    t = lambda x: torch.from_numpy(x)  # noqa: E731
    rep = lambda x: t(x).repeat_interleave(2, dim=2)  # noqa: E731
    ref_o, ref_S = hf.torch_recurrent_gated_delta_rule(rep(q), rep(k), t(v), g=t(g), beta=t(beta),
                                                       initial_state=t(S0.copy()),
                                                       output_final_state=True,
                                                       use_qk_l2norm_in_kernel=True)
    S = S0.copy()
    for s in range(B):
        for i in range(T):
            qn = G.l2_normalize(q[s, i]) / math.sqrt(128)
            kn = G.l2_normalize(k[s, i])
            for h in range(32):
                S[s, h], o = G.delta_rule_step(S[s, h], qn[h // 2], kn[h // 2], v[s, i, h],
                                               math.exp(g[s, i, h]), beta[s, i, h])
                assert np.allclose(o, ref_o[s, i, h].numpy(), rtol=1e-4, atol=1e-6)
    assert np.allclose(S, ref_S.numpy(), rtol=1e-4, atol=1e-6)


def test_decode_step_rounds_the_state_and_keeps_the_inputs():
    rng = _rng("decode")
    B = 2
    st = G.new_state(B, "f16")
    x = synth.normal_bf16_np(synth.stream_key("gdn_oracle", "x"), B * 8192).reshape(B, 8192)
    w = rng.standard_normal((8192, 4)) * 0.5
    a, b = rng.standard_normal((B, 32)), rng.standard_normal((B, 32))
    o = G.decode_step(st, x, a, b, w, np.log(rng.uniform(1, 16, 32)), rng.standard_normal(32),
                      [0, 5])
    assert st.S.dtype == np.float16 and np.all(np.isfinite(o))
    assert np.array_equal(st.conv[0, 0], x[0]) and np.array_equal(st.conv[1, 1], x[1])
    assert not np.any(st.conv[0, 1:]) and not np.any(st.conv[1, [0, 2, 3]])
    # from a zero state the first token stores S = beta k v^T, rounded to FP16
    alpha, beta = G.gates(a, b, np.log(np.ones(32)), np.zeros(32))
    # (recompute with the same parameters to compare one head)
    st2 = G.new_state(1, "f32")
    A_log, dtb = np.zeros(32), np.zeros(32)
    G.decode_step(st2, x[:1], a[:1], b[:1], w, A_log, dtb, [0])
    y, _ = G.conv_step(np.zeros((4, 8192)), O.bf16_to_f64(x[0]), w, 0)
    qq, kk, vv = G.split_heads(y)
    _, bt = G.gates(a[:1], b[:1], A_log, dtb)
    ref = bt[0, 7] * np.outer(G.l2_normalize(kk[3]), vv[7])
    assert np.allclose(st2.S[0, 7], ref, rtol=1e-6, atol=1e-7)
    assert alpha.shape == (B, 32)


def test_fp16_state_rounding_is_nearest_even():
    rng = _rng("half")
    x = rng.standard_normal(100000) * np.exp2(rng.uniform(-20, 15, 100000))
    x = x[np.abs(x) < 65504]  # the finite FP16 range
    r = G.round_state(x, "f16")
    # nearest FP16 value: no neighbour is closer, and a tie goes to the even code
    up = np.nextafter(r, np.float16(np.inf))
    dn = np.nextafter(r, np.float16(-np.inf))
    e = np.abs(x - r.astype(np.float64))
    assert np.all(e <= np.abs(x - up.astype(np.float64)))
    assert np.all(e <= np.abs(x - dn.astype(np.float64)))
    tie = (e == np.abs(x - up.astype(np.float64))) | (e == np.abs(x - dn.astype(np.float64)))
    assert np.all(r.view(np.uint16)[tie] % 2 == 0)
    # for FP32 inputs (one rounding only) torch's half cast agrees bit for bit
    x32 = x.astype(np.float32)
    got = G.round_state(x32, "f16").view(np.uint16)
    ref = torch.from_numpy(x32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_state_sizes_match_the_printed_inventory():
    MiB = 1 << 20
    # 24 MiB of recurrent matrices [FB "72 MiB 是怎么算出来的"] at the batched (FP16) precision
    assert G.GDN_LAYERS * G.V_HEADS * G.HEAD_K * G.HEAD_V * 2 == 24 * MiB
    # 25.50 MiB of recurrent state [FB "常见问题"]: matrices plus the last 4 convolution inputs
    assert G.state_bytes_per_sequence() == int(25.5 * MiB)
    # with the window's 71.97 MiB and the 0.29 MiB of progress metadata: 97.76 MiB in all
    window_and_rma = 2 * 8 * 4 * (1023 + 1024 + 256) * 256 * 2
    meta = 8 * (4 * 1024 * 8 + 256 * (4 * 4 + 4))
    total = (G.state_bytes_per_sequence() + window_and_rma + meta) / MiB
    assert round(total, 2) == 97.76
    # the head widths are the unique solution of the two printed sizes
    sols = [(dk, dv) for dk in range(1, 513) for dv in range(1, 513)
            if 24 * 32 * dk * dv * 2 == 24 * MiB and 24 * 4 * (2 * 16 * dk + 32 * dv) * 2 == 1.5 * MiB]
    assert sols == [(128, 128)]
