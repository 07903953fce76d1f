"""Pins of the oracle's BF16 codec, RMS normalisation and partial rotary embedding."""

import math

import numpy as np
import pytest
import torch

import oracle as O


# ---------------------------------------------------------------- BF16 codec
def test_bf16_roundtrip_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = O.bf16_to_f64(bits)
    back = O.f64_to_bf16(x)
    nan = np.isnan(x)
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(back[nan] == 0x7FC0)


def test_bf16_round_half_even_and_overflow():
    one = 0x3F80
    assert O.f64_to_bf16(1.0 + 2.0**-8) == one  # halfway, even neighbour is 1.0
    assert O.f64_to_bf16(1.0 + 3 * 2.0**-8) == one + 2  # halfway, rounds up to even
    assert O.f64_to_bf16(1.0 + 2.0**-8 + 2.0**-30) == one + 1  # just above halfway
    assert O.f64_to_bf16(-0.0) == 0x8000
    assert O.f64_to_bf16(3.5e38) == 0x7F80  # beyond the largest finite BF16
    assert O.f64_to_bf16(2.0**-133) == 0x0001  # smallest subnormal
    assert O.f64_to_bf16(2.0**-134) == 0x0000  # halfway to zero: even is zero


def test_bf16_encode_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16(x.astype(np.float64)), ref)


# ---------------------------------------------------------------- RMS norm
def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 256)) * 3.0
    gam = 1.0 + 0.1 * rng.standard_normal(256)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (256,), torch.from_numpy(gam),
                                       eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, gam, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_rmsnorm_scale_invariance_and_norm_closed_form():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(256)
    np.testing.assert_allclose(O.rms_norm(7.5 * x, np.ones(256), 0.0),
                               O.rms_norm(x, np.ones(256), 0.0), rtol=1e-13)
    eps = 1e-2
    y = O.rms_norm(x, np.ones(256), eps)
    m = np.mean(x * x)
    assert math.isclose(np.sum(y * y), 256 * m / (m + eps), rel_tol=1e-12)
    # the gain multiplies, elementwise
    gam = np.linspace(0.5, 2.0, 256)
    np.testing.assert_allclose(O.rms_norm(x, gam, eps), y * gam, rtol=1e-14)


# ---------------------------------------------------------------- rotary
def test_rope_position_zero_is_identity_and_tail_untouched():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(256)
    np.testing.assert_array_equal(O.rope(x, 0, 1e7), x)
    y = O.rope(x, 12345, 1e7)
    np.testing.assert_array_equal(y[64:], x[64:])


def test_rope_preserves_pair_norms_and_relative_shift():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(256), rng.standard_normal(256)
    y = O.rope(q, 777, 1e7)
    np.testing.assert_allclose(y[:32] ** 2 + y[32:64] ** 2, q[:32] ** 2 + q[32:64] ** 2,
                               rtol=1e-12)
    for p, s, d in ((100, 40, 7), (65536, 1000, 123456), (3, 3, 262140)):
        a = O.rope(q, p + d, 1e7) @ O.rope(k, s + d, 1e7)
        b = O.rope(q, p, 1e7) @ O.rope(k, s, 1e7)
        assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_pairing_and_frequency_ladder():
    # e_0 rotated at position 1 by the fastest pair (angle 1 rad) lands on dims 0 and 32.
    e0 = np.zeros(256)
    e0[0] = 1.0
    y = O.rope(e0, 1, 1e7)
    assert math.isclose(y[0], math.cos(1.0)) and math.isclose(y[32], math.sin(1.0))
    assert np.count_nonzero(y) == 2
    # angles recovered from the output form the ladder base^(-2i/64), i = 0..31
    x = np.zeros(256)
    x[:32] = 1.0
    y = O.rope(x, 1, 1e7)
    ang = np.arctan2(y[32:64], y[:32])
    np.testing.assert_allclose(ang[1:] / ang[:-1], 1e7 ** (-1.0 / 32), rtol=1e-12)
    assert math.isclose(ang[0], 1.0, rel_tol=1e-15)


def test_rope_matches_transformers_rotate_half():
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as m

    cfg = LlamaConfig(hidden_size=256, num_attention_heads=4, head_dim=64, rope_theta=1e7,
                      max_position_embeddings=262144)
    emb = m.LlamaRotaryEmbedding(cfg)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 256))
    pos = [0, 1, 17, 99, 250]
    cos, sin = emb(torch.zeros(1, 1, 5, 64, dtype=torch.float64), torch.tensor([pos]))
    xt = torch.from_numpy(x[None, None, :, :64].copy())
    ref, _ = m.apply_rotary_pos_emb(xt, xt, cos, sin)
    for i, p in enumerate(pos):
        y = O.rope(x[i], p, 1e7)
        # the library keeps its frequencies in float32: agree to its precision
        np.testing.assert_allclose(y[:64], ref[0, 0, i].numpy(), atol=3e-5 * max(1, p))
        np.testing.assert_array_equal(y[64:], x[i, 64:])
