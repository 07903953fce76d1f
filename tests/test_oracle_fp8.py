"""Pins of the FP8 K/V oracle (oracle/fp8_ref.py) against torch's float8_e4m3fn
conversions, exact identities and the pinned BF16 oracle."""

import numpy as np
import torch

import oracle as O
from oracle import fp8_ref as F
import synth


def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_for_every_code():
    ref = _torch_decode_all()
    got = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))  # -0 at 0x80
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_encode_matches_torch_on_codes_midpoints_and_neighbours():
    vals = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.sort(np.unique(np.abs(vals[~np.isnan(vals)])))
    mids = (fin[:-1] + fin[1:]) / 2  # every tie between neighbours (exact in fp32)
    pts = np.concatenate([fin, mids, [464.0, 463.99, 470.0, 480.0, 1e30]]).astype(np.float32)
    near = np.concatenate([np.nextafter(pts, np.float32(np.inf)),
                           np.nextafter(pts, np.float32(-np.inf))]).astype(np.float32)
    x = np.concatenate([pts, near, -pts, -near, [0.0, -0.0]]).astype(np.float32)
    assert np.array_equal(F.e4m3_encode(x), _torch_encode(x))


def test_encode_matches_torch_on_random_values():
    rng = synth.rng_np(synth.stream_key("fp8", "encode"))
    x = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-12, 9, 200_000))).astype(np.float32)
    x = x[np.abs(x) < 460]
    assert np.array_equal(F.e4m3_encode(x), _torch_encode(x))


def test_encode_decode_round_trip():
    c = np.array([i for i in range(256) if i not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(c)), c)


def test_quantize_rows_tiny_rows_are_stored_as_zero():
    """A row whose largest magnitude is below 448 * 2^-126 (for example a row of BF16
    subnormals) would need 448 / amax beyond 2^126 and a scale below the normal FP32
    range; it is stored as a zero row.  At the threshold the row is quantised as usual,
    its largest element going to +-448, and every code stays finite."""
    sub = (np.arange(1, 257, dtype=np.float64) * 2.0**-133).astype(np.float32)  # BF16 subnormals
    sub[::3] *= -1
    thr = np.float32(448.0 * 2.0**-126)
    at = np.full(256, thr / 2, np.float32)
    at[17] = -thr
    just_below = np.full(256, np.nextafter(thr, np.float32(0)), np.float32)
    codes, scale = F.quantize_rows(np.stack([sub, at, just_below]))
    assert np.all(codes[0] == 0) and scale[0] == 0
    assert np.all(codes[2] == 0) and scale[2] == 0
    assert scale[1] == np.float32(2.0**-126)
    dec = F.e4m3_decode(codes[1])
    assert not np.any(np.isnan(dec)) and dec[17] == -448.0 and np.all(dec[:17] == 224.0)
    # the stored zero row is within the threshold of the input
    assert np.all(np.abs(F.dequantize(codes[0], scale[0]) - sub) < float(thr))


def test_quantize_rows_matches_a_torch_implementation():
    rng = synth.rng_np(synth.stream_key("fp8", "rows"))
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    x[3] = 0.0
    codes, scale = F.quantize_rows(x)
    t = torch.from_numpy(x)
    amax = t.abs().amax(-1)
    inv = torch.where(amax == 0, torch.zeros_like(amax), 448.0 / torch.where(amax == 0, 1.0, amax))
    tc = (t * inv[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ts = (amax / 448.0).numpy()
    assert np.array_equal(codes, tc)
    assert np.array_equal(scale.view(np.uint32), ts.astype(np.float32).view(np.uint32))
    # invariants: the largest element maps to +-448; zero row -> zero codes and scale
    nz = np.arange(64) != 3
    assert np.all(np.max(np.abs(F.e4m3_decode(codes[nz])), axis=1) == 448.0)
    assert np.all(codes[3] == 0) and scale[3] == 0
    # error bound: half an E4M3 step of the scaled value (plus the FP32 product's rounding)
    deq = F.dequantize(codes, scale)
    y = x.astype(np.float64) * (448.0 / np.where(nz, np.abs(x).max(1), 1.0))[:, None]
    bound = (0.5 * F.e4m3_step(y) + np.abs(y) * 2.0 ** -23) * scale[:, None] * 1.0001 + 1e-45
    assert np.all(np.abs(deq - x) <= bound)


def _exact_state(tag, B=2, window=64, bank=32, block=16, G=4, D=256):
    """An FP8 state whose dequantised values are exact BF16 numbers (power-of-two
    scales), with the BF16 state holding the same values."""
    st8 = F.new_layer_state_fp8(B, window, bank, block, G, D)
    rng = synth.rng_np(synth.stream_key("fp8", tag))
    for nm in ("win", "bank", "pend"):
        for kv in ("k", "v"):
            arr = getattr(st8, f"{nm}_{kv}")
            c = rng.integers(0, 256, arr.shape, dtype=np.uint8)
            c[(c & 0x7F) == 0x7F] ^= 0x01  # no NaN codes
            arr[...] = c
            getattr(st8, f"{nm}_{kv}s")[...] = np.exp2(rng.integers(-9, -5, arr.shape[:-1]))
    st = O.new_layer_state(B, window, bank, block, G, D)
    for nm in ("win", "bank", "pend"):
        for kv in ("k", "v"):
            val = F.dequantize(getattr(st8, f"{nm}_{kv}"), getattr(st8, f"{nm}_{kv}s"))
            bits = O.f64_to_bf16(val)
            assert np.array_equal(O.bf16_to_f64(bits), val)  # exact in BF16
            getattr(st, f"{nm}_{kv}")[...] = bits
    for s in (st, st8):
        s.n_bank[:] = [bank, bank // 2]
        s.n_pend[:] = [block, 3]
        s.pos[:] = [1000, 40]
    return st8, st


def test_fp8_decode_equals_bf16_decode_on_identical_values():
    st8, st = _exact_state("decode")
    rng = synth.rng_np(synth.stream_key("fp8", "q"))
    q = O.f64_to_bf16(rng.standard_normal((2, 16, 256)))
    g = O.f64_to_bf16(1 + 0.1 * rng.standard_normal(256)).view(np.uint16)
    gq = O.bf16_to_f64(g)
    a = F.decode(st8, q, q, gq, gq, 1e-6, 1e7)
    b = O.decode(st, q, q, gq, gq, 1e-6, 1e7)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_fp8_commit_selects_like_bf16_commit_and_moves_codes_with_scales():
    st8, st = _exact_state("commit")
    rng = synth.rng_np(synth.stream_key("fp8", "scores"))
    for s in (st, st8):
        s.bank_score[...] = rng.standard_normal(s.bank_score.shape).astype(np.float32)
        s.pend_score[...] = rng.standard_normal(s.pend_score.shape).astype(np.float32)
        s.bank_src[...] = np.arange(s.bank_src.size).reshape(s.bank_src.shape) % 1000
        s.pend_src[...] = 2000 + np.arange(s.pend_src.size).reshape(s.pend_src.shape)
        rng = synth.rng_np(synth.stream_key("fp8", "scores"))  # same draws for both
    before = st8.copy()
    k8 = F.commit(st8)
    k16 = O.commit(st)
    assert np.array_equal(k8, k16)
    cap = st8.bank_k.shape[2]
    for b in range(2):
        for g in range(4):
            for sl in range(cap):
                i = k8[b, g, sl]
                if i >= cap:
                    assert np.array_equal(st8.bank_k[b, g, sl], before.pend_k[b, g, i - cap])
                    assert st8.bank_vs[b, g, sl] == before.pend_vs[b, g, i - cap]
                elif i >= 0:
                    assert np.array_equal(st8.bank_v[b, g, sl], before.bank_v[b, g, sl])
    # the dequantised bank equals the BF16 bank after the same commit
    assert np.array_equal(F.dequantize(st8.bank_k, st8.bank_ks), O.bf16_to_f64(st.bank_k))


def test_fp8_append_quantises_the_bf16_paths_fp32_keys_and_raw_values():
    B, window, block = 2, 64, 16
    st8 = F.new_layer_state_fp8(B, window, 32, block)
    st = O.new_layer_state(B, window, 32, block)
    for s in (st8, st):
        s.pos[:] = [70, 5]
    rec = [synth.normal_bf16_np(synth.stream_key("fp8", "rec", i), B * 1024).reshape(B, 4, 256)
           for i in range(4)]
    g = synth.normal_f32_np(synth.stream_key("fp8", "g"), (256,), 1.0, 0.1).astype(np.float64)
    F.append(st8, *rec, g, g, 1e-6, 1e7)
    O.append(st, *rec, g, g, 1e-6, 1e7)
    for b in range(B):
        slot = int(st.pos[b]) % window
        v8 = F.dequantize(st8.win_v[b, :, slot], st8.win_vs[b, :, slot])
        vr = O.bf16_to_f64(rec[1][b])
        c, s = F.quantize_rows(vr.astype(np.float32))
        assert np.array_equal(st8.win_v[b, :, slot], c) and np.array_equal(st8.win_vs[b, :, slot], s)
        k8 = F.dequantize(st8.win_k[b, :, slot], st8.win_ks[b, :, slot])
        kb = O.bf16_to_f64(st.win_k[b, :, slot])
        scale = st8.win_ks[b, :, slot][:, None]
        # FP8 key vs BF16 key of the same FP32 value: within an E4M3 half step + a BF16 ulp
        tol = 0.5 * F.e4m3_step(kb / scale) * scale * 1.01 + np.abs(kb) * 2.0 ** -8
        assert np.all(np.abs(k8 - kb) <= tol)
        assert np.all(np.abs(v8 - vr) <= 0.5 * F.e4m3_step(vr / st8.win_vs[b, :, slot][:, None])
                      * st8.win_vs[b, :, slot][:, None] * 1.01 + 1e-30)
    assert np.array_equal(st8.pend_src, st.pend_src) and np.array_equal(st8.n_pend, st.n_pend)


def test_fp8_unit_bytes_closed_form():
    # 2 x 4 groups x (1024 + 1024 + 256) rows x (256 code bytes + 4 scale bytes)
    assert F.kv_bytes_per_unit() == 2 * 4 * 2304 * 260 == 4_792_320
