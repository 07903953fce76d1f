"""Pins of the INT8 K/V oracle (oracle/int8_ref.py): exact grids, ties, the error
bound, tiny rows, two's-complement storage, and decode / commit / append against the
pinned BF16 oracle on identical values."""

import numpy as np

import oracle as O
from oracle import int8_ref as I
import synth


def test_codes_on_an_exact_grid_round_trip():
    """Rows of integer multiples k * c of a power of two c with max |k| = 127: the
    scale is c, 127 / amax is 1 / c exactly, and every code is k."""
    rng = synth.rng_np(synth.stream_key("i8", "grid"))
    k = rng.integers(-127, 128, (16, 256))
    k[:, 5] = 127
    k[::2, 9] = -127
    c = np.exp2(rng.integers(-20, 20, 16)).astype(np.float64)
    x = (k * c[:, None]).astype(np.float32)
    codes, scale = I.quantize_rows(x)
    assert np.array_equal(codes.view(np.int8).astype(np.int64), k)
    assert np.array_equal(scale.astype(np.float64), c)
    assert np.array_equal(I.dequantize(codes, scale), x.astype(np.float64))


def test_halves_round_to_even():
    """amax = 127 gives inv = 1, so x * inv = x: halves go to the even neighbour
    (a rounding away from zero would give 3, 5, -3, -1, 1, 127)."""
    x = np.zeros((1, 256), np.float32)
    x[0, :7] = [127.0, 2.5, 4.5, -2.5, -0.5, 0.5, 126.5]
    codes, scale = I.quantize_rows(x)
    assert scale[0] == np.float32(1.0)
    assert list(codes[0, :7].view(np.int8)) == [127, 2, 4, -2, 0, 0, 126]


def test_codes_are_twos_complement_bytes_and_never_minus_128():
    x = np.zeros((1, 256), np.float32)
    x[0, :4] = [-127.0, -1.0, 1.0, 127.0]
    codes, _ = I.quantize_rows(x)
    assert list(codes[0, :4]) == [0x81, 0xFF, 0x01, 0x7F]
    rng = synth.rng_np(synth.stream_key("i8", "range"))
    y = (rng.standard_normal((256, 256)) * np.exp2(rng.uniform(-30, 30, (256, 1)))).astype(np.float32)
    codes, _ = I.quantize_rows(y)
    assert not np.any(codes == 0x80)
    assert np.all(np.max(np.abs(codes.view(np.int8).astype(np.int64)), axis=1) == 127)


def test_error_is_at_most_half_a_step():
    """|stored - x| <= scale / 2, plus the FP32 rounding of 127 / amax and of the
    product (a few ulps of the scaled value, times the scale)."""
    rng = synth.rng_np(synth.stream_key("i8", "err"))
    x = (rng.standard_normal((128, 256)) * np.exp2(rng.uniform(-10, 10, (128, 1)))).astype(np.float32)
    codes, scale = I.quantize_rows(x)
    err = np.abs(I.dequantize(codes, scale) - x.astype(np.float64))
    bound = scale.astype(np.float64)[:, None] * (0.5 + 127.0 * 2.0**-22)
    assert np.all(err <= bound)
    # and the bound is not loose: some element comes within 1% of half a step
    assert np.max(err / (scale.astype(np.float64)[:, None] * 0.5)) > 0.99


def test_tiny_rows_are_stored_as_zero():
    thr = np.float32(127.0 * 2.0**-126)
    sub = (np.arange(1, 257, dtype=np.float64) * 2.0**-133).astype(np.float32)
    at = np.full(256, thr / 2, np.float32)
    at[3] = -thr
    below = np.full(256, np.nextafter(thr, np.float32(0)), np.float32)
    zero = np.zeros(256, np.float32)
    codes, scale = I.quantize_rows(np.stack([sub, at, below, zero]))
    for r in (0, 2, 3):
        assert np.all(codes[r] == 0) and scale[r] == 0
    assert scale[1] == np.float32(2.0**-126) and codes[1].view(np.int8)[3] == -127


def _exact_state(tag, B=2, window=64, bank=32, block=16, G=4, D=256):
    """An INT8 state whose dequantised values are exact BF16 numbers (|code| <= 127
    has at most 7 significant bits; power-of-two scales), and the BF16 state holding
    the same values."""
    st8 = I.new_layer_state_i8(B, window, bank, block, G, D)
    rng = synth.rng_np(synth.stream_key("i8", tag))
    for nm in ("win", "bank", "pend"):
        for kv in ("k", "v"):
            arr = getattr(st8, f"{nm}_{kv}")
            arr[...] = rng.integers(-127, 128, arr.shape).astype(np.int8).view(np.uint8)
            getattr(st8, f"{nm}_{kv}s")[...] = np.exp2(rng.integers(-9, -5, arr.shape[:-1]))
    st = O.new_layer_state(B, window, bank, block, G, D)
    for nm in ("win", "bank", "pend"):
        for kv in ("k", "v"):
            val = I.dequantize(getattr(st8, f"{nm}_{kv}"), getattr(st8, f"{nm}_{kv}s"))
            bits = O.f64_to_bf16(val)
            assert np.array_equal(O.bf16_to_f64(bits), val)
            getattr(st, f"{nm}_{kv}")[...] = bits
    for s in (st, st8):
        s.n_bank[:] = [bank, bank // 2]
        s.n_pend[:] = [block, 3]
        s.pos[:] = [1000, 40]
    return st8, st


def test_int8_decode_equals_bf16_decode_on_identical_values():
    st8, st = _exact_state("decode")
    rng = synth.rng_np(synth.stream_key("i8", "q"))
    q = O.f64_to_bf16(rng.standard_normal((2, 16, 256)))
    gq = O.bf16_to_f64(O.f64_to_bf16(1 + 0.1 * rng.standard_normal(256)))
    a = I.decode(st8, q, q, gq, gq, 1e-6, 1e7)
    b = O.decode(st, q, q, gq, gq, 1e-6, 1e7)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_int8_commit_selects_like_bf16_commit():
    st8, st = _exact_state("commit")
    for s in (st, st8):
        rng = synth.rng_np(synth.stream_key("i8", "scores"))
        s.bank_score[...] = rng.standard_normal(s.bank_score.shape).astype(np.float32)
        s.pend_score[...] = rng.standard_normal(s.pend_score.shape).astype(np.float32)
        s.bank_src[...] = np.arange(s.bank_src.size).reshape(s.bank_src.shape) % 1000
        s.pend_src[...] = 2000 + np.arange(s.pend_src.size).reshape(s.pend_src.shape)
    assert np.array_equal(I.commit(st8), O.commit(st))
    assert np.array_equal(I.dequantize(st8.bank_k, st8.bank_ks), O.bf16_to_f64(st.bank_k))
    assert np.array_equal(I.dequantize(st8.bank_v, st8.bank_vs), O.bf16_to_f64(st.bank_v))


def test_int8_append_quantises_the_bf16_paths_fp32_keys_and_raw_values():
    B, window, block = 2, 64, 16
    st8 = I.new_layer_state_i8(B, window, 32, block)
    st = O.new_layer_state(B, window, 32, block)
    for s in (st8, st):
        s.pos[:] = [70, 5]
    rec = [synth.normal_bf16_np(synth.stream_key("i8", "rec", i), B * 1024).reshape(B, 4, 256)
           for i in range(4)]
    gw = synth.normal_f32_np(synth.stream_key("i8", "gw"), (256,), 1.0, 0.1).astype(np.float64)
    gr = synth.normal_f32_np(synth.stream_key("i8", "gr"), (256,), 1.0, 0.1).astype(np.float64)
    I.append(st8, *rec, gw, gr, 1e-6, 1e7)
    O.append(st, *rec, gw, gr, 1e-6, 1e7)
    for b in range(B):
        slot = int(st.pos[b]) % window
        t = int(st.n_pend[b]) - 1
        for arr, sc, raw in ((st8.win_v[b, :, slot], st8.win_vs[b, :, slot], rec[1][b]),
                             (st8.pend_v[b, :, t], st8.pend_vs[b, :, t], rec[3][b])):
            c, s = I.quantize_rows(O.bf16_to_f64(raw).astype(np.float32))
            assert np.array_equal(arr, c) and np.array_equal(sc, s)
        for arr, sc, ref in ((st8.win_k[b, :, slot], st8.win_ks[b, :, slot], st.win_k[b, :, slot]),
                             (st8.pend_k[b, :, t], st8.pend_ks[b, :, t], st.pend_k[b, :, t])):
            k8 = I.dequantize(arr, sc)
            kb = O.bf16_to_f64(ref)
            # the INT8 key and the BF16 key of the same FP32 value: within half a step
            # of the row's grid plus a BF16 rounding
            tol = sc.astype(np.float64)[:, None] * (0.5 + 2.0**-18) + np.abs(kb) * 2.0**-8
            assert np.all(np.abs(k8 - kb) <= tol)
    for nm in ("pend_src", "n_pend", "pos"):
        assert np.array_equal(getattr(st8, nm), getattr(st, nm))


def _f32(v):
    return float(np.float32(v))


def _rne(frac):
    """Round a Fraction to the nearest integer, ties to even (exact)."""
    from fractions import Fraction
    fl = frac.numerator // frac.denominator
    rem = frac - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
        fl += 1
    return fl


def test_codes_follow_the_fp32_quotient_and_product_exactly():
    """The code is round-half-even of fp32(x * fp32(127 / amax)).  Cases are searched
    where that differs from a reading with inv = 127 * fp32(1 / amax) or with the
    product taken exactly, and the oracle must give the defined code there; the
    definition is evaluated in exact rational arithmetic."""
    from fractions import Fraction
    rng = synth.rng_np(synth.stream_key("i8", "exact"))
    found = 0
    for trial in range(400):
        a = np.float32(np.exp2(rng.uniform(-3, 3)) * (1 + rng.uniform()))
        inv = np.float32(np.float32(127.0) / a)                     # fp32 quotient
        inv_alt = np.float32(np.float32(127.0) * np.float32(np.float32(1.0) / a))
        k = int(rng.integers(-126, 126))
        for eps_ulps in (-2, -1, 0, 1, 2):
            x = np.float32((k + 0.5) / float(inv))
            x = np.float32(x + eps_ulps * np.spacing(x))
            if abs(float(x)) > float(a):
                continue
            y = Fraction(float(np.float32(x * inv)))                 # fp32 product, exact value
            want = _rne(y)
            alt = _rne(Fraction(float(np.float32(x * inv_alt))))
            exact = _rne(Fraction(float(x)) * Fraction(float(inv)))
            if want == alt and want == exact:
                continue
            row = np.zeros(256, np.float32)
            row[0], row[1] = a, x
            codes, scale = I.quantize_rows(row[None, :])
            assert int(codes[0, 1].view(np.int8)) == want, (a, x)
            assert int(codes[0, 0].view(np.int8)) == _rne(Fraction(float(np.float32(a * inv))))
            assert scale[0] == np.float32(a / np.float32(127.0))
            found += 1
    assert found >= 20
