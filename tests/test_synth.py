"""The seeded generators: host and device implementations draw identical bytes."""

import numpy as np
import torch

import synth
from synth import workloads as W


def test_counter_stream_host_equals_torch_slice():
    k = synth.stream_key("t", 1, "x")
    n = 100_003
    ref = synth.normal_bf16_np(k, n, start=123)
    out = torch.empty(n, dtype=torch.bfloat16)
    synth.normal_bf16_torch_(out, k, start=123, chunk=4096)
    assert np.array_equal(out.view(torch.int16).numpy().view(np.uint16), ref)
    # a slice regenerated from its own offset matches the full draw
    assert np.array_equal(synth.normal_bf16_np(k, 500, start=123 + 7000), ref[7000:7500])


def test_counter_stream_near_top_of_index_space():
    k = synth.stream_key("edge")
    start = (1 << 32) - 1000
    ref = synth.normal_bf16_np(k, 1000, start=start)
    out = torch.empty(1000, dtype=torch.int16)
    synth.normal_bf16_torch_(out, k, start=start)
    assert np.array_equal(out.numpy().view(np.uint16), ref)


def test_normal_table_moments():
    x = synth.bf16_bits_to_f32_np(synth.normal_bf16_np(synth.stream_key("m"), 1 << 20))
    assert abs(float(x.mean())) < 5e-3 and abs(float(x.std()) - 1.0) < 5e-3


def test_workload_slices_consistent():
    wl = W.STEADY_B64
    full = torch.empty(3, 4, 256, 256, dtype=torch.bfloat16)
    # a pending-block-sized tensor for the first three sequences
    synth.normal_bf16_torch_(full, W.key(wl, 2, "pend_k"))
    for b in range(3):
        assert np.array_equal(full[b].view(torch.int16).numpy().view(np.uint16),
                              W.kv_np(wl, 2, "pend_k", b))


def test_burst_scores_plant_ties():
    wl = W.Workload("burst_small", batch=4, layers=1, position=32767, gains="ones", src_hi=32512)
    d = W.burst_scores(wl, 0)
    bs, ps = d["bank_score"], d["pend_score"]
    assert bs.shape == (4, 4, 1024) and ps.shape == (4, 256, 4)
    allv = np.concatenate([bs, ps.transpose(0, 2, 1)], axis=-1)
    # at least 5% of values take part in exact ties
    ties = 0
    for b in range(4):
        for g in range(4):
            _, cnt = np.unique(allv[b, g], return_counts=True)
            ties += cnt[cnt > 1].sum()
    assert ties / allv.size > 0.05
    # some segments carry both signed zeros
    sb = np.signbit(allv) & (allv == 0)
    assert sb.any() and ((allv == 0) & ~np.signbit(allv)).any()
    for b in range(4):
        for g in range(4):
            assert len(set(d["bank_src"][b, g])) == 1024
            assert d["bank_src"][b, g].max() < 32512


def test_record_rows_at_positions():
    wl = W.LONG_STREAM_B1
    full = W.record_np(wl, 3, "k_rma", 100, 140)
    rows = W.record_rows_np(wl, 3, "k_rma", [139, 100, 117])
    assert np.array_equal(rows, full[[39, 0, 17]])
    out = torch.empty(40, 4, 256, dtype=torch.bfloat16)
    W.record_torch_(wl, 3, "k_rma", 100, out)
    assert np.array_equal(out.view(torch.int16).numpy().view(np.uint16), full)


def test_e4m3_streams_host_equal_torch_and_have_no_nan_codes():
    k = synth.stream_key("synth_test", "e4m3")
    a = synth.core.normal_e4m3_np(k, 70001, start=12345)
    t = torch.empty(70001, dtype=torch.uint8)
    synth.core.normal_e4m3_torch_(t, k, start=12345)
    assert np.array_equal(a, t.numpy())
    assert not np.any((a & 0x7F) == 0x7F)
    v = torch.from_numpy(a.copy()).view(torch.float8_e4m3fn).double().numpy() / 128.0
    assert abs(v.mean()) < 0.02 and abs(v.std() - 1.0) < 0.02
    s = synth.core.row_scale_np(k, 5000, start=99)
    ts = torch.empty(5000)
    synth.core.row_scale_torch_(ts, k, start=99)
    assert np.array_equal(s.view(np.uint32), ts.numpy().view(np.uint32))
    assert s.min() >= 3 / 512 and s.max() < 4 / 512


def test_fp8_workload_slices_consistent():
    wl = W.HEADLINE_B512_FP8
    codes = torch.empty(3, 4, W.BLOCK, 256, dtype=torch.uint8)
    scales = torch.empty(3, 4, W.BLOCK)
    W.kv_fp8_torch_(wl, 1, "pend_v", codes, scales)
    c, s = W.kv_fp8_np(wl, 1, "pend_v", 2)
    assert np.array_equal(codes[2].numpy(), c) and np.array_equal(scales[2].numpy(), s)


def test_prefill_chunk_slices_equal_the_device_fill():
    """A sequence's chunk records and queries drawn on the host are the same bits as
    that sequence's slice of the all-sequence fill (torch, here on the CPU)."""
    wl = W.Workload("prefill_b512", batch=3, layers=8, position=65535, gains="normal")
    C = 5
    rec = torch.empty(3, C, 4, 256, dtype=torch.bfloat16)
    W.prefill_record_torch_(wl, 2, "v_rma", rec)
    q = torch.empty(3, C, 16, 256, dtype=torch.bfloat16)
    W.prefill_q_torch_(wl, 2, q)
    for b in range(3):
        assert np.array_equal(rec[b].view(torch.int16).numpy().view(np.uint16),
                              W.prefill_record_np(wl, 2, "v_rma", b, C))
        assert np.array_equal(q[b].view(torch.int16).numpy().view(np.uint16),
                              W.prefill_q_np(wl, 2, b, C))


def test_planted_ties_on_given_scores():
    """plant_burst_ties keeps the given pending scores except where it plants ties,
    and puts an exact tie run across the 1024th place of every segment."""
    wl = W.Workload("burst_small", batch=8, layers=1, position=32767, gains="ones", src_hi=32512)
    rng = np.random.default_rng(3)
    given = (rng.standard_normal((8, 256, 4)) * 0.32).astype(np.float32)
    given[2, 7] = given[2, 9]  # an equal score row, as a duplicated hidden row gives
    d = W.plant_burst_ties(wl, 0, given)
    bs, ps = d["bank_score"], d["pend_score"]
    assert bs.shape == (8, 4, 1024) and ps.shape == (8, 256, 4)
    zero_seg = 0
    for b in range(8):
        for g in range(4):
            v = np.concatenate([bs[b, g], ps[b, :, g]]).astype(np.float64)
            s = np.sort(v)[::-1]
            assert np.all(s[1020:1028] == s[1023])  # the cut sits inside a run of 8 ties
            if s[1023] == 0.0:
                zero_seg += 1
                z = np.concatenate([bs[b, g], ps[b, :, g]])
                z = z[z == 0]
                assert np.signbit(z).sum() >= 4 and (~np.signbit(z)).sum() >= 4
            else:
                # outside the run, pending scores are the given ones
                keep = ps[b, :, g] != s[1023]
                assert np.array_equal(ps[b, keep, g], given[b, keep, g])
    assert zero_seg == 8  # every fourth segment
    assert np.array_equal(ps[2, 7], ps[2, 9]) or (ps[2, 7] == ps[2, 9]).sum() >= 3
