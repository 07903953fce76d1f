"""Pins of the oracle's size closed forms against the numbers the pages print."""

import json
import os

import numpy as np

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "state_sizes.json")))
MiB = 1 << 20
GiB = 1 << 30


def g(name):
    return GOLD[name]["value"]


def test_geometry_matches_pages():
    assert O.RMA_LAYERS == g("rma_layers")
    assert O.KV_GROUPS == g("kv_groups")
    assert O.Q_HEADS == g("query_heads")
    assert O.HEAD_DIM == g("head_dim")
    assert O.ROPE_DIMS == g("rotary_dims")
    assert [O.HIDDEN, O.SCORER_MID, O.KV_GROUPS] == g("scorer_widths")
    assert O.BANK == g("bank_records_per_group")
    assert O.BLOCK == g("commit_block")


def test_bank_pending_window_sizes():
    assert O.bank_bytes_per_sequence() == g("bank_mib_per_sequence") * MiB == 33554432
    assert O.pending_bytes_per_sequence() == g("pending_mib_per_sequence") * MiB == 8388608
    assert O.window_bytes_per_sequence() == g("window_mib_per_sequence") * MiB == 33554432
    assert (O.bank_bytes_per_sequence() + O.pending_bytes_per_sequence()
            == g("bank_plus_pending_mib") * MiB)
    assert O.kv_bytes_per_sequence() == g("attention_kv_mib_per_sequence") * MiB == 75497472


def test_printed_31_97_is_1023_persisted_positions():
    # 1024 ring slots are allocated; between steps 1023 past positions persist.
    w1023 = O.window_bytes_per_sequence(window=1023) / MiB
    assert round(w1023, 2) == g("window_persisted_mib_printed")
    total = (O.window_bytes_per_sequence(window=1023) + O.bank_bytes_per_sequence()
             + O.pending_bytes_per_sequence()) / MiB
    assert round(total, 2) == g("attention_kv_mib_printed")


def test_source_model_growth_and_reduction():
    per_tok = O.source_kv_bytes_per_token()
    assert per_tok == g("source_kv_kib_per_token") * 1024
    assert per_tok * 64 * 1024 == g("source_kv_gib_at_64k") * GiB
    assert per_tok * 256 * 1024 == g("source_kv_gib_at_256k") * GiB
    red = 100.0 * (1.0 - O.kv_bytes_per_sequence() / (per_tok * 256 * 1024))
    assert round(red, 1) == g("reduction_percent_at_256k")


def test_metadata_reading_fits_printed_totals():
    # 97.76 - 71.97 - 25.50 leaves 0.29 MiB for progress metadata; the per-record
    # score + source reading accounts for it to the printed precision.
    left = g("total_state_mib_printed") - g("attention_kv_mib_printed") - g(
        "recurrent_state_mib_printed")
    assert abs(O.metadata_bytes_per_sequence() / MiB - left) < 0.006


def test_state_size_is_independent_of_position():
    # Every part has a hard cap: the oracle's state arrays have the same sizes
    # whatever position the stream has reached.
    rng = np.random.default_rng(0)
    st = O.new_layer_state(1, window=8, bank=4, block=2, head_dim=64, groups=2)
    sizes0 = {k: v.nbytes for k, v in st.__dict__.items()}
    g1 = np.ones(64)
    for _ in range(23):
        if st.n_pend[0] == st.block:
            st.pend_score[...] = rng.standard_normal(st.pend_score.shape)
            O.commit(st)
        rec = [O.f64_to_bf16(rng.standard_normal((1, 2, 64))) for _ in range(4)]
        O.append(st, *rec, g1, g1, 1e-6, 1e7)
        assert {k: v.nbytes for k, v in st.__dict__.items()} == sizes0
    assert st.pos[0] == 22
