"""The C ABI library: it loads, exports every declared entry point, and rejects bad
arguments on the host (no GPU needed: validation happens before any launch)."""

import ctypes
import os
import re

import pytest

import swa_memory_anchor_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    inc = os.path.join(ROOT, "include")
    txt = "\n".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc))
                    if f.endswith(".h"))
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(R.LIB_PATH):
        pytest.skip("librma.so not built")
    return R.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(R.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_closed_form_sizes(lib):
    MiB = 1 << 20
    assert R.rma_layer_kv_bytes(1) == 9 * MiB
    assert 8 * R.rma_layer_kv_bytes(1) == 72 * MiB
    assert R.rma_layer_kv_bytes(512) * 8 == 36 * (1 << 30)
    meta = 4 * 1024 * 8 + 256 * (4 * 4 + 4) + 12
    assert R.rma_layer_state_bytes(3) == 3 * (9 * MiB + meta)
    assert R.rma_layer_state_bytes(0) == 0 and R.rma_layer_kv_bytes(-1) == 0


def test_split_policy_and_workspace(lib):
    assert R.rma_decode_splits(512) == 1 and R.rma_decode_workspace_bytes(512) == 0
    assert R.rma_decode_splits(64) == 1 and R.rma_decode_workspace_bytes(64) == 0
    assert R.rma_decode_splits(16) == 4
    assert R.rma_decode_splits(1) == 16
    assert R.rma_decode_workspace_bytes(16) == 16 * 8 * 4 * 4 * 260 * 4


def test_status_strings(lib):
    for s in range(5):
        assert R.rma_status_str(s).startswith("RMA_")


def _state(ptr=16):
    return R._StateC(*([ptr] * 13))


def _norm(ptr=16):
    return R._NormC(ptr, ptr, ptr, ptr, 1e-6, 1e7)


def test_host_validation_rejects_bad_arguments(lib):
    st, nm = _state(), _norm()
    by = ctypes.byref
    # null state / batch out of range / null output
    assert lib.swa_rma_decode_attn(None, 4, 16, 16, by(nm), 16, 16, 16, 16, None, 0, None) == 1
    assert lib.swa_rma_decode_attn(by(st), 0, 16, 16, by(nm), 16, 16, 16, 16, None, 0, None) == 1
    assert lib.swa_rma_decode_attn(by(st), 4, 16, 16, by(nm), None, 16, 16, 16, None, 0, None) == 1
    # misaligned query
    assert lib.swa_rma_decode_attn(by(st), 512, 18, 16, by(nm), 16, 16, 16, 16, None, 0, None) == 2
    # workspace missing or too small at a split batch
    assert lib.swa_rma_decode_attn(by(st), 4, 16, 16, by(nm), 16, 16, 16, 16, None, 0, None) == 3
    assert lib.swa_rma_decode_attn(by(st), 4, 16, 16, by(nm), 16, 16, 16, 16, 16, 100, None) == 3
    assert lib.swa_rma_append(by(st), 0, 16, 16, 16, 16, None, by(nm), None) == 1
    assert lib.swa_rma_append(by(st), 2, 16, 16, 20, 16, None, by(nm), None) == 2
    bad = _state()
    bad.pend_k = None
    assert lib.swa_rma_append(by(bad), 2, 16, 16, 16, 16, None, by(nm), None) == 1
    assert lib.rma_commit_topk(by(bad), 2, None, None) == 1
    assert lib.rma_commit_topk(by(st), -1, None, None) == 1
    assert lib.rma_score(16, -1, 2560, 16, 16, 16, 4, None) == 1
    assert lib.rma_score(16, 0, 2560, 16, 16, 16, 4, None) == 0  # empty is a no-op
    assert lib.rma_score(16, 5, 2559, 16, 16, 16, 4, None) == 1
    assert lib.rma_score(16, 5, 2564, 16, 16, 16, 4, None) == 2
    assert lib.rma_score(24, 5, 2560, 16, 16, 16, 4, None) == 2
    pf = lambda st_, b, n, ws, wsb, q=16: lib.swa_rma_prefill(  # noqa: E731
        st_, b, n, 16, 16, 16, 16, None, q, 16, by(nm), 16, 16, 16, 16, ws, wsb, None)
    need = R.rma_prefill_workspace_bytes(2, 100)
    assert need == 2 * 100 * 4 * 256 * 2
    assert pf(by(st), 2, 0, 16, need) == 1      # no tokens
    assert pf(by(st), 2, 257, 16, 1 << 30) == 1  # more than a pending block
    assert pf(by(st), 2, 100, None, 0) == 3      # no workspace
    assert pf(by(st), 2, 100, 16, need - 1) == 3
    assert pf(by(st), 2, 100, 16, need, q=24) == 2


def test_step_workspace_and_host_validation(lib):
    # the decode's partials, then one counter per sequence at a 256-byte offset
    assert R.rma_step_workspace_bytes(512) == 512 * 4
    assert R.rma_step_workspace_bytes(16) == 16 * 8 * 4 * 4 * 260 * 4 + 16 * 4
    d1 = R.rma_decode_workspace_bytes(1)
    assert R.rma_step_workspace_bytes(1) == (d1 + 255) // 256 * 256 + 4
    assert R.rma_step_workspace_bytes(0) == 0
    st, nm = _state(), _norm()
    by = ctypes.byref
    need = R.rma_step_workspace_bytes(4)
    step = lambda st_, b, ws, wsb, k=16, q=16, score=None: lib.swa_rma_step(  # noqa: E731
        st_, b, k, 16, 16, 16, score, q, 16, by(nm), 16, 16, 16, 16, ws, wsb, None)
    assert step(None, 4, 16, need) == 1
    assert step(by(st), 0, 16, need) == 1
    assert step(by(st), 4, 16, need, k=None) == 1
    assert step(by(st), 4, 16, need, k=20) == 2      # raw key rows are read 8 bytes at a time
    assert step(by(st), 4, 16, need, q=24) == 2
    assert step(by(st), 4, None, 0) == 3             # the counters are always needed
    assert step(by(st), 512, 16, 512 * 4 - 1) == 3
    assert step(by(st), 4, 16, need - 1) == 3
    assert step(by(st), 4, 24, need) == 2
    bad = _state()
    bad.pend_score = None
    assert step(by(bad), 4, 16, need, score=16) == 1  # a score needs somewhere to go
    bad = _state()
    bad.pend_src = None
    assert step(by(bad), 4, 16, need) == 1


def test_multi_call_host_validation(lib):
    job = R._ScoreJobC(16, 16, 16, 16)
    jobs = (R._ScoreJobC * 17)(*([job] * 17))
    assert lib.rma_score_multi(jobs, 0, 256, 2560, 4, None) == 1
    assert lib.rma_score_multi(jobs, 17, 256, 2560, 4, None) == 1   # past RMA_MAX_JOBS
    assert lib.rma_score_multi(None, 2, 256, 2560, 4, None) == 1
    assert lib.rma_score_multi(jobs, 16, 0, 2560, 4, None) == 0     # no rows: a no-op
    bad = (R._ScoreJobC * 2)(job, R._ScoreJobC(24, 16, 16, 16))
    assert lib.rma_score_multi(bad, 2, 256, 2560, 4, None) == 2     # one misaligned job
    assert lib.rma_score_multi(bad, 1, 256, 2559, 4, None) == 1
    # the split scorer path: workspace sizes and the checks made before any launch
    assert lib.rma_score_workspace_bytes(8, 256) == 8 * 256 * 1024
    assert lib.rma_score_workspace_bytes(1, 8192) == 8192 * 1024      # 256 row tiles
    assert lib.rma_score_workspace_bytes(1, 8193) == 0                # 257: one-launch path
    assert lib.rma_score_workspace_bytes(16, 512) == 16 * 512 * 1024
    assert lib.rma_score_workspace_bytes(16, 513) == 0
    assert lib.rma_score_workspace_bytes(0, 256) == 0
    assert lib.rma_score_workspace_bytes(17, 256) == 0
    assert lib.rma_score_workspace_bytes(1, 0) == 0
    need = 2 * 256 * 1024
    assert lib.rma_score_multi_ws(jobs, 0, 256, 2560, 4, 64, need, None) == 1
    assert lib.rma_score_multi_ws(jobs, 17, 256, 2560, 4, 64, need, None) == 1
    assert lib.rma_score_multi_ws(bad, 2, 256, 2560, 4, 64, need, None) == 2
    assert lib.rma_score_multi_ws(jobs, 2, 0, 2560, 4, None, 0, None) == 0   # no rows
    assert lib.rma_score_multi_ws(jobs, 2, 256, 2560, 4, None, need, None) == 3
    assert lib.rma_score_multi_ws(jobs, 2, 256, 2560, 4, 64, need - 1, None) == 3
    assert lib.rma_score_multi_ws(jobs, 2, 256, 2560, 4, 72, need, None) == 2  # misaligned
    st = _state()
    states = (R._StateC * 17)(*([st] * 17))
    assert lib.rma_commit_topk_multi(states, 0, 4, None, None) == 1
    assert lib.rma_commit_topk_multi(states, 17, 4, None, None) == 1
    assert lib.rma_commit_topk_multi(None, 2, 4, None, None) == 1
    assert lib.rma_commit_topk_multi(states, 2, 0, None, None) == 1
    broken = _state()
    broken.pend_src = None
    mixed = (R._StateC * 2)(st, broken)
    assert lib.rma_commit_topk_multi(mixed, 2, 4, None, None) == 1


def test_fp8_state_size_and_host_validation(lib):
    # codes (1 B) + one FP32 scale per K and V row, plus the same metadata
    rows = 2 * 4 * (1024 + 1024 + 256)
    meta = 4 * 1024 * 8 + 256 * (4 * 4 + 4) + 12
    assert R.rma_layer_state_fp8_bytes(3) == 3 * (rows * 260 + meta)
    assert R.rma_layer_state_fp8_bytes(0) == 0
    st8 = R._StateFp8C(*([16] * 19))
    nm = _norm()
    by = ctypes.byref
    assert lib.swa_rma_decode_attn_fp8(None, 4, 16, 16, by(nm), 16, 16, 16, 16, None, 0, None) == 1
    bad = R._StateFp8C(*([16] * 19))
    bad.pend_vs = None  # a missing scale array
    assert lib.swa_rma_decode_attn_fp8(by(bad), 512, 16, 16, by(nm), 16, 16, 16, 16, None, 0,
                                       None) == 1
    mis = R._StateFp8C(*([16] * 19))
    mis.bank_ks = 20  # misaligned scale array
    assert lib.swa_rma_decode_attn_fp8(by(mis), 512, 16, 16, by(nm), 16, 16, 16, 16, None, 0,
                                       None) == 2
    assert lib.swa_rma_decode_attn_fp8(by(st8), 4, 16, 16, by(nm), 16, 16, 16, 16, None, 0,
                                       None) == 3
    assert lib.swa_rma_append_fp8(by(bad), 2, 16, 16, 16, 16, None, by(nm), None) == 1
    assert lib.swa_rma_append_fp8(by(st8), 0, 16, 16, 16, 16, None, by(nm), None) == 1
    assert lib.rma_commit_topk_fp8(by(bad), 2, None, None) == 1
    assert lib.rma_commit_topk_fp8(None, 2, None, None) == 1


def test_int8_entry_points_validate_like_the_fp8_ones(lib):
    st8 = R._StateFp8C(*([16] * 19))
    nm = _norm()
    by = ctypes.byref
    dec = lambda st_, b, ws=None, wsb=0: lib.swa_rma_decode_attn_i8(  # noqa: E731
        st_, b, 16, 16, by(nm), 16, 16, 16, 16, ws, wsb, None)
    assert dec(None, 4) == 1
    bad = R._StateFp8C(*([16] * 19))
    bad.win_vs = None
    assert dec(by(bad), 512) == 1
    mis = R._StateFp8C(*([16] * 19))
    mis.pend_ks = 20
    assert dec(by(mis), 512) == 2
    assert dec(by(st8), 4) == 3          # split batch without a workspace
    assert dec(by(st8), 0) == 1
    app = lambda st_, b, k=16: lib.swa_rma_append_i8(  # noqa: E731
        st_, b, k, 16, 16, 16, None, by(nm), None)
    assert app(by(bad), 2) == 1
    assert app(by(st8), 0) == 1
    assert app(by(st8), 2, k=None) == 1
    assert app(by(st8), 2, k=20) == 2    # raw key rows are read 8 bytes at a time


def test_gdn_state_size_and_host_validation(lib):
    # 32 heads x 128 x 128 matrix entries + 4 convolution inputs of 8192 BF16 channels
    assert R.gdn_layer_state_bytes(3, 0) == 3 * (32 * 128 * 128 * 2 + 4 * 8192 * 2)
    assert R.gdn_layer_state_bytes(1, 1) == 32 * 128 * 128 * 4 + 4 * 8192 * 2
    assert 24 * R.gdn_layer_state_bytes(1, 0) == int(25.5 * (1 << 20))
    assert R.gdn_layer_state_bytes(0, 0) == 0 and R.gdn_layer_state_bytes(2, 7) == 0
    by = ctypes.byref
    st = R._GdnStateC(16, 16)
    pr = R._GdnParamsC(16, 16, 16)
    step = lib.gdn_decode_step
    assert step(None, 4, 0, 16, 16, 16, 16, by(pr), 16, None) == 1
    assert step(by(st), 4, 0, 16, 16, 16, 16, None, 16, None) == 1
    assert step(by(st), 4, 2, 16, 16, 16, 16, by(pr), 16, None) == 1  # unknown dtype
    assert step(by(st), 0, 0, 16, 16, 16, 16, by(pr), 16, None) == 1
    assert step(by(st), 4, 0, None, 16, 16, 16, by(pr), 16, None) == 1
    assert step(by(st), 4, 0, 16, 16, 16, None, by(pr), 16, None) == 1  # no positions
    assert step(by(R._GdnStateC(16, None)), 4, 0, 16, 16, 16, 16, by(pr), 16, None) == 1
    assert step(by(R._GdnStateC(24, 16)), 4, 0, 16, 16, 16, 16, by(pr), 16, None) == 2
    assert step(by(st), 4, 1, 16, 16, 16, 16, by(R._GdnParamsC(20, 16, 16)), 16, None) == 2
    assert step(by(st), 4, 0, 16, 16, 16, 16, by(pr), 40, None) == 2


def test_gdn_prefill_host_validation(lib):
    by = ctypes.byref
    st = R._GdnStateC(16, 16)
    pr = R._GdnParamsC(16, 16, 16)
    pf = lib.gdn_prefill
    assert pf(None, 4, 8, 0, 16, 16, 16, 16, by(pr), 16, None) == 1
    assert pf(by(st), 4, 0, 0, 16, 16, 16, 16, by(pr), 16, None) == 1        # no tokens
    assert pf(by(st), 4, 65537, 0, 16, 16, 16, 16, by(pr), 16, None) == 1    # past the maximum
    assert pf(by(st), 4, 8, 3, 16, 16, 16, 16, by(pr), 16, None) == 1        # unknown dtype
    assert pf(by(st), 0, 8, 0, 16, 16, 16, 16, by(pr), 16, None) == 1
    assert pf(by(st), 4, 8, 0, 16, 16, 16, None, by(pr), 16, None) == 1      # no positions
    assert pf(by(st), 4, 8, 0, 24, 16, 16, 16, by(pr), 16, None) == 2        # misaligned x
    assert pf(by(st), 4, 8, 1, 16, 16, 16, 16, by(pr), 40, None) == 2        # misaligned o


def test_block_graph_rejects_token_counts_that_cannot_end_a_block():
    """A graph that commits ends one pending block: 1..256 tokens (checked before any
    device memory is touched)."""
    from swa_memory_anchor_amd.graph import StreamBlockGraph

    for tokens in (0, 257, 512):
        with pytest.raises(ValueError):
            StreamBlockGraph([], [], [], 1, tokens=tokens, commit=True, device="cpu")
