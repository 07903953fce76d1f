"""Benchmark of the SWA||RMA decode step on one MI355X.

One step is the decode-step attention of all 8 SWA||RMA layers for every
sequence of the batch (8 dependent launches of ``swa_rma_decode_attn`` on one
stream; in a model, layer l+1's query needs layer l's output, so layers are not
fused).  The state is the synthetic steady state of the pages' 32K-in + 32K-out
serving shape: full 1024-slot window, full 1024-record bank and a full 256-record
pending block per KV group, BF16, drawn from seeded counter streams directly in
HBM before timing starts.

Prints one JSON line: sequence-steps/s (steps/s x batch), the per-launch
roofline of the attention kernel (algorithmic bytes / measured launch time
against 8 TB/s), and the float64 oracle timed on the host cores on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# per (sequence, layer): window + bank + pending K/V, BF16
STATE_BYTES_PER_UNIT = 2 * 4 * (1024 + 1024 + 256) * 256 * 2
# the same rows held as 256 E4M3 codes and one FP32 scale each
STATE_BYTES_PER_UNIT_FP8 = 2 * 4 * (1024 + 1024 + 256) * (256 + 4)
# per (sequence, layer): one query read for both branches (they alias), two
# outputs, two log-sum-exp rows
IO_BYTES_PER_UNIT = 16 * 256 * 2 + 2 * 16 * 256 * 2 + 2 * 16 * 4
METRIC = "SWA∥RMA decode steps/s ×batch and HBM GB/s (% peak) at batch 512"
TRAFFIC_FILES = {
    "headline_b512": os.path.join(ROOT, "profiles", "decode_attn_headline_b512_traffic.txt"),
    "headline_b512_fp8": os.path.join(ROOT, "profiles",
                                      "decode_attn_fp8_headline_b512_fp8_traffic.txt"),
    "headline_b512_i8": os.path.join(ROOT, "profiles",
                                     "decode_attn_i8_headline_b512_i8_traffic.txt"),
    "gdn_decode_b512": os.path.join(ROOT, "profiles", "gdn_decode_gdn_decode_b512_traffic.txt"),
    "gdn_prefill_b512": os.path.join(ROOT, "profiles", "gdn_prefill_gdn_prefill_b512_traffic.txt"),
    "commit_burst_b512": os.path.join(ROOT, "profiles", "score_commit_burst_b512_traffic.txt"),
    "commit_burst_b512:commit": os.path.join(ROOT, "profiles",
                                             "commit_commit_burst_b512_traffic.txt"),
}
KERNEL_SOURCES = ("swa_memory_anchor_amd/csrc/decode_attn.hip",
                  "swa_memory_anchor_amd/csrc/rma_device.h")
GDN_SOURCES = ("swa_memory_anchor_amd/csrc/gdn.hip", "swa_memory_anchor_amd/csrc/rma_device.h")
SCORE_SOURCES = ("swa_memory_anchor_amd/csrc/score.hip", "swa_memory_anchor_amd/csrc/rma_device.h")
COMMIT_SOURCES = ("swa_memory_anchor_amd/csrc/commit.hip", "swa_memory_anchor_amd/csrc/rma_device.h")


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, units_per_launch: int):
    """HBM bytes per launch from the committed counter summary, if it is current."""
    path = TRAFFIC_FILES.get(workload)
    if path is None or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    sources = (GDN_SOURCES if workload.startswith("gdn") else
               COMMIT_SOURCES if workload.endswith(":commit") else
               SCORE_SOURCES if workload.startswith("commit") else KERNEL_SOURCES)
    if kv.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    if int(kv.get("units_per_launch", -1)) != units_per_launch:
        return None
    return float(kv["hbm_bytes_per_launch"])


def _blas_threads() -> int:
    """Threads the oracle's NumPy/BLAS calls may use on this host."""
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def _host_cores() -> int:
    """CPU cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def with_single_thread(fn, wl, budget_s: float, *extra):
    """Run one oracle baseline twice: with the BLAS pool as wide as the cores this
    process may use (two thirds of the budget; the reported value), then with one
    thread (the rest).  Adds the thread count, the host's cores and CPU model."""
    from threadpoolctl import threadpool_limits

    n = _host_cores()
    with threadpool_limits(limits=n):
        used = _blas_threads()
        res = fn(wl, budget_s * 2.0 / 3.0, *extra)
    with threadpool_limits(limits=1):
        one = fn(wl, budget_s / 3.0, *extra)
    res["cores"] = int(used)
    res["host_cores"] = n
    res["cpu_model"] = _cpu_model()
    res["value_1thread"] = one["value"]
    res["sample_1thread"] = one["sample"]
    return res


def cpu_baseline(wl, budget_s: float, max_units: int):
    """The oracle, untuned, on a bounded sample of (sequence, layer) units."""
    import numpy as np

    import oracle as O
    from oracle import fp8_ref as F
    from synth import workloads as W

    fp8 = wl.extra.get("kv") in ("e4m3", "int8")
    if wl.extra.get("kv") == "int8":
        from oracle import int8_ref as I
        kv_np, deq = W.kv_i8_np, I.dequantize
    else:
        kv_np, deq = W.kv_fp8_np, F.dequantize

    cores = _blas_threads()
    rng = np.random.default_rng(7)
    units = 0
    spent = 0.0
    gains = {}
    # the sample is bounded by oracle time and, since regenerating a unit's 9 MiB of
    # inputs on the host costs more than the oracle itself, by wall time as well
    wall0 = last = time.perf_counter()
    while units < max_units and spent < budget_s and time.perf_counter() - wall0 < 2 * budget_s:
        if time.perf_counter() - last > 15:
            last = time.perf_counter()
            print(f"cpu_baseline: {units} units, {spent:.1f} s oracle time", file=sys.stderr,
                  flush=True)
        b, layer = int(rng.integers(0, wl.batch)), int(rng.integers(0, wl.layers))
        q = W.q_np(wl, layer, b)
        g = gains.setdefault(layer, W.gains(wl, layer))
        if fp8:
            s = {nm: kv_np(wl, layer, nm, b) for nm in W.KV_NAMES}
            t0 = time.perf_counter()
            rows = {nm: deq(*s[nm]) for nm in W.KV_NAMES}
            F.decode_one(list(rows["win_k"]), list(rows["win_v"]), q, g["gq_win"], wl.position,
                         wl.eps, wl.rope_base)
            keys = [np.concatenate([rows["bank_k"][i], rows["pend_k"][i]]) for i in range(4)]
            vals = [np.concatenate([rows["bank_v"][i], rows["pend_v"][i]]) for i in range(4)]
            F.decode_one(keys, vals, q, g["gq_rma"], wl.position, wl.eps, wl.rope_base)
        else:
            s = W.decode_state_np(wl, layer, b)
            t0 = time.perf_counter()
            O.decode_one(list(s["win_k"]), list(s["win_v"]), q, g["gq_win"], s["pos"], wl.eps,
                         wl.rope_base)
            keys = [np.concatenate([s["bank_k"][i], s["pend_k"][i]]) for i in range(4)]
            vals = [np.concatenate([s["bank_v"][i], s["pend_v"][i]]) for i in range(4)]
            O.decode_one(keys, vals, q, g["gq_rma"], s["pos"], wl.eps, wl.rope_base)
        spent += time.perf_counter() - t0
        units += 1
    units_per_s = units / spent
    return {
        "value": units_per_s / wl.layers,
        "unit": "seq-steps/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{units} random (sequence, layer) units of {wl.name} (both branches each), "
                  f"{spent:.1f} s of oracle time within {time.perf_counter() - wall0:.0f} s of "
                  f"wall time (inputs regenerated on the host); value = units/s / {wl.layers} "
                  f"layers",
    }


SCORER_FLOP_PER_ROW = 2 * 2560 * 256 + 2 * 256 * 4
FP32_MATRIX_PEAK_TFLOPS = 157.3
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X's published FP32 vector figure


def _timed(fn, reps, stream):
    """Average ms of fn() over reps calls, with a HIP event pair around each call."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return sum(ms) / len(ms), ms[len(ms) // 2]


def bench_commit_burst(args):
    """Scorer and commit of one 256-token burst per sequence at batch 512, all 8 layers."""
    import numpy as np
    import torch

    import swa_memory_anchor_amd as R
    from synth import workloads as W

    wl = W.COMMIT_BURST_B512
    B, L, dev = wl.batch, wl.layers, "cuda"
    stream = torch.cuda.current_stream()
    rows = B * 256
    H, w1s, w2s, outs, states, saved, keeps = [], [], [], [], [], [], []
    for layer in range(L):
        h = torch.empty(B, 256, 2560, dtype=torch.bfloat16, device=dev)
        W.burst_hidden_torch_(wl, layer, h)
        w1, w2 = W.scorer_weights(wl, layer)
        H.append(h)
        w1s.append(torch.from_numpy(w1).to(dev))
        w2s.append(torch.from_numpy(w2).to(dev))
        outs.append(torch.empty(rows, 4, device=dev))
        st = R.alloc_layer_state(B, dev, zero_kv=False)
        for nm in ("bank_k", "bank_v", "pend_k", "pend_v"):
            W.kv_torch_(wl, layer, nm, getattr(st, nm))
        sc = W.burst_scores(wl, layer)
        for k in ("bank_score", "pend_score", "bank_src", "pend_src", "n_bank", "n_pend", "pos"):
            getattr(st, k).copy_(torch.from_numpy(np.ascontiguousarray(sc[k])).to(dev))
        states.append(st)
        saved.append({k: getattr(st, k).clone() for k in ("bank_score", "bank_src", "n_bank",
                                                          "n_pend")})
        keeps.append(torch.empty(B, 4, 1024, dtype=torch.int32, device=dev))

    def score_all():
        for l in range(L):
            R.rma_score(H[l], rows, 2560, w1s[l], w2s[l], outs[l], 4, stream)

    for _ in range(args.warmup):
        score_all()
    s_avg, s_med = _timed(score_all, args.steps, stream)
    flop = L * rows * SCORER_FLOP_PER_ROW
    tflops = flop / (s_avg / 1e3) / 1e12

    def restore(l):
        for k, v in saved[l].items():
            getattr(states[l], k).copy_(v)

    c_ms = []
    for rep in range(args.warmup + args.steps):
        for l in range(L):
            restore(l)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            R.rma_commit_topk(states[l], B, keeps[l], stream)
            b.record(stream)
            torch.cuda.synchronize()
            if rep >= args.warmup:
                c_ms.append(a.elapsed_time(b))
    admitted = int(sum(int((k >= 1024).sum()) for k in keeps))
    c_avg = sum(c_ms) / len(c_ms)
    # the same 8 commits as one launch (rma_commit_topk_multi), as a block end runs them
    m_ms = []
    for rep in range(args.warmup + args.steps):
        for l in range(L):
            restore(l)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        R.rma_commit_topk_multi(states, B, keeps, stream)
        b.record(stream)
        torch.cuda.synchronize()
        if rep >= args.warmup:
            m_ms.append(a.elapsed_time(b) / L)
    m_avg = sum(m_ms) / len(m_ms)
    cpu = (None if args.no_cpu_baseline else
           with_single_thread(cpu_baseline_commit_burst, wl, min(args.cpu_budget, 20.0)))
    key_bytes = B * 4 * 1280 * 8  # score + source of every candidate
    copy_bytes = admitted / L * 2 * 2 * 512  # K and V rows, read and written
    out_bytes = B * 4 * 1024 * 4  # keep_idx
    return {
        "metric": "commit burst at batch 512: scorer TFLOP/s (FP32 MFMA) and commit time per layer",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s_avg + c_avg * L, 4),
        "higher_is_better": True,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "layers": L, "rows_per_layer": rows},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": FP32_MATRIX_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / FP32_MATRIX_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name, B),
                     "kernel": "score_kernel", "avg_launch_ms": round(s_avg / L, 4)},
        "commit": {"avg_launch_us": round(c_avg * 1e3, 1),
                   "admitted_rows_per_layer": admitted // L,
                   "algorithmic_bytes_per_launch": int(key_bytes + copy_bytes + out_bytes),
                   "gbps": round((key_bytes + copy_bytes + out_bytes) / (c_avg / 1e3) / 1e9, 1),
                   "frac": round((key_bytes + copy_bytes + out_bytes) / (c_avg / 1e3) / 1e9
                                 / HBM_PEAK_GBPS, 4),
                   "traffic": measured_traffic(wl.name + ":commit", B),
                   "multi_layer_us_per_layer": round(m_avg * 1e3, 1),
                   "multi_layer_gbps": round((key_bytes + copy_bytes + out_bytes) / (m_avg / 1e3)
                                             / 1e9, 1)},
        "cpu_baseline": cpu,
    }


def bench_long_stream(args):
    """Batch-1 stream: per token, one step (append + attention + split merge) in all 8
    layers; every 256 tokens the scorer and the commit of all 8 layers (one launch
    each for all layers).

    The first quarter of the stream runs eagerly (warm-up), the second quarter is timed
    eagerly (one fused-step call per layer), the second half is timed as replays of a
    HIP graph holding one whole 256-token block (inputs copied into the graph's static
    buffers before each replay, outside the timed events): blocks alternate between the
    fused-step graph (the reported value) and the graph of separate append, decode and
    merge launches (reported beside it).  Both give the same bits, so the stream is one
    stream whichever graph advances it.  The last 256 tokens time single tokens: a
    one-token fused graph per token, the block's score + commit after the last one."""
    import torch

    import swa_memory_anchor_amd as R
    from swa_memory_anchor_amd.graph import RECORD_NAMES, StreamBlockGraph
    from synth import workloads as W

    wl = W.LONG_STREAM_B1
    L, dev = wl.layers, "cuda"
    n = args.stream_tokens
    assert n % 1024 == 0 and n >= 2048
    stream = torch.cuda.current_stream()
    states = [R.alloc_layer_state(1, dev) for _ in range(L)]
    norms = []
    for l in range(L):
        g = W.gains(wl, l)
        norms.append(R.Norm(*[torch.from_numpy(g[k]).to(dev) for k in
                              ("gq_win", "gk_win", "gq_rma", "gk_rma")], wl.eps, wl.rope_base))
    rec = {nm: torch.empty(L, n, 4, 256, dtype=torch.bfloat16, device=dev)
           for nm in W.RECORD_NAMES}
    q = torch.empty(L, n, 16, 256, dtype=torch.bfloat16, device=dev)
    hid = torch.empty(L, n, 2560, dtype=torch.bfloat16, device=dev)
    w = []
    for l in range(L):
        for nm in W.RECORD_NAMES:
            W.record_torch_(wl, l, nm, 0, rec[nm][l])
        W.stream_q_torch_(wl, l, 0, q[l])
        W.stream_hidden_torch_(wl, l, 0, hid[l])
        w1, w2 = W.scorer_weights(wl, l)
        w.append((torch.from_numpy(w1).to(dev), torch.from_numpy(w2).to(dev)))
    outs = [(torch.empty(1, 16, 256, dtype=torch.bfloat16, device=dev),
             torch.empty(1, 16, device=dev), torch.empty(1, 16, 256, dtype=torch.bfloat16,
                                                         device=dev),
             torch.empty(1, 16, device=dev)) for _ in range(L)]
    ws = R.step_workspace(1, dev)
    lib = R.lib()
    import ctypes

    st_c = [ctypes.byref(R._state_c(s)) for s in states]
    nm_c = [ctypes.byref(R._norm_c(x)) for x in norms]
    sp = stream.cuda_stream
    rp = {nm: [rec[nm][l].data_ptr() for l in range(L)] for nm in W.RECORD_NAMES}
    qp = [q[l].data_ptr() for l in range(L)]
    op = [[o.data_ptr() for o in os_] for os_ in outs]
    wsp, wsn = ws.data_ptr(), ws.numel()

    sws = R.score_workspace(L, 256, dev)

    def commit_block(t):
        # every layer's scores (stage 1 spread over the chip, then the row sums), then
        # every layer's commit in one launch
        R.rma_score_multi_ws([(hid[l, t - 255:t + 1], w[l][0], w[l][1], states[l].pend_score)
                              for l in range(L)], 256, 2560, 4, sws, stream)
        R.rma_commit_topk_multi(states, 1, None, stream)

    def token(t):
        for l in range(L):
            r = [rp[nm][l] + t * 2048 for nm in W.RECORD_NAMES]
            qq = qp[l] + t * 8192
            o = op[l]
            lib.swa_rma_step(st_c[l], 1, r[0], r[1], r[2], r[3], None, qq, qq, nm_c[l], o[0],
                             o[1], o[2], o[3], wsp, wsn, sp)
        if (t + 1) % 256 == 0:
            commit_block(t)

    quarter, half, tail = n // 4, n // 2, 256
    for t in range(quarter):
        token(t)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for t in range(quarter, half):
        token(t)
    b.record(stream)
    torch.cuda.synchronize()
    eager_us = a.elapsed_time(b) * 1e3 / (half - quarter)

    # whole blocks as graph replays, alternating the fused and the separate-launch graph
    # (the separate path's kernels run once eagerly first, so their code is loaded)
    qq, o = qp[0] + (half - 1) * 8192, op[0]
    scratch = R.alloc_layer_state(1, dev)
    sc_c = ctypes.byref(R._state_c(scratch))
    dws = R.decode_workspace(1, dev)
    lib.swa_rma_append(sc_c, 1, *[rp[nm][0] for nm in W.RECORD_NAMES], None, nm_c[0], sp)
    lib.swa_rma_decode_attn(sc_c, 1, qq, qq, nm_c[0], o[0], o[1], o[2], o[3], dws.data_ptr(),
                            dws.numel(), sp)
    blocks = {True: StreamBlockGraph(states, norms, w, 1, fused=True).capture(),
              False: StreamBlockGraph(states, norms, w, 1, fused=False).capture()}

    def load_block(blk, t0):
        for nm, src in zip(RECORD_NAMES, W.RECORD_NAMES):
            blk.rec[nm].copy_(rec[src][:, t0:t0 + 256].unsqueeze(2))
        blk.q_win.copy_(q[:, t0:t0 + 256].unsqueeze(2))
        blk.q_rma.copy_(blk.q_win)
        blk.hidden.copy_(hid[:, t0:t0 + 256].unsqueeze(1))

    graph_ms = {True: 0.0, False: 0.0}
    ntok = {True: 0, False: 0}
    for i, t0 in enumerate(range(half, n - tail, 256)):
        fused = i % 2 == 0
        blk = blocks[fused]
        load_block(blk, t0)
        a.record(stream)
        blk.replay()
        b.record(stream)
        torch.cuda.synchronize()
        graph_ms[fused] += a.elapsed_time(b)
        ntok[fused] += 256
    graph_us = graph_ms[True] * 1e3 / ntok[True]
    separate_us = graph_ms[False] * 1e3 / ntok[False]
    ntok_graph = ntok[True]

    # single tokens: one-token graph (all layers' append + decode) per token
    # (the block's last token: one graph with its step, the scorer and the commit)
    one = StreamBlockGraph(states, norms, w, 1, tokens=1, commit=False).capture()
    one_end = StreamBlockGraph(states, norms, w, 1, tokens=1, commit=True).capture()
    lat = []
    for t in range(n - tail, n):
        g = one_end if (t + 1) % 256 == 0 else one
        for nm, src in zip(RECORD_NAMES, W.RECORD_NAMES):
            g.rec[nm].copy_(rec[src][:, t:t + 1].unsqueeze(2))
        g.q_win.copy_(q[:, t:t + 1].unsqueeze(2))
        g.q_rma.copy_(g.q_win)
        if g is one_end:
            g.hidden.copy_(hid[:, t - 255:t + 1].unsqueeze(1))
        torch.cuda.synchronize()
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        lat.append(a.elapsed_time(b) * 1e3)
    lat_sorted = sorted(lat)
    cpu = (None if args.no_cpu_baseline else
           with_single_thread(cpu_baseline_long_stream, wl, min(args.cpu_budget, 20.0)))
    state_bytes = sum(x.numel() * x.element_size() for x in states[0].__dict__.values())
    return {
        "metric": "batch-1 stream: microseconds per token (8 layers append + decode, "
                  "scorer + commit every 256 tokens)",
        "value": round(graph_us, 2),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": ntok_graph,
        "warmup": half,
        "ms_per_step": round(graph_us / 1e3, 5),
        "higher_is_better": False,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": 1, "layers": L,
                   "positions_timed_graph": [half, n - tail - 1],
                   "positions_timed_eager": [quarter, half - 1],
                   "state_bytes_per_layer": state_bytes,
                   "tokens_per_s": round(1e6 / graph_us, 1),
                   "launch": "one HIP graph per 256-token block (all layers), one fused "
                             "step launch per layer and token"},
        "eager_us_per_token": round(eager_us, 2),
        "separate_launches_us_per_token": round(separate_us, 2),
        "latency_us": {"tokens": tail, "median": round(lat_sorted[tail // 2], 1),
                       "p99": round(lat_sorted[int(0.99 * tail)], 1),
                       "max": round(lat_sorted[-1], 1),
                       "block_end_token": round(lat[-1], 1),
                       "note": "one-token graph per token, synchronised on its own; the "
                               "block's last token runs the scorer and the commit in its "
                               "graph"},
        "cpu_baseline": cpu,
    }


BF16_MATRIX_PEAK_TFLOPS = 2500.0


def bench_prefill(args):
    """Chunked prefill of one 256-token block per sequence in all 8 layers (steady state:
    full window and bank, empty pending block, chunk at positions 65536..65791)."""
    import numpy as np
    import torch

    import swa_memory_anchor_amd as R
    from synth import workloads as W

    wl = W.WORKLOADS[args.workload]
    B, L, C, dev = wl.batch, wl.layers, 256, "cuda"
    stream = torch.cuda.current_stream()
    states, saved, norms, ins, outs = [], [], [], [], []
    for layer in range(L):
        st = R.alloc_layer_state(B, dev, zero_kv=False)
        for nm in W.KV_NAMES:
            W.kv_torch_(wl, layer, nm, getattr(st, nm))
        meta = W.decode_meta(wl, layer)
        meta["n_pend"][:] = 0
        for k, v in meta.items():
            getattr(st, k).copy_(torch.from_numpy(v).to(dev))
        states.append(st)
        saved.append((st.n_pend.clone(), st.pos.clone()))
        g = W.gains(wl, layer)
        norms.append(R.Norm(*[torch.from_numpy(g[k]).to(dev) for k in
                              ("gq_win", "gk_win", "gq_rma", "gk_rma")], wl.eps, wl.rope_base))
        rec = []
        for nm in W.RECORD_NAMES:
            t = torch.empty(B, C, 4, 256, dtype=torch.bfloat16, device=dev)
            W.prefill_record_torch_(wl, layer, nm, t)
            rec.append(t)
        q = torch.empty(B, C, 16, 256, dtype=torch.bfloat16, device=dev)
        W.prefill_q_torch_(wl, layer, q)
        ins.append((rec, q))
        outs.append((torch.empty(B, C, 16, 256, dtype=torch.bfloat16, device=dev),
                     torch.empty(B, C, 16, device=dev),
                     torch.empty(B, C, 16, 256, dtype=torch.bfloat16, device=dev),
                     torch.empty(B, C, 16, device=dev)))
    ws = R.prefill_workspace(B, C, dev)
    torch.cuda.synchronize()

    def reset():
        for l in range(L):
            states[l].n_pend.copy_(saved[l][0])
            states[l].pos.copy_(saved[l][1])

    def step():
        for l in range(L):
            rec, q = ins[l]
            o = outs[l]
            R.swa_rma_prefill(states[l], B, C, rec[0], rec[1], rec[2], rec[3], None, q, q,
                              norms[l], o[0], o[1], o[2], o[3], ws, stream)

    ms = []
    for rep in range(args.warmup + args.steps):
        reset()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        if rep >= args.warmup:
            ms.append(a.elapsed_time(b))
    step_ms = sum(ms) / len(ms)
    # algorithmic flops: token i sees 1024 window keys and 1024 + i + 1 anchor keys;
    # q.k and p.v are 2 * 256 flops each per (key, head)
    keys = sum(2048 + i + 1 for i in range(C))
    flop = B * L * keys * 16 * 256 * 4
    tflops = flop / (step_ms / 1e3) / 1e12
    return {
        "metric": "chunked prefill: tokens/s (256-token chunk per sequence, 8 layers)",
        "value": round(B * C / (step_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "layers": L, "chunk": C,
                   "positions": [65536, 65536 + C - 1]},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                     "peak": BF16_MATRIX_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_MATRIX_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill (write + attention + ring)"},
    }


def bench_gdn(args):
    """One decode step of the 24 Gated DeltaNet layers for every sequence (24 dependent
    launches of gdn_decode_step on one stream): FP16 matrices at batch 512, FP32 at
    batch 1.  The state evolves from step to step, as in a stream."""
    import numpy as np
    import torch

    import oracle.gdn_ref as G
    import swa_memory_anchor_amd as R
    from synth import workloads as W

    wl = W.GDN_DECODE_B512 if args.workload == "gdn_decode_b512" else W.GDN_DECODE_B1
    B, L, dev = wl.batch, wl.layers, "cuda"
    f32 = wl.extra["state"] == "f32"
    dt = torch.float32 if f32 else torch.float16
    stream = torch.cuda.current_stream()
    layers = []
    for layer in range(L):
        st = R.GdnState(torch.empty(B, 32, 128, 128, dtype=dt, device=dev),
                        torch.empty(B, 4, 8192, dtype=torch.bfloat16, device=dev))
        W.gdn_state_torch_(wl, layer, st.S)
        W.gdn_conv_torch_(wl, layer, st.conv)
        x = torch.empty(B, 8192, dtype=torch.bfloat16, device=dev)
        W.gdn_x_torch_(wl, layer, x)
        a, b = W.gdn_gate_inputs(wl, layer)
        p = W.gdn_params(wl, layer)
        prm = R.GdnParams(*[torch.from_numpy(p[k]).to(dev) for k in ("conv_w", "a_log",
                                                                     "dt_bias")])
        layers.append((st, x, torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev),
                       torch.full((B,), wl.position, dtype=torch.int32, device=dev), prm,
                       torch.empty(B, 32, 128, dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()

    def step(ev=None):
        for l, (st, x, a, b, pos, prm, o) in enumerate(layers):
            if ev is not None:
                ev[l][0].record(stream)
            R.gdn_decode_step(st, B, x, a, b, pos, prm, o, stream)
            if ev is not None:
                ev[l][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(L)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    launch_ms = sorted(e[0].elapsed_time(e[1]) for s_ in evs for e in s_)
    avg_launch = sum(launch_ms) / len(launch_ms)
    unit = G.step_bytes_per_unit(4 if f32 else 2)
    bytes_per_launch = B * unit
    achieved = bytes_per_launch / (avg_launch / 1e3) / 1e9
    res = {
        "metric": "GDN decode steps/s ×batch and HBM GB/s (24 Gated DeltaNet layers)",
        "value": round(B / (step_ms / 1e3), 1),
        "unit": "seq-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if f32 else "f16 state, f32 math",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "layers": L, "position": wl.position,
                   "state": wl.extra["state"], "bytes_per_unit": unit,
                   "workgroups_per_launch": B * 32 * (1 if B >= 16 else 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(wl.name, B),
                     "kernel": "gdn_decode_kernel", "avg_launch_ms": round(avg_launch, 4),
                     "median_launch_ms": round(launch_ms[len(launch_ms) // 2], 4),
                     "bytes_per_launch": bytes_per_launch},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = with_single_thread(cpu_baseline_gdn, wl, min(args.cpu_budget, 10.0))
    return res


def cpu_baseline_commit_burst(wl, budget_s: float):
    """The oracle's scorer and commit, untuned, on a bounded sample of one burst.

    Scorer: the float64 chain on the 256 hidden rows of random (sequence, layer)
    pairs, scaled to every row of the burst.  Commit: the selection of random
    (sequence, layer, group) segments on the burst's own scores, plus the copies of
    the admitted K/V rows (into scratch rows of the real size: the copy's cost does
    not depend on the values), scaled to every segment."""
    import numpy as np

    import oracle as O
    from synth import workloads as W

    rng = np.random.default_rng(13)
    B, L = wl.batch, wl.layers
    w = {}
    rows, s_spent = 0, 0.0
    while s_spent < budget_s / 2:
        b, layer = int(rng.integers(0, B)), int(rng.integers(0, L))
        w1, w2 = w.setdefault(layer, W.scorer_weights(wl, layer))
        h = W.burst_hidden_np(wl, layer, b)
        t0 = time.perf_counter()
        O.score(h, w1, w2)
        s_spent += time.perf_counter() - t0
        rows += h.shape[0]
    sc = {0: W.burst_scores(wl, 0)}
    k_src, v_src = np.zeros((2, 256, 256), np.uint16)
    k_dst, v_dst = np.zeros((2, 1024, 256), np.uint16)
    segs, c_spent = 0, 0.0
    while c_spent < budget_s / 2:
        layer = int(rng.integers(0, 2))  # the scores of two layers are enough to sample from
        if layer not in sc:
            sc[layer] = W.burst_scores(wl, layer)
        d = sc[layer]
        b, g = int(rng.integers(0, B)), int(rng.integers(0, 4))
        t0 = time.perf_counter()
        _, moves = O.commit_segment(d["bank_score"][b, g], d["bank_src"][b, g],
                                    int(d["n_bank"][b]), d["pend_score"][b, :, g],
                                    d["pend_src"][b], int(d["n_pend"][b]), 1024)
        for t, slot in moves:
            k_dst[slot] = k_src[t]
            v_dst[slot] = v_src[t]
        c_spent += time.perf_counter() - t0
        segs += 1
    score_s = s_spent / rows * B * 256 * L
    commit_s = c_spent / segs * B * 4 * L
    return {"value": round(score_s + commit_s, 2), "unit": "s/burst", "cores": _blas_threads(),
            "kind": "oracle",
            "score_s_per_burst": round(score_s, 2), "commit_s_per_burst": round(commit_s, 2),
            "sample": f"scorer: {rows} rows ({rows // 256} random (sequence, layer) pairs) in "
                      f"{s_spent:.1f} s, scaled to {B * 256 * L} rows; commit: {segs} random "
                      f"segments in {c_spent:.1f} s, scaled to {B * 4 * L} segments"}


def cpu_baseline_long_stream(wl, budget_s: float):
    """The oracle, untuned, on the batch-1 stream: per token append + decode of one
    layer on a steady-state state (full bank, window wrapped), then one block's
    scorer + commit; scaled to 8 layers and amortised over the 256-token block."""
    import numpy as np

    import oracle as O
    import synth
    from synth import workloads as W

    layer, p0 = 0, 8191
    st = O.new_layer_state(1)
    for nm in ("win_k", "win_v", "bank_k", "bank_v", "pend_k", "pend_v"):
        a = getattr(st, nm)
        a[...] = synth.normal_bf16_np(W.key(wl, "cpu", nm), a.size).reshape(a.shape)
    st.n_bank[0], st.n_pend[0], st.pos[0] = 1024, 0, p0
    st.bank_score[...] = synth.normal_f32_np(W.key(wl, "cpu", "bank_score"), st.bank_score.shape,
                                             0.0, 0.3)
    st.bank_src[...] = np.arange(1024, dtype=np.int32)[None, None, :] * 7
    g = W.gains(wl, layer)
    recs = {nm: W.record_np(wl, layer, nm, p0 + 1, p0 + 257) for nm in W.RECORD_NAMES}
    q = W.stream_q_np(wl, layer, p0 + 1, p0 + 257)
    tok, spent = 0, 0.0
    while tok < 256 and spent < budget_s:
        r = [recs[nm][tok:tok + 1] for nm in W.RECORD_NAMES]
        t0 = time.perf_counter()
        O.append(st, *r, g["gk_win"], g["gk_rma"], wl.eps, wl.rope_base)
        O.decode(st, q[tok:tok + 1], q[tok:tok + 1], g["gq_win"], g["gq_rma"], wl.eps,
                 wl.rope_base)
        spent += time.perf_counter() - t0
        tok += 1
    st.n_pend[0] = 256  # the block as it stands at its end
    w1, w2 = W.scorer_weights(wl, layer)
    h = W.stream_hidden_np(wl, layer, p0 + 1, p0 + 257)
    t0 = time.perf_counter()
    st.pend_score[0] = O.score(h, w1, w2)
    O.commit(st)
    block_s = time.perf_counter() - t0
    ms = wl.layers * (spent / tok + block_s / 256) * 1e3
    return {"value": round(ms, 3), "unit": "ms/token", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{tok} tokens of one layer at positions {p0 + 1}.. in {spent:.1f} s plus "
                      f"one block's scorer + commit ({block_s:.2f} s), x {wl.layers} layers, "
                      f"the block part amortised over 256 tokens"}


def bench_gdn_prefill(args):
    """One 256-token chunk per sequence through the 24 Gated DeltaNet layers (24
    dependent gdn_prefill launches): batch 512 with FP16 matrices, or batch 1 with
    FP32 ones.  Each layer has its own state; the chunk inputs (2 GiB of projected
    inputs and the gates at batch 512) are drawn once and fed to every layer (values
    do not change the work)."""
    import torch

    import swa_memory_anchor_amd as R
    from synth import workloads as W

    wl = W.WORKLOADS[args.workload]
    B, L, C, dev = wl.batch, wl.layers, wl.extra["chunk"], "cuda"
    sdt = torch.float16 if wl.extra["state"] == "f16" else torch.float32
    stream = torch.cuda.current_stream()
    x = torch.empty(B, C, 8192, dtype=torch.bfloat16, device=dev)
    W.gdn_chunk_x_torch_(wl, 0, x)
    a, b = W.gdn_chunk_gates(wl, 0, C)
    a, b = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    pos = torch.full((B,), wl.position, dtype=torch.int32, device=dev)
    o = torch.empty(B, C, 32, 128, dtype=torch.bfloat16, device=dev)
    layers = []
    for layer in range(L):
        st = R.GdnState(torch.empty(B, 32, 128, 128, dtype=sdt, device=dev),
                        torch.empty(B, 4, 8192, dtype=torch.bfloat16, device=dev))
        W.gdn_state_torch_(wl, layer, st.S)
        W.gdn_conv_torch_(wl, layer, st.conv)
        p = W.gdn_params(wl, layer)
        prm = R.GdnParams(*[torch.from_numpy(p[k]).to(dev) for k in ("conv_w", "a_log",
                                                                     "dt_bias")])
        layers.append((st, prm))
    torch.cuda.synchronize()

    def step(ev=None):
        for l, (st, prm) in enumerate(layers):
            if ev is not None:
                ev[l][0].record(stream)
            R.gdn_prefill(st, B, C, x, a, b, pos, prm, o, stream)
            if ev is not None:
                ev[l][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(L)] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for k in range(args.steps):
        step(evs[k])
    t1.record(stream)
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps
    launch_ms = sorted(e[0].elapsed_time(e[1]) for s_ in evs for e in s_)
    avg_launch = sum(launch_ms) / len(launch_ms)
    # per token and value head: the two column sums over the 128 x 128 matrix
    # (2 x 2 flops per element) and the update (3 flops per element)
    flop = B * C * 32 * 128 * 128 * 7
    tflops = flop / (avg_launch / 1e3) / 1e12
    return {
        "metric": "GDN chunked prefill: tokens/s (256-token chunk per sequence, 24 layers)",
        "value": round(B * C / (step_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "dtype": "f16 state, f32 math" if wl.extra["state"] == "f16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "layers": L, "chunk": C,
                   "positions": [wl.position, wl.position + C - 1], "state": wl.extra["state"]},
        "roofline": {"bound": "alu", "achieved": round(tflops, 2), "peak": FP32_VECTOR_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / FP32_VECTOR_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name, B), "kernel": "gdn_prefill_kernel",
                     "avg_launch_ms": round(avg_launch, 4)},
    }


def cpu_baseline_gdn(wl, budget_s: float):
    """The GDN oracle, untuned, on random (sequence, layer) units (all 32 heads each)."""
    import numpy as np

    import oracle.gdn_ref as G
    from synth import workloads as W

    rng = np.random.default_rng(11)
    units, spent = 0, 0.0
    wall0 = time.perf_counter()
    while spent < budget_s and time.perf_counter() - wall0 < 3 * budget_s:
        b, layer = int(rng.integers(0, wl.batch)), int(rng.integers(0, wl.layers))
        dt = np.float16 if wl.extra["state"] == "f16" else np.float32
        st = G.GdnState(np.stack([W.gdn_state_np(wl, layer, b, h) for h in range(32)])[None]
                        .astype(dt), W.gdn_conv_np(wl, layer, b)[None].copy())
        a, bb = W.gdn_gate_inputs(wl, layer)
        p = W.gdn_params(wl, layer)
        x = W.gdn_x_np(wl, layer, b)[None]
        t0 = time.perf_counter()
        G.decode_step(st, x, a[b:b + 1], bb[b:b + 1], p["conv_w"], p["a_log"], p["dt_bias"],
                      [wl.position])
        spent += time.perf_counter() - t0
        units += 1
    return {"value": units / spent / wl.layers, "unit": "seq-steps/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"{units} random (sequence, layer) units of {wl.name} (32 heads each), "
                      f"{spent:.1f} s of oracle time; value = units/s / {wl.layers} layers"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline_b512",
                    choices=["headline_b512", "headline_b512_fp8", "headline_b512_i8",
                             "steady_b64", "batch1",
                             "commit_burst_b512", "long_stream_b1", "prefill_b512",
                             "prefill_b64", "gdn_decode_b512", "gdn_decode_b1",
                             "gdn_prefill_b512", "gdn_prefill_b1"])
    ap.add_argument("--stream-tokens", type=int, default=16384,
                    help="long_stream_b1: tokens streamed (the second half is timed)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time")
    ap.add_argument("--cpu-max-units", type=int, default=6000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the RMA hot path is data parallel over "
              "sequences and needs no exchange, so every GPU would run this same kernel on "
              "its own sequences; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": 1 << 30, "launches": 3}))
        return 0

    import swa_memory_anchor_amd as R
    from synth import workloads as W

    if args.workload == "commit_burst_b512":
        print(json.dumps(bench_commit_burst(args)))
        return 0
    if args.workload == "long_stream_b1":
        print(json.dumps(bench_long_stream(args)))
        return 0
    if args.workload.startswith("prefill"):
        print(json.dumps(bench_prefill(args)))
        return 0
    if args.workload.startswith("gdn_prefill"):
        print(json.dumps(bench_gdn_prefill(args)))
        return 0
    if args.workload.startswith("gdn"):
        print(json.dumps(bench_gdn(args)))
        return 0
    if args.workload == "headline_b512":
        wl = W.HEADLINE_B512
    elif args.workload == "headline_b512_fp8":
        wl = W.HEADLINE_B512_FP8
    elif args.workload == "headline_b512_i8":
        wl = W.HEADLINE_B512_I8
    elif args.workload == "steady_b64":
        wl = W.STEADY_B64
    else:
        wl = W.Workload("batch1", batch=1, layers=8, position=65536, gains="normal")
    B, L = wl.batch, wl.layers
    dev = "cuda"

    i8 = wl.extra.get("kv") == "int8"
    fp8 = wl.extra.get("kv") == "e4m3" or i8  # an 8-bit state: codes + row scales
    attn = (R.swa_rma_decode_attn_i8 if i8 else R.swa_rma_decode_attn_fp8) if fp8 else \
        R.swa_rma_decode_attn
    state_bytes = STATE_BYTES_PER_UNIT_FP8 if fp8 else STATE_BYTES_PER_UNIT
    states, qs, norms, outs = [], [], [], []
    for layer in range(L):
        if fp8:
            st = R.alloc_layer_state_fp8(B, dev)
            fill = W.kv_i8_torch_ if i8 else W.kv_fp8_torch_
            for nm in W.KV_NAMES:
                fill(wl, layer, nm, getattr(st, nm), getattr(st, nm + "s"))
        else:
            st = R.alloc_layer_state(B, dev, zero_kv=False)
            for nm in W.KV_NAMES:
                W.kv_torch_(wl, layer, nm, getattr(st, nm))
        for k, v in W.decode_meta(wl, layer).items():
            getattr(st, k).copy_(torch.from_numpy(v).to(dev))
        q = torch.empty(B, 16, 256, dtype=torch.bfloat16, device=dev)
        W.q_torch_(wl, layer, q)
        g = W.gains(wl, layer)
        nm_ = R.Norm(*[torch.from_numpy(g[k]).to(dev) for k in ("gq_win", "gk_win", "gq_rma",
                                                                "gk_rma")], wl.eps, wl.rope_base)
        o = (torch.empty(B, 16, 256, dtype=torch.bfloat16, device=dev),
             torch.empty(B, 16, dtype=torch.float32, device=dev),
             torch.empty(B, 16, 256, dtype=torch.bfloat16, device=dev),
             torch.empty(B, 16, dtype=torch.float32, device=dev))
        states.append(st)
        qs.append(q)
        norms.append(nm_)
        outs.append(o)
    ws = R.decode_workspace(B, dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(ev=None):
        for layer in range(L):
            o = outs[layer]
            if ev is not None:
                ev[layer][0].record(stream)
            attn(states[layer], B, qs[layer], qs[layer], norms[layer], o[0], o[1], o[2], o[3],
                 ws, stream)
            if ev is not None:
                ev[layer][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, bracketed by synchronisation
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)

    # per-launch durations of the attention call (same stream, separate pass)
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(L)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    launch_ms = [e[0].elapsed_time(e[1]) for s in evs for e in s]
    launch_ms.sort()
    avg_launch_ms = sum(launch_ms) / len(launch_ms)

    ms_per_step = total_ms / args.steps
    value = B * args.steps / (total_ms / 1e3)
    bytes_per_launch = B * (state_bytes + IO_BYTES_PER_UNIT)
    achieved = bytes_per_launch / (avg_launch_ms / 1e3) / 1e9
    traffic = measured_traffic(wl.name, B)

    res = {
        "metric": METRIC if B == 512 else METRIC.replace("at batch 512", f"at batch {B}"),
        "value": round(value, 1),
        "unit": "seq-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int8+bf16" if i8 else "fp8e4m3+bf16") if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": B,
            "layers": L,
            "position": wl.position,
            "kv_format": (("int8" if i8 else "e4m3") + " codes + fp32 row scale") if fp8
                         else "bf16",
            "state_bytes_per_step": B * L * state_bytes,
            "decode_splits": R.rma_decode_splits(B),
            "hbm_gbps_step": round(B * L * (state_bytes + IO_BYTES_PER_UNIT)
                                   / (ms_per_step / 1e3) / 1e9, 1),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": ("decode_attn_q8_kernel<int8>" if i8 else "decode_attn_q8_kernel<e4m3>")
                      if fp8 else "decode_attn_kernel",
            "avg_launch_ms": round(avg_launch_ms, 4),
            "median_launch_ms": round(launch_ms[len(launch_ms) // 2], 4),
            "bytes_per_launch": bytes_per_launch,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = with_single_thread(cpu_baseline, wl, args.cpu_budget,
                                                 args.cpu_max_units)
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
