#!/usr/bin/env python3
"""Benchmark of the HSTU attention layer on one MI355X.

Headline workload: 8 users x 8,192 tokens, 4 heads x 128, bf16, causal, position
(128 buckets) + log-time (128 buckets) bias, LayerNorm and U gating. One step
is one pass of the hot path over that batch: the jagged tile scheduler, the
fused attention kernel and the LayerNorm/gating epilogue (hstu_attn_fwd),
with inputs already resident in HBM.

Metric: algorithmic TFLOP/s = 4 * d * H * (allowed query-key pairs) / step
time, and its fraction of the bf16 dense MFMA peak (2.5 PFLOP/s). The
attention kernel's own time is measured with HIP events recorded around it on
the launch stream (roofline.achieved), in a pass of its own; the step time
(ms_per_step, value) comes from the same number of calls without those events. Other serving variants (KV-cache delta
with paged append, M-FALCON, the jagged training shape, and the full layer with
its f1/f2 products) are reported under
"variants". The fp64 CPU oracle is timed on a bounded sample of the headline
workload for reference (cpu_baseline).

Prints exactly one JSON line on stdout.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FLOP_PER_CU_CYCLE_BF16 = 4096  # dense bf16 MFMA per CU per cycle (256 CUs x 2.4 GHz x 4096 = 2.5 PFLOP/s)
PMC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_causal_B8_L8192_H4_d128_traffic.json")
KERNEL_SOURCES = ("attn_fwd.hip", "tile.h", "common.h", "kernels.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "hstu_jagged_silu_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter runs,
    or None when absent or taken on a different kernel source."""
    try:
        with open(PMC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


BENCH_FULL_EVENTS = {"ms": None}  # step time of bench_full's loop with per-kernel events (for the record)
WARM = {"s": 0.25, "steps": 0}   # minimum warm-up time per timed region; last warm-up run (for the record)
LAST_TIMED = {"ms_with_events": None}  # the last timed() call's pass with per-kernel events


def timed(fn, steps, warmup, torch, n_events=4, warm_s=None):
    """Run fn(events) at least `warmup` times and for at least warm_s seconds
    of wall time (the GPU's clocks settle only after some continuous load).
    With n_events > 0, one pass of `steps` calls records that many HIP events
    inside each call (the per-kernel spans); then `steps` calls without
    events are timed as a whole, since recording events inside a call adds
    GPU-side latency that a caller does not pay. Returns (ms per step of the
    event-free pass, list of per-step event tuples)."""
    warm_s = WARM["s"] if warm_s is None else warm_s
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < warm_s:
        fn(None)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    WARM["steps"], WARM["elapsed"] = n, time.perf_counter() - t0
    import hstu_jagged_silu_amd as hs
    evs = [[hs.HipEvent() for _ in range(n_events)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    LAST_TIMED["ms_with_events"] = None
    if n_events > 0:
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            fn(evs[i])
        end.record()
        torch.cuda.synchronize()
        LAST_TIMED["ms_with_events"] = start.elapsed_time(end) / steps
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        fn(None)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, evs


def sustained_clock(torch, fn, samples=3):
    """Shader clock (MHz) under the step's own load: the mean of amd-smi's
    per-XCD gfx clocks, read `samples` times while fn runs back to back, and
    the median of those reads. Returns (MHz, samples) or (None, reason)."""
    import shutil
    import subprocess
    tool = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    reads = []
    for _ in range(samples):
        try:
            pr = subprocess.Popen([tool, "metric", "-c", "--json"], stdout=subprocess.PIPE,
                                  stderr=subprocess.DEVNULL, text=True)
        except OSError as e:
            return None, f"amd-smi not runnable: {e}"
        n = 0
        while pr.poll() is None:
            fn(None)
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        try:
            data = json.loads(pr.stdout.read())
            gpus = data["gpu_data"] if isinstance(data, dict) else data
            clk = gpus[0]["clock"]
            mhz = [float(v["clk"]["value"]) for k, v in clk.items() if k.startswith("gfx_")]
        except (ValueError, KeyError, IndexError, TypeError) as e:
            return None, f"amd-smi output not parsed: {e}"
        if not mhz or n == 0:
            return None, "amd-smi returned no gfx clock"
        reads.append(sum(mhz) / len(mhz))
    reads.sort()
    return reads[len(reads) // 2], [round(r, 1) for r in reads]


def mean_span(evs, a, b):
    return sum(e[a].elapsed_ms(e[b]) for e in evs) / len(evs)


def graph_replay_ms(fn, steps, warmup, torch):
    """fn() captured once as a HIP graph (after an eager warm-up on a side
    stream), then replayed: ms per replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    ms, _ = timed(lambda ev: graph.replay(), steps, warmup, torch, n_events=0)
    return ms


def dev(torch, x, dt=None):
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.to(dt) if dt is not None else t).cuda()


def bench_full(torch, hs, W, steps, warmup, flags=0):
    inp = W.long_seq()
    bf = torch.bfloat16
    q, k, v, u = (dev(torch, x, bf) for x in (inp.q, inp.k, inp.v, inp.u))
    ts, off = dev(torch, inp.ts), dev(torch, inp.seq_offsets)
    p = hs.LayerParams(num_heads=4, head_dim=128, dtype=bf, pos_tab=dev(torch, inp.tables.pos),
                       time_tab=dev(torch, inp.tables.time), flags=flags)
    y = torch.empty_like(u)
    ws = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_FULL, p, inp.batch, inp.total, inp.max_len),
                     dtype=torch.uint8, device="cuda")
    fn = lambda ev: hs.hstu_attn_fwd(q, k, v, u, ts, off, inp.max_len, p, y=y, workspace=ws, timing_events=ev)
    ms, evs = timed(fn, steps, warmup, torch)
    BENCH_FULL_EVENTS["ms"] = LAST_TIMED["ms_with_events"]
    pairs = 4 * hs.pair_count("full", [int(x) for x in inp.lengths])
    flop = 4 * 128 * pairs
    return inp, ms, evs, flop, fn


def cold_runs(torch, hs, fn, n=10, flush_mib=512):
    """Attention-kernel time with L2 and the Infinity Cache flushed before each
    call (a flush_mib write in between); returns per-call ms."""
    flush = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda")
    out = []
    for i in range(n):
        flush.fill_(i & 0xFF)
        ev = [hs.HipEvent() for _ in range(4)]
        fn(ev)
        torch.cuda.synchronize()
        out.append(ev[1].elapsed_ms(ev[2]))
    del flush
    return out


def bench_cached(torch, hs, W, steps, warmup):
    import numpy as np
    ci = W.kv_cache_delta()
    h = ci.hist
    bf = torch.bfloat16
    p = hs.LayerParams(num_heads=4, head_dim=128, dtype=bf, pos_tab=dev(torch, h.tables.pos),
                       time_tab=dev(torch, h.tables.time))
    cache = hs.PagedKVCache.empty(ci.num_pages, 4, 128, dev(torch, ci.page_table), dtype=bf)
    pre, new = ci.split()
    hs.hstu_kv_append(cache, dev(torch, ci.prefix_offsets()), dev(torch, np.zeros(ci.batch, np.int32)),
                      dev(torch, h.k[pre], bf), dev(torch, h.v[pre], bf), dev(torch, h.ts[pre]), p)
    qn, un, kn, vn = (dev(torch, x[new], bf) for x in (h.q, h.u, h.k, h.v))
    tsn, noff, cl = dev(torch, h.ts[new]), dev(torch, ci.new_offsets()), dev(torch, ci.cache_lens)
    max_total = int((ci.cache_lens + ci.new_lens).max())
    max_new = int(ci.new_lens.max())
    y = torch.empty_like(un)
    ws = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_CACHED, p, ci.batch, len(new), max_total),
                     dtype=torch.uint8, device="cuda")

    def step(ev):
        if ev is not None:
            ev[4].record()
        hs.hstu_kv_append(cache, noff, cl, kn, vn, tsn, p)
        hs.hstu_attn_fwd_cached(qn, un, tsn, noff, cl, max_new, max_total, cache, p, y=y, workspace=ws,
                                timing_events=ev)

    ms, evs = timed(step, steps, warmup, torch, n_events=5)
    # the same step captured once as a HIP graph and replayed: a serving loop
    # at this size is bound by launch latency (4 kernels per step)
    graph_ms = graph_replay_ms(lambda: step(None), steps, warmup, torch)
    pairs = 4 * hs.pair_count("cached", [int(x) for x in ci.new_lens], [int(x) for x in ci.cache_lens])
    flop = 4 * 128 * pairs
    kv_bytes = int(np.sum(ci.cache_lens + ci.new_lens)) * 4 * 128 * 2 * 2
    attn_ms = mean_span(evs, 1, 2)
    append_ms = mean_span(evs, 4, 0)
    append_bytes = len(new) * 4 * 128 * 2 * 2 * 2 + len(new) * 8 * 2   # K and V read and written, ts
    return {
        "workload": ci.name,
        "ms_per_step": round(ms, 4),
        "step": "paged append of the new tokens + cached forward (schedule, attention, split reduce + LN/gate)",
        "attn_kernel_ms": round(attn_ms, 4),
        "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
        "graph_ms_per_step": round(graph_ms, 4),
        "graph_tflops": round(flop / (graph_ms * 1e-3) / 1e12, 2),
        "attn_kernel_tflops": round(flop / (attn_ms * 1e-3) / 1e12, 2),
        "attn_kernel_kv_gbs": round(kv_bytes / (attn_ms * 1e-3) / 1e9, 1),
        "kv_bytes": kv_bytes,
        "append_ms": round(append_ms, 4),
        "append_gbs": round(append_bytes / (append_ms * 1e-3) / 1e9, 1),
        "append_bytes": append_bytes,
        "epilogue_ms": round(mean_span(evs, 2, 3), 4),
        "scheduler_ms": round(mean_span(evs, 0, 1), 4),
        "algorithmic_gflop": round(flop / 1e9, 3),
    }


def bench_kv_cache_8_layers(torch, hs, W, steps, warmup, layers=8):
    """What the KV cache buys: an 8-layer serving step at batch 8 x (8,192
    cached + 128 new tokens), per layer a paged append of the new tokens and
    the cached forward, against recomputing the full causal path over the
    8,320 tokens of every user at each of the 8 layers, on the same kernels.
    Each layer has its own page pool and inputs (device copies of one drawn
    layer), so no layer reads another's data from the caches."""
    import numpy as np
    ci = W.kv_cache_delta()
    h = ci.hist
    bf = torch.bfloat16
    p = hs.LayerParams(num_heads=4, head_dim=128, dtype=bf, pos_tab=dev(torch, h.tables.pos),
                       time_tab=dev(torch, h.tables.time))
    table = dev(torch, ci.page_table)
    base = hs.PagedKVCache.empty(ci.num_pages, 4, 128, table, dtype=bf)
    pre, new = ci.split()
    hs.hstu_kv_append(base, dev(torch, ci.prefix_offsets()), dev(torch, np.zeros(ci.batch, np.int32)),
                      dev(torch, h.k[pre], bf), dev(torch, h.v[pre], bf), dev(torch, h.ts[pre]), p)
    pools = [base] + [hs.PagedKVCache(base.k_pages.clone(), base.v_pages.clone(), base.ts_pages.clone(), table)
                      for _ in range(layers - 1)]
    new_rows = [tuple(dev(torch, x[new], bf) for x in (h.q, h.u, h.k, h.v)) for _ in range(1)]
    new_rows += [tuple(t.clone() for t in new_rows[0]) for _ in range(layers - 1)]
    tsn, noff, cl = dev(torch, h.ts[new]), dev(torch, ci.new_offsets()), dev(torch, ci.cache_lens)
    max_total = int((ci.cache_lens + ci.new_lens).max())
    max_new = int(ci.new_lens.max())
    ys = [torch.empty_like(r[1]) for r in new_rows]
    ws = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_CACHED, p, ci.batch, len(new), max_total),
                     dtype=torch.uint8, device="cuda")

    def cached_step(ev=None):
        for pool, (qn, un, kn, vn), y in zip(pools, new_rows, ys):
            hs.hstu_kv_append(pool, noff, cl, kn, vn, tsn, p)
            hs.hstu_attn_fwd_cached(qn, un, tsn, noff, cl, max_new, max_total, pool, p, y=y, workspace=ws)

    cached_ms, _ = timed(cached_step, steps, warmup, torch, n_events=0)
    cached_graph_ms = graph_replay_ms(lambda: cached_step(None), steps, warmup, torch)

    # the full causal path over the whole 8,320 tokens of every user, per layer
    full_in = [tuple(dev(torch, x, bf) for x in (h.q, h.k, h.v, h.u))]
    full_in += [tuple(t.clone() for t in full_in[0]) for _ in range(layers - 1)]
    ts_all, off_all = dev(torch, h.ts), dev(torch, h.seq_offsets)
    yf = [torch.empty_like(f[3]) for f in full_in]
    wsf = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_FULL, p, ci.batch, h.total, h.max_len),
                      dtype=torch.uint8, device="cuda")

    def full_step(ev=None):
        for (q, k, v, u), y in zip(full_in, yf):
            hs.hstu_attn_fwd(q, k, v, u, ts_all, off_all, h.max_len, p, y=y, workspace=wsf)

    full_ms, _ = timed(full_step, steps, warmup, torch, n_events=0)
    full_graph_ms = graph_replay_ms(lambda: full_step(None), max(5, steps // 5), warmup, torch)
    cached_flop = layers * 4 * 128 * 4 * hs.pair_count("cached", [int(x) for x in ci.new_lens],
                                                       [int(x) for x in ci.cache_lens])
    full_flop = layers * 4 * 128 * 4 * hs.pair_count("full", [int(x) for x in h.lengths])
    del full_in, yf, wsf, pools, new_rows
    return {
        "workload": f"{layers} layers x {ci.name}",
        "layers": layers,
        "cached_step": "per layer: paged append of 128 new tokens per user + cached forward over 8,320 keys",
        "full_step": "per layer: full causal forward over 8 users x 8,320 tokens",
        "cached_ms_per_step": round(cached_ms, 4),
        "cached_graph_ms_per_step": round(cached_graph_ms, 4),
        "full_ms_per_step": round(full_ms, 4),
        "full_graph_ms_per_step": round(full_graph_ms, 4),
        "latency_ratio_full_over_cached": round(full_ms / cached_ms, 2),
        "latency_ratio_graphs": round(full_graph_ms / cached_graph_ms, 2),
        "cached_algorithmic_gflop": round(cached_flop / 1e9, 3),
        "full_algorithmic_gflop": round(full_flop / 1e9, 3),
        "pages_context": "the pages report a 5.93x latency reduction for an 8-layer model at this shape with every "
                         "history cached, on other hardware and against their own full path (context, not a target)",
    }


def bench_mfalcon(torch, hs, W, steps, warmup):
    ci = W.mfalcon_scoring()
    inp = ci.inputs
    bf = torch.bfloat16
    q, k, v, u = (dev(torch, x, bf) for x in (inp.q, inp.k, inp.v, inp.u))
    ts, off, nc = dev(torch, inp.ts), dev(torch, inp.seq_offsets), dev(torch, ci.num_candidates)
    p = hs.LayerParams(num_heads=4, head_dim=128, dtype=bf, pos_tab=dev(torch, inp.tables.pos),
                       time_tab=dev(torch, inp.tables.time))
    y = torch.empty_like(u)
    ws = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_MFALCON, p, inp.batch, inp.total, inp.max_len),
                     dtype=torch.uint8, device="cuda")
    fn = lambda ev: hs.hstu_mfalcon_fwd(q, k, v, u, ts, off, nc, inp.max_len, p, y=y, workspace=ws,
                                        timing_events=ev)
    ms, evs = timed(fn, steps, warmup, torch)
    pairs = 4 * hs.pair_count("mfalcon", [int(x) for x in ci.hist_lens], [int(x) for x in ci.num_candidates])
    flop = 4 * 128 * pairs
    naive_pairs = 4 * sum(int(m) * hs.pair_count("full", [int(n) + 1]) for n, m in zip(ci.hist_lens, ci.num_candidates))
    attn_ms = mean_span(evs, 1, 2)
    return {
        "workload": ci.name,
        "ms_per_step": round(ms, 4),
        "attn_kernel_ms": round(attn_ms, 4),
        "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
        "attn_kernel_tflops": round(flop / (attn_ms * 1e-3) / 1e12, 2),
        "algorithmic_gflop": round(flop / 1e9, 3),
        "per_candidate_recompute_gflop": round(4 * 128 * naive_pairs / 1e9, 1),
    }


def bench_mfalcon_paged(torch, hs, W, steps, warmup):
    """M-FALCON with the history in the paged cache: only candidate rows are computed."""
    import numpy as np
    ci = W.mfalcon_scoring()
    inp = ci.inputs
    bf = torch.bfloat16
    hist, cand = ci.split()
    num_pages, table = ci.history_pages(8)
    p = hs.LayerParams(num_heads=4, head_dim=128, dtype=bf, pos_tab=dev(torch, inp.tables.pos),
                       time_tab=dev(torch, inp.tables.time))
    cache = hs.PagedKVCache.empty(num_pages, 4, 128, dev(torch, table), dtype=bf)
    hs.hstu_kv_append(cache, dev(torch, W.offsets_from_lengths(ci.hist_lens)),
                      dev(torch, np.zeros(len(ci.hist_lens), np.int32)), dev(torch, inp.k[hist], bf),
                      dev(torch, inp.v[hist], bf), dev(torch, inp.ts[hist]), p)
    q, k, v, u = (dev(torch, x[cand], bf) for x in (inp.q, inp.k, inp.v, inp.u))
    ts, coff, hl = dev(torch, inp.ts[cand]), dev(torch, W.offsets_from_lengths(ci.num_candidates)), \
        dev(torch, ci.hist_lens)
    max_cand, max_hist = int(ci.num_candidates.max()), int(ci.hist_lens.max())
    y = torch.empty_like(u)
    ws = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_MFALCON_CACHED, p, len(ci.hist_lens), len(cand), max_hist),
                     dtype=torch.uint8, device="cuda")
    fn = lambda ev: hs.hstu_mfalcon_fwd_cached(q, k, v, u, ts, coff, hl, max_cand, max_hist, cache, p, y=y,
                                               workspace=ws, timing_events=ev)
    ms, evs = timed(fn, steps, warmup, torch)
    graph_ms = graph_replay_ms(lambda: fn(None), steps, warmup, torch)
    # candidate pairs only: each candidate sees its user's history and itself
    pairs = 4 * sum(int(m) * (int(n) + 1) for n, m in zip(ci.hist_lens, ci.num_candidates))
    flop = 4 * 128 * pairs
    attn_ms = mean_span(evs, 1, 2)
    kv_bytes = int(ci.hist_lens.sum()) * 4 * 128 * 2 * 2
    return {
        "workload": ci.name + "_paged_history",
        "ms_per_step": round(ms, 4),
        "attn_kernel_ms": round(attn_ms, 4),
        "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
        "graph_ms_per_step": round(graph_ms, 4),
        "graph_tflops": round(flop / (graph_ms * 1e-3) / 1e12, 2),
        "attn_kernel_tflops": round(flop / (attn_ms * 1e-3) / 1e12, 2),
        "attn_kernel_kv_gbs": round(kv_bytes / (attn_ms * 1e-3) / 1e9, 1),
        "algorithmic_gflop": round(flop / 1e9, 3),
        "epilogue_ms": round(mean_span(evs, 2, 3), 4),
        "scheduler_ms": round(mean_span(evs, 0, 1), 4),
    }


def bench_training_shape(torch, hs, W, steps, warmup):
    inp = W.training_shape()
    bf = torch.bfloat16
    q, k, v, u = (dev(torch, x, bf) for x in (inp.q, inp.k, inp.v, inp.u))
    ts, off = dev(torch, inp.ts), dev(torch, inp.seq_offsets)
    p = hs.LayerParams(num_heads=4, head_dim=128, dtype=bf, pos_tab=dev(torch, inp.tables.pos),
                       time_tab=dev(torch, inp.tables.time))
    y = torch.empty_like(u)
    ws = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_FULL, p, inp.batch, inp.total, inp.max_len),
                     dtype=torch.uint8, device="cuda")
    fn = lambda ev: hs.hstu_attn_fwd(q, k, v, u, ts, off, inp.max_len, p, y=y, workspace=ws, timing_events=ev)
    ms, evs = timed(fn, steps, warmup, torch)
    graph_ms = graph_replay_ms(lambda: fn(None), steps, warmup, torch)
    flop = 4 * 128 * 4 * hs.pair_count("full", [int(x) for x in inp.lengths])
    attn_ms = mean_span(evs, 1, 2)
    return {
        "workload": inp.name,
        "total_tokens": inp.total,
        "ms_per_step": round(ms, 4),
        "scheduler_ms": round(mean_span(evs, 0, 1), 4),
        "attn_kernel_ms": round(attn_ms, 4),
        "epilogue_ms": round(mean_span(evs, 2, 3), 4),
        "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
        "graph_ms_per_step": round(graph_ms, 4),
        "graph_tflops": round(flop / (graph_ms * 1e-3) / 1e12, 2),
        "attn_kernel_tflops": round(flop / (attn_ms * 1e-3) / 1e12, 2),
        "algorithmic_gflop": round(flop / 1e9, 3),
    }


def _bench_backward(torch, hs, W, inp, steps, warmup):
    """hstu_attn_bwd: recomputed forward, norm backward, attention backward."""
    bf = torch.bfloat16
    H, d = inp.num_heads, inp.head_dim
    q, k, v, u = (dev(torch, x, bf) for x in (inp.q, inp.k, inp.v, inp.u))
    ts, off = dev(torch, inp.ts), dev(torch, inp.seq_offsets)
    dy = dev(torch, W.upstream_grad(81, inp.u.shape), bf)
    w, b = W.affine_terms(82, H * d)
    p = hs.LayerParams(num_heads=H, head_dim=d, dtype=bf, pos_tab=dev(torch, inp.tables.pos),
                       time_tab=dev(torch, inp.tables.time), ln_w=dev(torch, w), ln_b=dev(torch, b))
    ws = torch.empty(hs.hstu_workspace_size(hs.HSTU_FN_FULL_BWD, p, inp.batch, inp.total, inp.max_len),
                     dtype=torch.uint8, device="cuda")
    fn = lambda ev: hs.hstu_attn_bwd(q, k, v, u, ts, off, inp.max_len, dy, p, workspace=ws, timing_events=ev)
    ms, evs = timed(fn, steps, warmup, torch)
    pairs = H * hs.pair_count("full", [int(x) for x in inp.lengths])
    bwd_flop = 5 * 2 * d * pairs      # S recomputed, dP, dV, dQ, dK: five products of 2*d FLOP per pair
    fwd_ms, ln_ms, attn_ms = mean_span(evs, 0, 1), mean_span(evs, 1, 2), mean_span(evs, 2, 3)
    # the same backward on the forward's workspace (HSTU_FLAG_SAVED_FORWARD):
    # no recomputed forward, the norm backward reads the forward's norm-ready store
    ps = hs.LayerParams(num_heads=H, head_dim=d, dtype=bf, pos_tab=p.pos_tab, time_tab=p.time_tab, ln_w=p.ln_w,
                        ln_b=p.ln_b, flags=hs.HSTU_FLAG_SAVED_FORWARD)
    hs.hstu_attn_fwd(q, k, v, u, ts, off, inp.max_len, ps, workspace=ws)
    fn_s = lambda ev: hs.hstu_attn_bwd(q, k, v, u, ts, off, inp.max_len, dy, ps, workspace=ws, timing_events=ev)
    ms_s, evs_s = timed(fn_s, steps, 0, torch)
    saved = {"ms_per_step": round(ms_s, 4), "schedule_ms": round(mean_span(evs_s, 0, 1), 4),
             "norm_backward_ms": round(mean_span(evs_s, 1, 2), 4),
             "attention_backward_ms": round(mean_span(evs_s, 2, 3), 4)}
    return {
        "workload": inp.name,
        "total_tokens": inp.total,
        "ms_per_step": round(ms, 4),
        "forward_recompute_ms": round(fwd_ms, 4),
        "norm_backward_ms": round(ln_ms, 4),
        "attention_backward_ms": round(attn_ms, 4),
        "attention_backward_tflops": round(bwd_flop / (attn_ms * 1e-3) / 1e12, 2),
        "attention_backward_pct_bf16_peak": round(100 * bwd_flop / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "algorithmic_gflop": round(bwd_flop / 1e9, 3),
        "norm_backward_gbs": round(inp.total * H * d * (4 + 2 + 2 + 2 + 2) / (ln_ms * 1e-3) / 1e9, 1),
        "saved_forward": saved,
    }


def bench_backward_training(torch, hs, W, steps, warmup):
    return _bench_backward(torch, hs, W, W.training_shape(), steps, warmup)


def bench_backward_long(torch, hs, W, steps, warmup):
    return _bench_backward(torch, hs, W, W.long_seq(), steps, warmup)


def bench_layer(torch, hs, W, steps, warmup, products=0):
    """Full layer: f1 + SiLU (hipBLASLt, or the library's own MFMA product), attention, f2."""
    inp = W.full_layer()
    bf = torch.bfloat16
    H, d, E = inp.num_heads, inp.head_dim, inp.x.shape[1]
    x, w1, w2 = dev(torch, inp.x, bf), dev(torch, inp.w1, bf), dev(torch, inp.w2, bf)
    ts, off = dev(torch, inp.ts), dev(torch, inp.seq_offsets)
    p = hs.LayerParams(num_heads=H, head_dim=d, dtype=bf, pos_tab=dev(torch, inp.tables.pos),
                       time_tab=dev(torch, inp.tables.time))
    out = torch.empty_like(x)
    ws = torch.empty(hs.hstu_layer_workspace_size(p, E, len(inp.lengths), inp.total, inp.max_len), dtype=torch.uint8,
                     device="cuda")
    fn = lambda ev: hs.hstu_layer_fwd(x, w1, w2, ts, off, inp.max_len, p, out=out, workspace=ws, timing_events=ev,
                                      products=products)
    ms, evs = timed(fn, steps, warmup, torch)
    T, HD = inp.total, H * d
    f1_flop, f2_flop = 2 * T * E * 4 * HD, 2 * T * HD * E
    attn_flop = 4 * d * H * hs.pair_count("full", [int(x) for x in inp.lengths])
    f1_ms, attn_ms, f2_ms = mean_span(evs, 0, 1), mean_span(evs, 1, 2), mean_span(evs, 2, 3)
    return {
        "workload": inp.name,
        "products": {0: "hipBLASLt", 1: "own MFMA kernel", 2: "own f1 (fused SiLU/split) + hipBLASLt f2"}[products],
        "total_tokens": T,
        "ms_per_step": round(ms, 4),
        "tflops": round((f1_flop + f2_flop + attn_flop) / (ms * 1e-3) / 1e12, 2),
        "f1_silu_ms": round(f1_ms, 4),
        "f1_tflops": round(f1_flop / (f1_ms * 1e-3) / 1e12, 2),
        "attention_ms": round(attn_ms, 4),
        "attention_tflops": round(attn_flop / (attn_ms * 1e-3) / 1e12, 2),
        "f2_ms": round(f2_ms, 4),
        "f2_tflops": round(f2_flop / (f2_ms * 1e-3) / 1e12, 2),
        "algorithmic_gflop": {"f1": round(f1_flop / 1e9, 1), "attention": round(attn_flop / 1e9, 1),
                              "f2": round(f2_flop / 1e9, 1)},
    }


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(inp, rows, users):
    """The fp64 oracle on rows 0..rows-1 of each of the first `users` users (all
    heads, N = 8,192): exactly those rows of the headline workload. Returns the
    cpu_baseline object."""
    import numpy as np
    import oracle
    L = int(inp.lengths[0])
    off = inp.seq_offsets
    t0 = time.perf_counter()
    for b in range(users):
        sl = slice(int(off[b]), int(off[b]) + rows)
        oracle.hstu_full(inp.q[sl], inp.k[sl], inp.v[sl], inp.u[sl], inp.ts[sl], np.array([0, rows]),
                         inp.tables.pos, inp.tables.time, norm_n=L)
    dt = time.perf_counter() - t0
    flop = users * 4 * 128 * 4 * rows * (rows + 1) // 2
    return {
        "value": round(flop / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(oracle_threads()),
        "kind": "oracle",
        "sample": f"fp64 oracle, rows 0..{rows - 1} of users 0..{users - 1} of the 8x8192 workload, 4 heads, "
                  f"N fixed at {L}; {flop / 1e9:.2f} GFLOP in {dt:.2f} s",
        "seconds": round(dt, 3),
    }


def oracle_per_config(variants):
    """The fp64 oracle timed on the host for each measured configuration: the
    whole configuration where that takes seconds, otherwise a stated subset
    scaled to the whole by its share of the algorithmic FLOP (marked
    extrapolated). gpu_speedup = oracle time of the whole configuration /
    the GPU step time of the variant."""
    import numpy as np
    import oracle
    import workloads as W
    out = {}

    def record(names, fn, timed_gflop, full_gflop, scope):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        whole = dt * full_gflop / timed_gflop
        for name in names:
            r = {"oracle_s": round(dt, 3), "timed_gflop": round(timed_gflop, 3), "scope": scope,
                 "oracle_s_whole_config": round(whole, 3), "extrapolated": timed_gflop != full_gflop}
            if name in variants:
                r["gpu_speedup"] = round(whole / (variants[name]["ms_per_step"] * 1e-3), 1)
            out[name] = r
        log(f"  oracle {names}: {dt:.2f} s ({scope})")

    pairs_full = lambda lengths: sum(int(n) * (int(n) + 1) // 2 for n in lengths)
    t = W.training_shape()
    g = 4 * 128 * 4 * pairs_full(t.lengths) / 1e9
    record(["jagged_training_shape"], lambda: oracle.hstu_full(t.q, t.k, t.v, t.u, t.ts, t.seq_offsets,
                                                               t.tables.pos, t.tables.time), g, g, "whole")
    ci = W.kv_cache_delta()
    h = ci.hist
    _, new = ci.split()
    g = 4 * 128 * 4 * sum(int(m) * int(c) + int(m) * (int(m) + 1) // 2
                          for c, m in zip(ci.cache_lens, ci.new_lens)) / 1e9
    record(["kv_cache_delta"], lambda: oracle.hstu_cached(h.q[new], h.u[new], h.ts[new], h.k, h.v, h.ts,
                                                          h.seq_offsets, ci.cache_lens, ci.new_offsets(),
                                                          h.tables.pos, h.tables.time), g, g, "whole")
    mc = W.mfalcon_scoring()
    mi = mc.inputs
    hl = [int(n) - int(c) for n, c in zip(mi.lengths, mc.num_candidates)]
    mf_gflop = lambda pairs: 4 * 128 * 4 * sum(pairs_full([n]) + int(c) * (n + 1) for n, c in pairs) / 1e9
    e0 = int(mi.seq_offsets[1])
    record(["mfalcon", "mfalcon_paged_history"],
           lambda: oracle.hstu_mfalcon(mi.q[:e0], mi.k[:e0], mi.v[:e0], mi.u[:e0], mi.ts[:e0],
                                       mi.seq_offsets[:2], mc.num_candidates[:1], mi.tables.pos, mi.tables.time),
           mf_gflop(zip(hl[:1], mc.num_candidates[:1])), mf_gflop(zip(hl, mc.num_candidates)),
           "user 0 of the packed [history | candidates] batch, scaled by FLOP (the paged variant returns "
           "the candidate rows of the same computation)")
    li = W.full_layer()
    off = li.seq_offsets
    k = 1
    while k < len(li.lengths) and off[k] < 2048:
        k += 1
    E, HD = li.x.shape[1], li.num_heads * li.head_dim
    layer_gflop = lambda lengths: (2 * sum(lengths) * E * 4 * HD + 4 * li.head_dim * li.num_heads *
                                   pairs_full(lengths) + 2 * sum(lengths) * HD * E) / 1e9
    sub = [int(n) for n in li.lengths[:k]]
    T = int(off[k])
    record(["full_layer", "full_layer_own_products"],
           lambda: oracle.hstu_layer(li.x[:T], li.w1, li.w2, li.ts[:T], off[:k + 1], li.num_heads, li.head_dim,
                                     li.tables.pos, li.tables.time),
           layer_gflop(sub), layer_gflop([int(n) for n in li.lengths]),
           f"users 0..{k - 1} ({T} tokens) of the 16-user layer, scaled by FLOP")
    bt = W.training_shape()
    dy = W.upstream_grad(81, bt.u.shape)
    w, b = W.affine_terms(82, 4 * 128)
    g = 5 * 2 * 128 * 4 * pairs_full(bt.lengths) / 1e9
    record(["backward_training_shape"],
           lambda: oracle.hstu_full_bwd(bt.q, bt.k, bt.v, bt.u, bt.ts, bt.seq_offsets, dy, bt.tables.pos,
                                        bt.tables.time, gamma=w, beta=b), g, g,
           "whole (forward and backward of the fp64 oracle)")
    lq = W.long_seq()
    n = 1024
    dyl = W.upstream_grad(81, lq.u.shape)
    wl, bl = W.affine_terms(82, 4 * 128)
    record(["backward_causal_B8_L8192"],
           lambda: oracle.hstu_full_bwd(lq.q[:n], lq.k[:n], lq.v[:n], lq.u[:n], lq.ts[:n], np.array([0, n]),
                                        dyl[:n], lq.tables.pos, lq.tables.time, gamma=wl, beta=bl),
           5 * 2 * 128 * 4 * pairs_full([n]) / 1e9, 5 * 2 * 128 * 4 * pairs_full(lq.lengths) / 1e9,
           f"the first {n} tokens of user 0 as one sequence, scaled by the pair count")
    return {"cores": int(oracle_threads()), "configs": out}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--warmup-seconds", type=float, default=1.5,
                    help="warm up the headline step for at least this long (on top of --warmup steps)")
    ap.add_argument("--variant-warmup-seconds", type=float, default=0.3)
    ap.add_argument("--no-variants", action="store_true", help="time only the headline workload")
    ap.add_argument("--variants", default="", help="comma-separated subset of the variants to run (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock-read", action="store_true",
                    help="skip the amd-smi clock reads (peak_sustained null); for counter runs, where the "
                         "profiler's preloaded library makes every child process a GPU client")
    ap.add_argument("--cpu-sample-rows", type=int, default=8192)
    ap.add_argument("--cpu-sample-users", type=int, default=3)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB; used to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU sharding is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)

    import torch
    import hstu_jagged_silu_amd as hs
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    log("headline: 8 x 8192, 4 x 128, bf16")
    WARM["s"] = args.warmup_seconds
    inp, ms, evs, flop, step_fn = bench_full(torch, hs, W, args.steps, args.warmup)
    ms_with_events = BENCH_FULL_EVENTS["ms"]
    warm_steps, warm_elapsed = WARM["steps"], WARM["elapsed"]
    WARM["s"] = args.variant_warmup_seconds
    attn_ms = mean_span(evs, 1, 2)
    attn_each = sorted(e[1].elapsed_ms(e[2]) for e in evs)
    attn_median = attn_each[len(attn_each) // 2]
    cold = sorted(cold_runs(torch, hs, step_fn))
    sched_ms = mean_span(evs, 0, 1)
    ln_ms = mean_span(evs, 2, 3)
    value = flop / (ms * 1e-3) / 1e12
    achieved = flop / (attn_ms * 1e-3) / 1e12
    hd = 4 * 128
    # norm-ready store: bf16 deviations + 8 bytes per (token, head) read, U read, Y written (bf16)
    ln_bytes = inp.total * hd * (2 + 2 + 2) + inp.total * 4 * 8
    log(f"step {ms:.4f} ms ({value:.1f} TFLOP/s), attention kernel {attn_ms:.4f} ms ({achieved:.1f} TFLOP/s), "
        f"scheduler {sched_ms:.4f} ms, epilogue {ln_ms:.4f} ms")

    clock_mhz, clock_reads = ((None, "skipped (--no-clock-read)") if args.no_clock_read
                              else sustained_clock(torch, step_fn))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    peak_sustained = None
    if clock_mhz is not None:
        # 32x32x16 bf16 MFMA: 32,768 FLOP per 32 cycles per SIMD, 4 SIMDs per CU
        sus = cus * clock_mhz * 1e6 * FLOP_PER_CU_CYCLE_BF16 / 1e12
        peak_sustained = {"value": round(sus, 1), "unit": "TFLOP/s", "cus": cus, "clock_mhz": round(clock_mhz, 1),
                          "flop_per_cu_cycle": FLOP_PER_CU_CYCLE_BF16, "frac": round(achieved / sus, 4),
                          "clock_reads_mhz": clock_reads,
                          "source": "amd-smi metric -c: mean of the per-XCD gfx clocks, median of 3 reads "
                                    "taken while the headline step ran back to back"}
        log(f"sustained clock {clock_mhz:.0f} MHz -> peak {sus:.0f} TFLOP/s, attention at {achieved / sus:.3f}")
    else:
        log(f"sustained clock not measured: {clock_reads}")

    result = {
        "metric": "HSTU attention TFLOP/s + % bf16 MFMA peak (1 GPU); ms/layer at seq 8192, d=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": {"steps": warm_steps, "seconds": round(warm_elapsed, 3), "min_seconds": args.warmup_seconds},
        "ms_per_step": round(ms, 4),
        "ms_per_layer": round(ms, 4),
        "ms_per_step_with_kernel_events": round(ms_with_events, 4),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Q,K,V,U ~ N(0,1), tables ~ N(0,0.02), exponential timestamp gaps mean 60 s)",
        "config": {"workload": inp.name, "batch": inp.batch, "seq_len": int(inp.lengths[0]), "heads": 4,
                   "head_dim": 128, "rab": "position 128 + log2 time 128 buckets", "mask": "causal",
                   "algorithmic_gflop": round(flop / 1e9, 3)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                     "kernel": "attn_fwd_kernel<bf16,128,full>", "kernel_ms": round(attn_ms, 4),
                     "kernel_ms_median": round(attn_median, 4),
                     "kernel_ms_cold_median": round(cold[len(cold) // 2], 4)},
        "peak_sustained": peak_sustained,
        "kernels_ms": {"scheduler": round(sched_ms, 4), "attention": round(attn_ms, 4),
                       "ln_gate": round(ln_ms, 4)},
        "epilogue": {"bound": "hbm", "achieved_gbs": round(ln_bytes / (ln_ms * 1e-3) / 1e9, 1),
                     "peak_gbs": PEAK_HBM_GBS, "bytes": ln_bytes},
    }
    if not args.no_variants:
        # the same step with the attention output making an fp32 round trip to
        # the norm (the path before the norm-ready store)
        _, ms32, evs32, _, _ = bench_full(torch, hs, W, args.steps, args.warmup, flags=hs.HSTU_FLAG_FP32_NORM_INPUT)
        result["norm_input"] = {
            "norm_ready_store": {"ms_per_step": round(ms, 4), "attention_ms": round(attn_ms, 4),
                                 "norm_ms": round(ln_ms, 4),
                                 "attention_output_bytes": inp.total * hd * 2 + inp.total * 4 * 8},
            "fp32_round_trip": {"ms_per_step": round(ms32, 4), "attention_ms": round(mean_span(evs32, 1, 2), 4),
                                "norm_ms": round(mean_span(evs32, 2, 3), 4),
                                "attention_output_bytes": inp.total * hd * 4},
        }
        log(f"fp32 norm input: step {ms32:.4f} ms, attention {mean_span(evs32, 1, 2):.4f} ms, "
            f"norm {mean_span(evs32, 2, 3):.4f} ms")
    if args.copy_calibration_mib > 0:
        # a plain device-to-device copy of n bytes; a 1 GiB write in between
        # evicts the source from L2 and the 256 MB Infinity Cache first
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        flush.fill_(3)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n
        del src, dst, flush
    if not args.no_variants:
        variants = {}
        for name, fn in (("kv_cache_delta", bench_cached), ("kv_cache_8_layers", bench_kv_cache_8_layers),
                         ("mfalcon", bench_mfalcon),
                         ("mfalcon_paged_history", bench_mfalcon_paged),
                         ("jagged_training_shape", bench_training_shape), ("full_layer", bench_layer),
                         ("full_layer_own_products",
                          lambda torch, hs, W, st, wu: bench_layer(torch, hs, W, st, wu, products=1)),
                         ("full_layer_auto_products",
                          lambda torch, hs, W, st, wu: bench_layer(torch, hs, W, st, wu, products=2)),
                         ("backward_training_shape", bench_backward_training),
                         ("backward_causal_B8_L8192", bench_backward_long)):
            if args.variants and name not in args.variants.split(","):
                continue
            log(f"variant {name}")
            variants[name] = fn(torch, hs, W, args.steps, args.warmup)
            log(f"  {variants[name]}")
        result["variants"] = variants
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_sample_rows} rows of {args.cpu_sample_users} users")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_rows, args.cpu_sample_users)
        log(f"  {result['cpu_baseline']}")
        if not args.no_variants:
            log("oracle per configuration")
            result["oracle_per_config"] = oracle_per_config(result.get("variants", {}))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
