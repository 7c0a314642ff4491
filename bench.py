"""Benchmark of the PISA forward hot path on one MI355X.

One step = one causal prefill pass over one batch of synthetic input:
key pyramid -> PISA Top-K block selection -> block-sparse attention, on the
128K-token workload (B=1, H=4 MHA, N=131072, d=128, C=64, g=2, K=16, bf16,
N(0, 1/d) entries).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line: tokens/s of the whole step, per-stage times, the
selection-latency comparison with the GPU BSA baseline across N (crossover;
three sweeps: 4 heads at d = 128 with K = 16 and with K = 8, and the pages'
latency shape of 16 query heads per KV head at d = 64, K = 8),
the roofline of the dominant kernel (HIP events on the launch stream) and the
CPU oracle timed on a bounded sample of the same workload (cpu_baseline).
Beside it (not part of the step): the backward of the block-sparse attention
with the step's block lists held fixed, and the GQA decode step.

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--no-sweep] [--no-sweep-g16]
                       [--no-sweep-k8] [--no-cpu] [--no-decode]
                       [--no-backward] [--no-cold] [--cpu-seconds 15] [--calibrate-copy-mb 0]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (select+attn) at 128K d=128; selection ms vs BSA"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
# Packed fp32 instructions are disabled in this build, so vector fp32 FMA
# peaks at 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz.
FP32_UNPACKED_PEAK_TFLOPS = 78.6


# ----------------------------------------------------------------------------
# Algorithmic work (host-side counting; depends on t only, not on the data)
# ----------------------------------------------------------------------------

def level_sizes(n, c):
    sizes = [-(-n // c)]
    while sizes[-1] > 1:
        sizes.append(-(-sizes[-1] // 2))
    return sizes


def descent_counts(n, c, k, force=True):
    """For every query row t of a causal prefill, the dot products the PISA
    descent performs per head, by level: rankable candidates at level l >= 2
    score their two child summaries, rankable leaves score their C raw keys
    (descent_row_counts; the counts depend on t only through its leaf t // C).
    Returns {level: int64 array over t}."""
    import numpy as np
    sizes = level_sizes(n, c)
    L = len(sizes)
    out = {lvl: np.zeros(n, dtype=np.int64) for lvl in range(1, L + 1)}
    for cur in range(sizes[0]):
        t0, t1 = cur * c, min((cur + 1) * c, n)
        for lvl, v in descent_row_counts(n, c, k, t0, force).items():
            out[lvl][t0:t1] = v
    return out


def descent_row_counts(n, c, k, t, force=True):
    """Child rows (levels >= 2) or raw keys (level 1) scored for query row t of
    the causal descent, {level: count}.  Exact, and data-independent: every
    ranked candidate lies strictly left of t's path, so it has all its
    children; only the path node's right child can lie in the future."""
    sizes = level_sizes(n, c)
    L = len(sizes)
    out = {}
    cur = t // c
    cand = 1  # level L: the root's only candidate, node 0
    for lvl in range(L, 0, -1):
        sh = lvl - 1
        lim = cur >> sh
        forced = {lim}
        if force:
            forced |= {0}
            if cur >= 1:
                forced |= {(cur - 1) >> sh}
        if cand > k:
            ranked = cand - len(forced)
            out[lvl] = 2 * ranked if lvl >= 2 else c * ranked
            kept = k
        else:
            out[lvl] = 0
            kept = cand
        if lvl > 1:
            # children of the kept nodes; the path node's right child is in
            # the future when t's path continues through its left child
            cand = 2 * kept - (1 if (cur >> (lvl - 2)) == 2 * lim else 0)
    return out


def source_hash():
    """Hash of the library's kernel sources (to tie stored counter data to them)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hierarchical_block_selection_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            key, val = line.split("=", 1)
            rec[key.strip()] = val.strip()
    if rec.get("source_hash") != source_hash():
        return None
    try:
        return float(rec["fetch_bytes"]) + float(rec["write_bytes"])
    except (KeyError, ValueError):
        return None


def stored_counters(kernel):
    """Per-launch counter figures of `kernel` from the committed rocprofv3
    summary profiles/mfma_<kernel>.txt (MFMA busy fraction, executed MFMA
    flops, VALU busy fraction), if it was taken on the current kernel
    sources; else None."""
    path = os.path.join(ROOT, "profiles", f"mfma_{kernel}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            key, val = line.split("=", 1)
            rec[key.strip()] = val.strip()
    if rec.get("source_hash") != source_hash():
        return None
    try:
        return {"mfma_busy_frac": float(rec["mfma_busy_frac"]),
                "mfma_flops": float(rec["mfma_flops"]),
                "valu_busy_frac": float(rec["valu_busy_frac"])}
    except (KeyError, ValueError):
        return None


def attended_keys(n, c, k):
    import numpy as np
    t = np.arange(n)
    cur = t // c
    return np.where(cur + 1 <= k, t + 1, (k - 1) * c + (t % c) + 1)


# ----------------------------------------------------------------------------
# GPU timing helpers
# ----------------------------------------------------------------------------

def copy_bandwidth(dev, mib=1024, reps=5):
    """GB/s of a plain device-to-device copy of `mib` MiB (bytes read plus
    bytes written over the copy's time): the HBM bandwidth a streaming kernel
    can reach on this GPU, beside the 8 TB/s specification."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * src.numel() * 4 / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def timed_call(fn, reps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def run(args):
    import numpy as np
    import torch

    import hierarchical_block_selection_amd as pisa
    from hierarchical_block_selection_amd.inputs import WORKLOADS, prefill_inputs

    dev = torch.device("cuda:0")
    cfg = WORKLOADS["c4b"]
    prob = pisa.Problem(cfg["batch"], cfg["heads_q"], cfg["heads_kv"], cfg["seq_len"],
                        cfg["head_dim"], block=cfg["block"], topk=cfg["topk"], dtype=cfg["dtype"])
    B, H, N, d, C, K = prob.batch, prob.heads_q, prob.seq_len, prob.head_dim, prob.block, prob.topk
    inp = prefill_inputs(B, H, H, N, d, prob.dtype, seed=cfg["seed"], recipe=cfg["recipe"],
                         device=dev)
    q, k, v = inp.q, inp.k, inp.v
    rows = pisa.pisa_pyramid_layout(N, C)[-1]
    pyr = torch.empty((B, H, rows, d), dtype=torch.float32, device=dev)
    idx = torch.empty((B, H, N, K), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws_sel_n = pisa.pisa_workspace_bytes(prob, "select")
    ws_sel = torch.empty(max(ws_sel_n, 1), dtype=torch.uint8, device=dev)
    ws_att_n = pisa.pisa_workspace_bytes(prob, "attn")
    ws_att = torch.empty(max(ws_att_n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(events=None):
        if events:
            events[0].record(stream)
        pisa.pisa_build_pyramid(prob, k, pyr, stream=stream)
        if events:
            events[1].record(stream)
        pisa.pisa_select(prob, q, k, pyr, idx, None, workspace=ws_sel if ws_sel_n else None,
                         stream=stream, want_score=False)
        if events:
            events[2].record(stream)
        pisa.pisa_block_sparse_attn(prob, q, k, v, idx, out, None,
                                    workspace=ws_att if ws_att_n else None, stream=stream,
                                    want_lse=False)
        if events:
            events[3].record(stream)

    if args.calibrate_copy_mb:
        # A plain elementwise pass of known size (reads and writes
        # calibrate_copy_mb MiB each), launched once so that a counter run
        # sees it beside the kernels it calibrates.
        n_el = args.calibrate_copy_mb * (1 << 20) // 4
        src = torch.ones(n_el, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region 1 (the metric): K steps back to back, two events around
    # them and nothing else recorded inside.
    t0 = time.perf_counter()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_per_step = start.elapsed_time(stop) / args.steps
    # Timed region 2 (the breakdown): the same K steps again with events
    # between the stages and the library's events around every kernel launch
    # (these add about 2% to a step, so they stay out of region 1).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    pisa.pisa_profile_report()  # drop anything recorded earlier
    pisa.pisa_profile_enable(True)
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    pisa.pisa_profile_enable(False)
    kernels = {k: tot / cnt for k, (tot, cnt) in pisa.pisa_profile_report().items()}
    per_step = np.array([e[0].elapsed_time(e[3]) for e in ev])
    # Cold-cache steps: before each, 1 GiB of writes evicts L2 and the 256 MB
    # Infinity Cache; the step itself is bracketed by events on the stream.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for i in range(0 if args.no_cold else 5):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    # The same step replayed from a HIP graph: the library's launch sequence
    # allocates nothing and never waits on the host, so a caller can capture
    # it.  K replays between two events; reported beside the metric, which
    # stays the eager launch sequence.
    graph_ms = None
    if not args.no_graph:
        def gstep():  # on the current stream: the capture stream while capturing
            pisa.pisa_build_pyramid(prob, k, pyr)
            pisa.pisa_select(prob, q, k, pyr, idx, None, workspace=ws_sel if ws_sel_n else None,
                             want_score=False)
            pisa.pisa_block_sparse_attn(prob, q, k, v, idx, out, None,
                                        workspace=ws_att if ws_att_n else None, want_lse=False)

        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            gstep()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            gstep()
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph
    step_stats = {"warm_p10": float(np.percentile(per_step, 10)),
                  "warm_p50": float(np.percentile(per_step, 50)),
                  "warm_p90": float(np.percentile(per_step, 90)),
                  "cold_p50": float(np.median(cold)) if cold else None,
                  "cold_max": float(np.max(cold)) if cold else None,
                  "note": "per-step events of the breakdown region; value is the mean of the "
                          "event-free timed region (warm)"}
    stage = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev]))
             for i, name in enumerate(("pyramid", "select", "attn"))}

    # Algorithmic work of the step (the method's own dot products and bytes).
    per_level = descent_counts(N, C, K)
    L = len(per_level)
    dots_l3 = sum(float(per_level[lvl].sum()) for lvl in range(3, L + 1))
    dots_l2 = float(per_level[2].sum()) if L >= 2 else 0.0
    dots_l1 = float(per_level[1].sum())
    keys = attended_keys(N, C, K)
    sel_flops = 2.0 * d * (dots_l3 + dots_l2 + dots_l1) * H * B
    attn_flops = 4.0 * d * float(keys.sum()) * H * B
    elt = 2 if prob.dtype == torch.bfloat16 else 4
    pyr_bytes = B * H * (N * d * elt + rows * d * 4)
    attn_bytes = B * H * N * d * elt * 4  # Q, K, V read once, O written once
    # Stage 1 scores every child row below a wave's causal bound on the
    # matrix cores (bf16 hi/lo planes of the summaries), far more than the
    # method's dots: with counters on the current sources its roofline is
    # the executed MFMA flops against the bf16 MFMA peak, else the method's
    # dots against the unpacked fp32 ceiling of this build.
    s1c = stored_counters("select_stage1")
    s1_roof = (("mfma", s1c["mfma_flops"], BF16_MFMA_PEAK_TFLOPS, "TFLOP/s",
                "executed dense MFMA flops (counters)") if s1c else
               ("alu", 2.0 * d * dots_l3 * H * B, FP32_UNPACKED_PEAK_TFLOPS, "TFLOP/s",
                "method's intermediate-level dots vs unpacked fp32 FMA"))
    roof_table = {
        "pyramid_chunk": ("hbm", pyr_bytes, HBM_PEAK_GBS, "GB/s", "K read + pyramid written"),
        "select_stage1": s1_roof,
        "select_stage2": ("mfma", 2.0 * d * (dots_l2 + dots_l1) * H * B, BF16_MFMA_PEAK_TFLOPS,
                          "TFLOP/s", "method's leaf and level-2 dots"),
        "select_fused": ("alu", sel_flops, FP32_UNPACKED_PEAK_TFLOPS, "TFLOP/s",
                         "method's dots vs unpacked fp32 FMA"),
        "attn_partial": ("mfma", attn_flops, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s",
                         "4 C d flops per (query head, attended block)"),
        "attn_query": ("alu", attn_flops, FP32_UNPACKED_PEAK_TFLOPS, "TFLOP/s",
                       "eq. (2) flops vs unpacked fp32 FMA"),
        "attn_combine": ("hbm", B * H * N * d * elt, HBM_PEAK_GBS, "GB/s", "O written"),
    }
    copy_gbs = copy_bandwidth(dev)
    kernels_roofline = {}
    for kname, (kb, kw, kp, ku, basis) in roof_table.items():
        if kname in kernels and kernels[kname] > 0:
            ks = 1e9 if ku == "GB/s" else 1e12
            ka = kw / (kernels[kname] * 1e-3) / ks
            kernels_roofline[kname] = {"bound": kb, "achieved": round(ka, 1), "peak": kp,
                                       "unit": ku, "frac": round(ka / kp, 4), "basis": basis}
            if ku == "GB/s":
                kernels_roofline[kname]["frac_of_copy"] = round(ka / copy_gbs, 4)
            kt = stored_traffic(kname)
            if kt is not None:
                # HBM bytes the counters saw (on the current sources) per launch
                tg = kt / (kernels[kname] * 1e-3) / 1e9
                kernels_roofline[kname]["traffic_gbs"] = round(tg, 1)
                kernels_roofline[kname]["traffic_frac_of_copy"] = round(tg / copy_gbs, 4)
            kc = stored_counters(kname)
            if kc:
                kernels_roofline[kname]["mfma_busy_frac"] = kc["mfma_busy_frac"]
                kernels_roofline[kname]["valu_busy_frac"] = kc["valu_busy_frac"]
    dominant = max(kernels, key=kernels.get)
    bound, work, peak, unit, _basis = roof_table.get(dominant,
                                                     ("hbm", 0.0, HBM_PEAK_GBS, "GB/s", ""))
    scale = 1e9 if unit == "GB/s" else 1e12
    achieved = work / (kernels[dominant] * 1e-3) / scale
    traffic = stored_traffic(dominant)
    roof = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": traffic,
            "kernel": dominant, "avg_kernel_ms": kernels[dominant],
            "algorithmic_work": work,
            "work_unit": "bytes" if unit == "GB/s" else "flop"}
    if traffic is not None:
        # the counters' HBM bytes over the same launch time, against the HBM peak
        roof["traffic_gbs"] = traffic / (kernels[dominant] * 1e-3) / 1e9
        roof["traffic_frac_of_hbm_peak"] = roof["traffic_gbs"] / HBM_PEAK_GBS
        roof["traffic_frac_of_copy"] = roof["traffic_gbs"] / copy_gbs
    counters = stored_counters(dominant)
    if counters is not None:
        # SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs), and
        # the MFMA flops the kernel executed (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)
        roof["mfma_busy_frac"] = counters["mfma_busy_frac"]
        roof["mfma_executed_tflops"] = counters["mfma_flops"] / (kernels[dominant] * 1e-3) / 1e12
        roof["valu_busy_frac"] = counters["valu_busy_frac"]

    result = {
        "metric": METRIC,
        "value": B * N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal prefill B=1 H=4 (MHA) N=131072 d=128 C=64 g=2 K=16 "
                               "bf16 N(0,1/d), forced first/prev/current blocks",
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "stages_ms": stage,
        "step_ms": step_stats,
        "kernels_ms": kernels,
        "wall_ms_per_step": wall_ms,
        "graph": None if graph_ms is None else {
            "ms_per_step": graph_ms, "tokens_per_s": B * N / (graph_ms * 1e-3),
            "note": "the same step captured once and replayed K times (launch gaps removed); "
                    "value is the eager launch sequence"},
        "algorithmic": {"select_gflop": sel_flops / 1e9, "attn_gflop": attn_flops / 1e9,
                        "pyramid_mb": pyr_bytes / 1e6, "attn_compulsory_mb": attn_bytes / 1e6,
                        "source_hash": source_hash()},
        "roofline": roof,
        "kernels_roofline": kernels_roofline,
        "hbm_copy_gbs": copy_gbs,
    }

    if not args.no_backward:
        result["backward"] = backward_bench(prob, inp, idx, dev)
    if not args.no_decode:
        result["decode"] = decode_bench(args)
        result["decode"]["frac_of_copy"] = result["decode"]["achieved_gbs"] / copy_gbs
    if not args.no_sweep:
        result["selection_sweep"] = selection_sweep(args)
        if not args.no_sweep_g16:
            # the pages' own latency shape: 16 query heads per KV head, d=64, K=8
            result["selection_sweep_g16"] = selection_sweep(
                args, heads_q=16, heads_kv=1, head_dim=64, topk=8,
                sizes=(16384, 65536, 131072, 262144, 524288, 1048576), seed=4100)
        if not args.no_sweep_k8:
            # one query head per KV head as the default sweep, at the pages' K = 8
            result["selection_sweep_k8"] = selection_sweep(
                args, heads_q=4, heads_kv=4, head_dim=128, topk=8,
                sizes=(16384, 32768, 65536, 131072, 262144), seed=4200)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args, inp, prob)
    return result


def backward_bench(prob, inp, idx, dev):
    """Backward of the block-sparse attention for the timed workload, with the
    block lists of the last timed step held fixed: the forward is run once
    more for out / row_lse, dO is a seeded N(0, 1/d) tensor, and one backward
    (delta, stable sort, main kernel, dk/dv reduce, dq combine) is timed."""
    import torch

    import hierarchical_block_selection_amd as pisa
    from hierarchical_block_selection_amd.inputs import seeded_normal

    B, H, N, d, C = prob.batch, prob.heads_q, prob.seq_len, prob.head_dim, prob.block
    G = prob.heads_q // prob.heads_kv
    out, lse = pisa.pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx)
    dout = seeded_normal(tuple(inp.q.shape), 4017, 1.0 / math.sqrt(d), prob.dtype, dev)
    ws = torch.empty(pisa.pisa_workspace_bytes(prob, "attn_bwd"), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(inp.q), torch.empty_like(inp.k), torch.empty_like(inp.v)

    def bwd():
        pisa.pisa_block_sparse_attn_backward(prob, inp.q, inp.k, inp.v, idx, out, lse, dout,
                                             dq, dk, dv, workspace=ws)

    ms = timed_call(bwd, 5, 2)
    pisa.pisa_profile_report()
    pisa.pisa_profile_enable(True)
    timed_call(bwd, 3, 0)
    pisa.pisa_profile_enable(False)
    kernels = {k: tot / cnt for k, (tot, cnt) in pisa.pisa_profile_report().items()}
    m1 = -(-N // C)
    live = int(((idx >= 0) & (idx < m1)).sum().item())
    cols = live * G  # (row, slot, query head) columns
    elt = 2
    # per column: q, dO read, its dQ contribution written (bf16), lse and D;
    # per leaf block: K and V read, dK and dV written once
    main_bytes = cols * (3 * d * elt + 8) + B * prob.heads_kv * m1 * 4 * C * d * elt
    main_flop = cols * 5 * 2.0 * C * d  # S, dP, dV, dK, dQ products over the block
    main_ms = kernels.get("attn_bwd_main", float("nan"))
    achieved = main_bytes / (main_ms * 1e-3) / 1e9
    traffic = stored_traffic("bwd_main")
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "algorithmic_bytes": main_bytes,
            "mfma_tflops": main_flop / (main_ms * 1e-3) / 1e12}
    if traffic is not None:
        roof["traffic_gbs"] = traffic / (main_ms * 1e-3) / 1e9
        roof["traffic_frac_of_hbm_peak"] = roof["traffic_gbs"] / HBM_PEAK_GBS
    return {
        "ms": ms,
        "kernels_ms": kernels,
        "columns": cols,
        "roofline_main": roof,
        "tokens_per_s": B * N / (ms * 1e-3),
    }


def decode_bench(args):
    """Per-step latency of the GQA decode step: 32 sequences with 131072 cached
    tokens each, 32 query heads over 8 KV heads, d=128, K=16, bf16, pyramid of
    the cache prebuilt; one step = selection + attention for every sequence."""
    import torch

    import hierarchical_block_selection_amd as pisa
    from hierarchical_block_selection_amd.inputs import WORKLOADS, decode_inputs

    cfg = WORKLOADS["c5"]
    dev = torch.device("cuda:0")
    prob = pisa.Problem(cfg["batch"], cfg["heads_q"], cfg["heads_kv"], cfg["seq_len"],
                        cfg["head_dim"], block=cfg["block"], topk=cfg["topk"], dtype=cfg["dtype"])
    inp = decode_inputs(prob.batch, prob.heads_q, prob.heads_kv, prob.seq_len, prob.head_dim,
                        prob.dtype, seed=cfg["seed"], device=dev)
    pyr = pisa.pisa_build_pyramid(prob, inp.k_cache)
    idx = torch.empty((prob.batch, prob.heads_kv, prob.topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(inp.q)
    ws_n = pisa.pisa_workspace_bytes(prob, "decode")
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def step():
        pisa.pisa_decode_step(prob, inp.cache_len, inp.q, inp.k_cache, inp.v_cache, pyr, idx,
                              None, out, None, workspace=ws if ws_n else None)

    ms = timed_call(step, 20, 3)
    # Pyramid upkeep for the token each sequence appends (its leaf and the
    # ancestors rewritten), timed separately: the decode step above reads a
    # pyramid that is current.
    append_ms = timed_call(lambda: pisa.pisa_pyramid_append(prob, inp.cache_len, inp.k_cache, pyr),
                           20, 3)
    # compulsory bytes per step: the level summaries the descent scores, the
    # raw keys of the scored leaves and the K/V rows of the kept leaves
    summaries = 0
    t = prob.seq_len - 1
    cnt = descent_row_counts(prob.seq_len, prob.block, prob.topk, t)
    for lvl, dots in cnt.items():
        if lvl >= 2:
            summaries += dots  # child summaries read (fp32)
    leaf_keys = cnt.get(1, 0)  # raw keys scored
    attn_keys = int(attended_keys(prob.seq_len, prob.block, prob.topk)[t])
    units = prob.batch * prob.heads_kv
    bytes_step = units * (summaries * prob.head_dim * 4 + leaf_keys * prob.head_dim * 2 +
                          2 * attn_keys * prob.head_dim * 2)
    del inp, pyr
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "tokens_per_s": prob.batch / (ms * 1e-3),
            "compulsory_mb": bytes_step / 1e6,
            "achieved_gbs": bytes_step / (ms * 1e-3) / 1e9,
            "pyramid_append_ms": append_ms,
            "workload": "decode B=32 cache=131072 Hq=32 Hkv=8 d=128 C=64 K=16 bf16, "
                        "pyramid prebuilt"}


def selection_sweep(args, heads_q=4, heads_kv=4, head_dim=128, topk=16,
                    sizes=(16384, 32768, 65536, 131072, 262144, 524288), seed=4000):
    """Selection latency (pyramid + selection, attention excluded) of PISA and
    of the GPU BSA baseline for N over `sizes` (default: H=4, d=128, K=16)."""
    import torch

    import hierarchical_block_selection_amd as pisa
    from hierarchical_block_selection_amd.inputs import prefill_inputs

    dev = torch.device("cuda:0")
    only = ({int(x) for x in args.sweep_sizes.split(",")} if args.sweep_sizes else None)
    pts = []
    for i, n in enumerate(sizes):
        if only is not None and n not in only:
            continue  # a subset keeps each size's own seed
        prob = pisa.Problem(1, heads_q, heads_kv, n, head_dim, block=64, topk=topk,
                            dtype=torch.bfloat16)
        inp = prefill_inputs(1, heads_q, heads_kv, n, head_dim, torch.bfloat16,
                             seed=seed + 10 * i, device=dev)
        rows = pisa.pisa_pyramid_layout(n, 64)[-1]
        pyr = torch.empty((1, heads_kv, rows, head_dim), dtype=torch.float32, device=dev)
        idx = torch.empty((1, heads_kv, n, topk), dtype=torch.int32, device=dev)
        ws_s = pisa.pisa_workspace_bytes(prob, "select")
        wsel = torch.empty(max(ws_s, 1), dtype=torch.uint8, device=dev)
        # past 4096 leaf blocks BSA needs a multiple of 4 leaf blocks (its
        # Top-K then takes rows in segments); else PISA is timed alone
        bsa_ok = -(-n // 64) <= 4096 or -(-n // 64) % 4 == 0
        ws_b = pisa.pisa_workspace_bytes(prob, "bsa") if bsa_ok else 0
        wbsa = torch.empty(max(ws_b, 1), dtype=torch.uint8, device=dev)

        def pisa_sel():
            pisa.pisa_build_pyramid(prob, inp.k, pyr)
            pisa.pisa_select(prob, inp.q, inp.k, pyr, idx, None, workspace=wsel if ws_s else None,
                             want_score=False)

        def bsa_sel():
            pisa.pisa_build_pyramid(prob, inp.k, pyr)
            pisa.pisa_bsa_select(prob, inp.q, pyr, idx, None, workspace=wbsa, want_score=False)

        reps = 5 if n <= 65536 else 3
        p_ms = timed_call(pisa_sel, reps, 3)
        b_ms = timed_call(bsa_sel, reps, 3) if bsa_ok else None
        # one more call of each with the library's per-kernel events
        kern = {"bsa": {}}
        for name, fn in (("pisa", pisa_sel), ("bsa", bsa_sel)):
            if name == "bsa" and not bsa_ok:
                continue
            pisa.pisa_profile_enable(True)
            fn()
            torch.cuda.synchronize()
            rep = pisa.pisa_profile_report()
            pisa.pisa_profile_enable(False)
            kern[name] = {k: round(v[0] / v[1], 4) for k, v in rep.items()}
        # BSA's score matrix: row t holds its c + 1 eligible leaves (c = t // C),
        # padded to a multiple of 4, fp32; written by bsa_scores, read by bsa_topk
        c = 64
        m1 = -(-n // c)
        s_bytes = heads_kv * c * sum(4 * ((i + 1 + 3) // 4) * 4 for i in range(m1))
        q_bytes = heads_q * n * head_dim * 2
        idx_bytes = heads_kv * n * topk * 4
        bsa_frac = {}
        if "bsa_scores" in kern["bsa"]:
            bsa_frac["bsa_scores"] = (s_bytes + q_bytes) / (kern["bsa"]["bsa_scores"] * 1e-3) \
                / 1e9 / HBM_PEAK_GBS
        if "bsa_topk" in kern["bsa"]:
            bsa_frac["bsa_topk"] = (s_bytes + idx_bytes) / (kern["bsa"]["bsa_topk"] * 1e-3) \
                / 1e9 / HBM_PEAK_GBS
        pts.append({"N": n, "pisa_ms": p_ms, "bsa_ms": b_ms,
                    "speedup_vs_bsa": b_ms / p_ms if bsa_ok else None,
                    "pisa_kernels_ms": kern["pisa"], "bsa_kernels_ms": kern["bsa"],
                    "bsa_score_matrix_mb": s_bytes / 1e6 if bsa_ok else None,
                    "bsa_hbm_frac": {k: round(v, 3) for k, v in bsa_frac.items()}})
        del wbsa, inp
        torch.cuda.empty_cache()
    cross = None
    timed = [p for p in pts if p["bsa_ms"] is not None]
    for a, b in zip(timed, timed[1:]):
        if a["speedup_vs_bsa"] < 1.0 <= b["speedup_vs_bsa"]:
            la, lb = math.log(a["N"]), math.log(b["N"])
            ra, rb = math.log(a["speedup_vs_bsa"]), math.log(b["speedup_vs_bsa"])
            cross = math.exp(la + (lb - la) * (0 - ra) / (rb - ra))
    if timed and timed[0]["speedup_vs_bsa"] >= 1.0:
        cross = f"<= {timed[0]['N']}"
    if cross is None and timed:
        cross = f"> {timed[-1]['N']}"
    return {"points": pts, "crossover_N": cross,
            # the PISA reading page's order-of-magnitude estimate of the
            # crossover (section 5.2): N/C summaries per query for BSA against
            # g*K*C raw leaf keys for PISA, equal at N = g*K*C^2 for one head;
            # with G query heads per KV head PISA pays it per head (eq. (11)
            # sums per-head LSEs) while this BSA scores one group-summed query
            # (eq. (1) is linear in q), so the balance moves to g*K*C^2*G
            "estimate_N": 2 * topk * 64 * 64 * (heads_q // heads_kv),
            "note": f"timings include pyramid construction (all levels) for both selectors; "
                    f"attention excluded; Hq={heads_q} Hkv={heads_kv}, d={head_dim}, C=64, "
                    f"K={topk}, bf16; bsa_hbm_frac: algorithmic bytes of each BSA kernel "
                    f"(score matrix written / read, queries, leaf ids) over its launch time, "
                    f"as a fraction of {HBM_PEAK_GBS:.0f} GB/s"}


def q_tile_study(args):
    """Stage-2 work decomposition against the Q_tile trade-off of the PISA
    reading page (§5.1, eqs. (12)-(15); Table 4's Q1/Q2/Q4 axis).  In this
    implementation a level-3 node's keys (4 leaves, 4C raw keys) are loaded
    once per work item and reused for up to `item_rows` (pair, head) columns
    (the pages' Q_tile, in query heads); the queries pass through LDS in
    batches of `batch_rows` columns and through MFMA 32x32x16 tiles of 32
    columns.  Sweeps both (PISA_S2_ITEM_ROWS, PISA_S2_BATCH_ROWS) for three
    group sizes, and times the single-stage (fused) selector beside the
    two-stage one."""
    import torch

    import hierarchical_block_selection_amd as pisa
    from hierarchical_block_selection_amd.inputs import prefill_inputs

    dev = torch.device("cuda:0")
    shapes = [("G1_d128_K16", 4, 4, 128, 16), ("G4_d128_K16", 16, 4, 128, 16),
              ("G16_d64_K8", 16, 1, 64, 8)]
    n = args.q_tile_n
    out = {"study": "stage-2 item and batch sizes", "N": n, "points": [], "fused_vs_two_stage": []}
    saved = {k: os.environ.get(k) for k in ("PISA_S2_ITEM_ROWS", "PISA_S2_BATCH_ROWS")}
    try:
        for name, hq, hkv, d, k in shapes:
            g = hq // hkv
            prob = pisa.Problem(1, hq, hkv, n, d, block=64, topk=k, dtype=torch.bfloat16)
            inp = prefill_inputs(1, hq, hkv, n, d, torch.bfloat16, seed=4100, device=dev)
            pyr = pisa.pisa_build_pyramid(prob, inp.k)
            for item in (64, 128, 256, 512, 1024, 2048, 4096):
                for rows in (32, 64, 128):
                    os.environ["PISA_S2_ITEM_ROWS"] = str(item)
                    os.environ["PISA_S2_BATCH_ROWS"] = str(rows)
                    ws = torch.empty(pisa.pisa_workspace_bytes(prob, "select"), dtype=torch.uint8,
                                     device=dev)
                    run = lambda: pisa.pisa_select(prob, inp.q, inp.k, pyr, workspace=ws,
                                                   want_score=False)
                    sel_ms = timed_call(run, 5, 2)
                    pisa.pisa_profile_enable(True)
                    run()
                    torch.cuda.synchronize()
                    rep = pisa.pisa_profile_report()
                    pisa.pisa_profile_enable(False)
                    s2 = rep.get("select_stage2", (float("nan"), 1))
                    out["points"].append({
                        "shape": name, "group": g, "item_rows": item, "batch_rows": rows,
                        "pairs_per_key_load": item // g, "select_ms": round(sel_ms, 4),
                        "stage2_ms": round(s2[0] / s2[1], 4)})
                    del ws
            for k_env in ("PISA_S2_ITEM_ROWS", "PISA_S2_BATCH_ROWS"):
                os.environ.pop(k_env, None)
            for nn in (4096, 16384):
                p2 = pisa.Problem(1, hq, hkv, nn, d, block=64, topk=k, dtype=torch.bfloat16)
                i2 = prefill_inputs(1, hq, hkv, nn, d, torch.bfloat16, seed=4101, device=dev)
                y2 = pisa.pisa_build_pyramid(p2, i2.k)
                f_ms = timed_call(lambda: pisa.pisa_select(p2, i2.q, i2.k, y2, strategy="fused",
                                                           want_score=False), 3, 1)
                t_ms = timed_call(lambda: pisa.pisa_select(p2, i2.q, i2.k, y2,
                                                           strategy="two_stage",
                                                           want_score=False), 5, 2)
                out["fused_vs_two_stage"].append({"shape": name, "N": nn, "fused_ms": round(f_ms, 4),
                                                  "two_stage_ms": round(t_ms, 4)})
            del inp, pyr
            torch.cuda.empty_cache()
    finally:
        for k_env, v in saved.items():
            if v is None:
                os.environ.pop(k_env, None)
            else:
                os.environ[k_env] = v
    return out


def cpu_baseline(args, inp, prob):
    """The CPU oracle on a bounded sample of the same workload: the full pyramid
    of KV head 0 plus selection + attention for random rows, on the host's
    cores.  The inputs go to a temporary directory and a child process that
    never touches the GPU runs a pool of single-threaded oracle workers (one
    per core of this process's CPU share, at most 16)."""
    import subprocess
    import tempfile

    import numpy as np

    with tempfile.TemporaryDirectory() as tmp:
        np.save(os.path.join(tmp, "keys.npy"), inp.k[0, 0].float().cpu().numpy())
        np.save(os.path.join(tmp, "vals.npy"), inp.v[0, 0].float().cpu().numpy())
        np.save(os.path.join(tmp, "q.npy"), inp.q[0, 0:1].float().cpu().numpy())
        cmd = [sys.executable, os.path.abspath(__file__), "--cpu-worker", tmp,
               "--cpu-seconds", str(args.cpu_seconds), "--cpu-block", str(prob.block),
               "--cpu-topk", str(prob.topk)]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=600,
                             env=dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1",
                                      MKL_NUM_THREADS="1"))
    if res.returncode != 0:
        raise RuntimeError(f"cpu baseline worker failed: {res.stderr[-2000:]}")
    r = json.loads(res.stdout.strip().splitlines()[-1])
    N, H = prob.seq_len, prob.heads_q
    # per (token, head): the pyramid prorated per token plus one row's selection
    # and attention; rows run concurrently on r["procs"] cores
    per_token_head = r["row_seconds"] / r["rows"] + r["pyramid_seconds"] / N
    value = r["procs"] / (H * per_token_head)
    return {"value": value, "unit": "tokens/s", "cores": r["procs"], "kind": "oracle",
            "sample": f"KV head 0 of the 128K workload: full pyramid ({r['pyramid_seconds']:.2f} s, "
                      f"prorated per token) + selection and attention of {r['rows']} random rows "
                      f"t >= K*C ({r['row_seconds']:.1f} core-s over {r['procs']} single-threaded "
                      f"worker processes), scaled to all {H} heads",
            "host_cpus": os.cpu_count(), "affinity_cpus": r["affinity"]}


_CPU = {}


def _cpu_rows(seed):
    """One oracle worker: random rows for the time budget (no GPU in here)."""
    import numpy as np

    import oracle

    keys, vals, qh, levels = _CPU["keys"], _CPU["vals"], _CPU["q"], _CPU["levels"]
    C, K, budget = _CPU["block"], _CPU["topk"], _CPU["seconds"]
    n = keys.shape[0]
    rng = np.random.default_rng(seed)
    done, spent = 0, 0.0
    while spent < budget and done < 65536:
        t = int(rng.integers(K * C, n))
        t1 = time.perf_counter()
        sel = oracle.select_pisa_row(qh[:, t], keys, levels, t, C, K, True, True)
        oracle.attend_row(qh[:, t], keys, vals, sel.leaves, t, C, True)
        spent += time.perf_counter() - t1
        done += 1
    return done, spent


def cpu_worker(args):
    """--cpu-worker DIR: load the sample, build the pyramid once, then fork the
    oracle workers and print one JSON line with the totals."""
    import multiprocessing

    import numpy as np

    import oracle

    d = args.cpu_worker
    keys = np.load(os.path.join(d, "keys.npy")).astype(np.float64)
    _CPU.update(keys=keys, vals=np.load(os.path.join(d, "vals.npy")).astype(np.float64),
                q=np.load(os.path.join(d, "q.npy")).astype(np.float64), block=args.cpu_block,
                topk=args.cpu_topk, seconds=args.cpu_seconds)
    t0 = time.perf_counter()
    _CPU["levels"] = oracle.build_pyramid(keys, args.cpu_block)
    t_pyr = time.perf_counter() - t0
    affinity = len(os.sched_getaffinity(0))
    procs = max(1, min(16, affinity))
    with multiprocessing.get_context("fork").Pool(procs) as pool:
        out = pool.map(_cpu_rows, range(procs))
    print(json.dumps({"rows": sum(o[0] for o in out), "row_seconds": sum(o[1] for o in out),
                      "pyramid_seconds": t_pyr, "procs": procs, "affinity": affinity}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--sweep-sizes", default=None,
                    help="comma-separated subset of the selection sweeps' N (default: all)")
    ap.add_argument("--no-sweep-g16", action="store_true",
                    help="skip the 16-heads-per-KV-head selection sweep")
    ap.add_argument("--no-sweep-k8", action="store_true",
                    help="skip the K = 8 selection sweep (4 heads, d = 128)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replayed timing of the step")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache steps (counter runs)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-worker", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-block", type=int, default=64, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-topk", type=int, default=16, help=argparse.SUPPRESS)
    ap.add_argument("--q-tile-study", action="store_true",
                    help="run only the stage-2 item/batch size study and print its JSON")
    ap.add_argument("--q-tile-n", type=int, default=65536)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="launch one elementwise copy of this many MiB before the steps "
                         "(HBM counter calibration)")
    args = ap.parse_args()
    if args.cpu_worker:
        cpu_worker(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the (batch, KV head) units would shard across GPUs without communication)",
              file=sys.stderr)
        sys.exit(2)
    if args.q_tile_study:
        print(json.dumps(q_tile_study(args)), flush=True)
        return
    res = run(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
