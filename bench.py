#!/usr/bin/env python3
"""Throughput of the CSA layer on one MI355X at 64K context, plus its roofline and the
CPU oracle timed on a bounded sample of the same work.

Prints ONE JSON line.  ``value`` is decode tokens/s at 64K context: batch 8, context 65,536,
the ratio-128 layer (512 compressed rows, all attended, 128-token window, 64 heads over a
512 latent, bf16); a step is one decode token for every sequence (compressor step + decode
attention with its window-ring update).  The K timed steps are captured once as a HIP graph
and replayed (the serving form of a decode loop); the same K steps issued eagerly, one
library call at a time from Python, are reported beside it under ``eager``.  The same line carries ``prefill``: the 2048-token
chunk 63,488 -> 65,536 of a ratio-4 layer (overlapping compressor on both lanes, indexer
top-512 over 15,872..16,384 rows, sparse attention), as tokens/s.

Both workloads start from a prefix cache built through the library itself (compressor over
the whole prefix in 8192-token blocks, then one attention call that fills the window ring).
Inputs are seeded synthetic tensors already resident in HBM when timing starts.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import re
import sys
import time
from collections import defaultdict

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_attention_dsv4_amd as K  # noqa: E402
import synth.csa as SC  # noqa: E402
from sparse_attention_dsv4_amd.layer import (CsaLayer, LayerSpec, SharedCsaLayer, compressor_lanes,  # noqa: E402
                                             output_path)
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
BLOCK = 8192


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ prefix caches
def build_prefix(layer: CsaLayer, spec: LayerSpec, seed: int, L: int):
    """Bring every sequence of ``layer`` to L tokens: compress the whole prefix, then one
    attention call over the last W tokens to fill the window ring."""
    B = layer.batch
    P = layer.params
    for t0 in range(0, L, BLOCK):
        S = min(BLOCK, L - t0)
        f = ["a", "g"] + (["ai", "gi"] if spec.has_indexer else [])
        tok = SC.batch_token_inputs(spec, seed, [t0] * B, S, device="cuda", fields=f)
        if spec.has_rows:
            K.dsv4_compress_prefill(spec.comp_cfg(), layer.state, tok["a"], tok["g"], [t0] * B,
                                    P["ape"], P["norm_w"], P["inv_freq"], layer.rows)
        if spec.has_indexer:
            K.dsv4_compress_prefill(spec.index_comp_cfg(), layer.state_i, tok["ai"], tok["gi"],
                                    [t0] * B, P["ape_i"], P["norm_w_i"], P["inv_freq"], layer.rows_i)
    t0 = L - spec.window
    tok = SC.batch_token_inputs(spec, seed, [t0] * B, spec.window, device="cuda",
                                fields=["q", "kv", "qi", "w"])
    n_rows = [L // spec.ratio] * B if spec.has_rows else None
    sel = None
    if spec.has_indexer:
        sel = torch.empty(B, spec.window, spec.topk, dtype=torch.int32, device="cuda")
        K.dsv4_index_topk(spec.index_cfg(), tok["qi"], tok["w"], layer.rows_i, n_rows, [t0] * B,
                          sel, layer.ws_index)
    out = torch.empty_like(tok["q"])
    K.dsv4_csa_attn_prefill(spec.attn_cfg(), tok["q"], tok["kv"], layer.ring,
                            layer.rows if spec.has_rows else None, sel, n_rows, [t0] * B,
                            P["sinks"], out, layer.ws_attn)
    layer.lengths = [L] * B
    torch.cuda.synchronize()


def kernel_time(name: str):
    n, ms = K.dsv4_trace_read("=" + name)
    return n, ms


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max(int(i.get("num_threads", 1)) for i in threadpool_info()) or 1
    except Exception:
        return os.cpu_count() or 1


_SLEEP_CYCLES_PER_MS = None


def _sleep_ms(ms: float):
    """Hold the stream for about ``ms`` on the GPU (torch's spin kernel), so that the host can
    enqueue the launches that follow before the GPU reaches them."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 1_000_000 / max(1e-3, e0.elapsed_time(e1))
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))


def traced(run, launches_hint: int):
    """Kernel durations of the library launches that ``run()`` enqueues, from the library's
    event trace.  A GPU-side wait goes first, long enough for the host to enqueue every
    launch, so the kernels then run back to back as they do in a graph replay (not each
    from an idle GPU).  Returns {kernel: (launches, total_ms)}."""
    torch.cuda.synchronize()
    K.dsv4_trace_reset()
    K.dsv4_trace_enable(True)
    _sleep_ms(0.05 * launches_hint + 2.0)
    run()
    torch.cuda.synchronize()
    K.dsv4_trace_enable(False)
    return {n: kernel_time(n) for n in K.dsv4_trace_kernels()}


def traced_min(run, launches_hint: int, reset, passes: int = 2):
    """``traced`` over the same work ``passes`` times (``reset()`` puts the work back before
    each pass: the same steps at the same positions write the same values), keeping the pass
    with the least summed kernel time: one pass of a few dozen short launches varies by
    ~15% from run to run."""
    best = None
    for _ in range(passes):
        reset()
        pk = traced(run, launches_hint)
        if best is None or sum(v[1] for v in pk.values()) < sum(v[1] for v in best.values()):
            best = pk
    return best


def scan_kernel(per_kernel):
    """The decode indexer's scoring kernel among the traced ones (the fused scorer, or the
    plain streamed one where the fused path does not apply)."""
    return max((n for n in per_kernel if n.startswith("index_score")), key=lambda n: per_kernel[n][1])


def kernel_table(per_kernel, per=1):
    return {n: {"launches": v[0], "avg_us": v[1] / max(1, v[0]) * 1e3,
                "us_per_step": v[1] / per * 1e3} for n, v in per_kernel.items() if v[0]}


def graph_of(fn):
    """Capture ``fn()`` (library launches on the current stream) as a HIP graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def replay_ms(graph, restore, reps: int = 1):
    """Wall time of one replay (the mean over ``reps``), the state restored before each."""
    t = 0.0
    for _ in range(reps):
        restore()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        t += time.perf_counter() - t0
    return t / reps * 1e3


# ------------------------------------------------------------------ algorithmic work
def decode_step_bytes(spec: LayerSpec, batch: int, step_positions) -> dict:
    """Algorithmic HBM bytes of one decode step of one layer for ``batch`` sequences, averaged
    over the steps at ``step_positions`` (every sequence at that position): inputs read once
    and outputs written once, no re-reads counted.  A row emission, which happens at one step
    in r, is counted as 1/r of its bytes at every step (its natural rate)."""
    e = 2 if spec.dtype == torch.bfloat16 else 4
    H, D, W = spec.heads, spec.dim, spec.window
    out = defaultdict(float)
    for p in step_positions:
        n = (p + 1) // spec.ratio if spec.has_rows else 0
        keys = W + ((min(n, spec.topk) if spec.has_indexer else n) if spec.has_rows else 0)
        # q, out, the attended keys (the window's newest from kv_new), the ring slot store
        out["attention"] += 2 * H * D * e + keys * D * e + D * e
        if spec.has_rows:
            lanes = [(spec.coff * spec.dim, spec.dim)]
            if spec.has_indexer:
                lanes.append((spec.coff * spec.index_dim, spec.index_dim))
            for width, dim in lanes:
                out["compressor"] += 2 * width * e * 2            # a, g read; frontier store
                # an emission reads value and gate of coff*r slots per channel, writes the row
                out["compressor"] += (2 * spec.coff * spec.ratio * dim * e + dim * e) / spec.ratio
        if spec.has_indexer:
            out["indexer"] += (n * spec.index_dim * e + spec.index_heads * (spec.index_dim * e + 4)
                               + spec.topk * 4)
    out = {k: v * batch / len(step_positions) for k, v in out.items()}
    out["total"] = sum(out.values())
    return out


def prefill_chunk_flops(spec: LayerSpec, start: int, S: int) -> dict:
    """Algorithmic flops of one prefill chunk (queries start .. start+S-1): the indexer's
    2*H_i*d_i per (query, visible row), attention's 4*H*D per (query, attended key)."""
    idx = att = 0.0
    for p in range(start, start + S):
        n = (p + 1) // spec.ratio
        idx += 2.0 * spec.index_heads * spec.index_dim * n
        att += 4.0 * spec.heads * spec.dim * (min(p + 1, spec.window) + min(spec.topk, n))
    return {"indexer": idx, "attention": att, "total": idx + att}


def emission_positions(p0: int, n: int, ratio: int) -> int:
    """Steps among positions p0 .. p0+n-1 at which a row completes."""
    return sum(1 for p in range(p0, p0 + n) if (p + 1) % ratio == 0) if ratio > 0 else 0


def emission_cost(layer: CsaLayer, tok: dict, reps: int = 32):
    """Extra cost of a decode step that completes a row over one that does not, for one
    layer: each step is captured ``reps`` times in one graph at a fixed position (a step at a
    fixed position rewrites the same ring slot, frontier slot and row, so repeats are
    identical work) and replayed; kernel durations come from a traced run of the same repeats.
    Returns (extra wall ms per emission, extra kernel ms per emission, kernel table)."""
    r = layer.spec.ratio
    p_now = layer.lengths[0]
    p_emit = p_now + (r - 1 - p_now % r)           # (p + 1) % r == 0
    p_plain = p_emit - 1 if r > 1 else None
    res = {}
    for name, p in (("emit", p_emit), ("plain", p_plain)):
        if p is None:
            continue

        def run(p=p):
            for _ in range(reps):
                layer.lengths = [p] * layer.batch
                layer.decode(tok)
        g = graph_of(run)
        g.replay()
        torch.cuda.synchronize()
        ms = replay_ms(g, lambda: None, reps=5) / reps
        kern = traced(run, 4 * reps)
        res[name] = (ms, sum(v[1] for v in kern.values()) / reps, kern)
        del g
    layer.lengths = [p_now] * layer.batch
    if "plain" not in res:
        return 0.0, 0.0, {}
    return (res["emit"][0] - res["plain"][0], res["emit"][1] - res["plain"][1],
            kernel_table(res["emit"][2], reps))


def step_roofline(bytes_per_step: float, kernel_ms_per_step: float, dominant: dict):
    ach = bytes_per_step / (kernel_ms_per_step * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS, "scope": "whole step: algorithmic bytes per step over "
                                                 "the summed kernel time of one step",
            "bytes_per_step": bytes_per_step, "kernel_us_per_step": kernel_ms_per_step * 1e3,
            "traffic": dominant.pop("step_traffic", None), "dominant_kernel": dominant}


# ------------------------------------------------------------------ decode @ 64K
def bench_decode(args, seed=0):
    spec = LayerSpec(ratio=128, indexer=False, topk=0)
    B, L = args.decode_batch, args.context
    steps, warm = args.steps, args.warmup
    r = spec.ratio
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, L + warm + 3 * steps + 2 * r + 8, params, device="cuda",
                     max_chunk=spec.window)
    t_setup = time.time()
    build_prefix(layer, spec, seed, L)
    log(f"[decode] prefix of {L} tokens x {B} built in {time.time() - t_setup:.1f}s")
    # inputs of every step, resident before timing
    toks = []
    for i in range(warm + steps):
        t = SC.batch_token_inputs(spec, seed, [L + i] * B, 1, device="cuda",
                                  fields=["q", "kv", "a", "g"])
        toks.append({k: v[:, 0].contiguous() for k, v in t.items()})
    for i in range(warm):
        layer.decode(toks[i])
    torch.cuda.synchronize()
    # eager: one library call at a time from Python
    p_eager = layer.lengths[0]
    t0 = time.perf_counter()
    for i in range(warm, warm + steps):
        layer.decode(toks[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # kernel durations of the same K steps, run back to back
    p_trace = layer.lengths[0]

    def reset_trace():
        layer.lengths = [p_trace] * B

    per_kernel = traced_min(lambda: [layer.decode(toks[i]) for i in range(warm, warm + steps)],
                            3 * steps, reset_trace)
    # the K steps captured once as a HIP graph and replayed: every launch and argument is
    # recorded, so a replay costs no host work per launch.  The state is restored before each
    # replay (outside the timed region), so every replay recomputes the captured positions.
    snap = {n: getattr(layer, n).clone() for n in ("ring", "state", "rows")}
    p_graph = layer.lengths[0]
    graph = graph_of(lambda: [layer.decode(toks[i]) for i in range(warm, warm + steps)])

    def restore():
        for n, v in snap.items():
            getattr(layer, n).copy_(v)
        torch.cuda.synchronize()

    restore()
    graph.replay()                       # warm replay
    torch.cuda.synchronize()
    restore()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    g_wall = time.perf_counter() - t0
    g_ev = g0.elapsed_time(g1) * 1e-3
    del graph
    # a row completes once every r steps; the K-step window holds n_e such steps, not K/r.
    # The emission step's extra cost is measured on its own and the window corrected to the
    # natural rate.
    layer.lengths = [p_graph + steps] * B
    emit_wall_ms, emit_kernel_ms, emit_kernels = emission_cost(layer, toks[warm])
    n_e_graph = emission_positions(p_graph, steps, r)
    n_e_trace = emission_positions(p_trace, steps, r)
    corr_graph = (steps / r - n_e_graph) * emit_wall_ms * 1e-3
    corr_trace = (steps / r - n_e_trace) * emit_kernel_ms
    g_amort = g_wall + corr_graph
    kernel_ms_step = (sum(v[1] for v in per_kernel.values()) + corr_trace) / steps
    # algorithmic bytes per step at the traced positions (the emission at 1/r)
    by = decode_step_bytes(spec, B, range(p_trace, p_trace + steps))
    attn_name = max((n for n in per_kernel if n.startswith("attn")), key=lambda n: per_kernel[n][1])
    n_l, ms_l = per_kernel[attn_name]
    keys = spec.window + (p_trace + steps // 2 + 1) // r
    bytes_launch = B * (2 * spec.heads * spec.dim * 2 + keys * spec.dim * 2 + 2 * spec.dim * 2)
    achieved = bytes_launch / (ms_l / n_l * 1e-3) / 1e9
    dominant = {"kernel": attn_name, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": traffic_from_profile(TRAFFIC_DECODE, attn_name),
                "bytes_per_launch": bytes_launch, "avg_us": ms_l / n_l * 1e3}
    dominant["step_traffic"] = step_traffic_from_profile(TRAFFIC_DECODE_STEP, per_kernel, steps)
    res = {
        "tok_s": B * steps / g_amort, "ms_per_step": g_amort / steps * 1e3,
        "mode": "hip-graph replay of the K captured steps; the row emission (one step in "
                f"{r}) amortized at its natural rate",
        "raw": {"ms_per_step": g_wall / steps * 1e3, "emission_steps_in_window": n_e_graph,
                "graph_events_ms_per_step": g_ev / steps * 1e3},
        "emission": {"extra_us_per_emission": emit_wall_ms * 1e3,
                     "extra_kernel_us_per_emission": emit_kernel_ms * 1e3,
                     "kernels_of_an_emission_step": emit_kernels},
        "eager": {"tok_s": B * steps / wall, "ms_per_step": wall / steps * 1e3,
                  "mode": "one library call per lane per step from Python"},
        "kernels": kernel_table(per_kernel, steps),
        "bytes_per_step": by,
        "roofline": step_roofline(by["total"], kernel_ms_step, dominant),
    }
    return res, (spec, seed)


def bench_decode_batch_scan(args, batches=(32, 128)):
    """The headline decode workload at larger batches (same layer, context and step count),
    where the launches' fixed latency is spread over more sequences: graph time per step and
    the whole step's fraction of HBM on its algorithmic bytes."""
    out = []
    for B in batches:
        a = argparse.Namespace(**vars(args))
        a.decode_batch = B
        res, _ = bench_decode(a, seed=5)
        out.append({"batch": B, "tok_s": res["tok_s"], "ms_per_step": res["ms_per_step"],
                    "whole_step_hbm_frac": res["roofline"]["frac"],
                    "bytes_per_step": res["bytes_per_step"]["total"],
                    "kernel_us_per_step": res["roofline"]["kernel_us_per_step"],
                    "kernels": res["kernels"]})
        torch.cuda.empty_cache()
    return out


def bench_stack(args, seed=23, ratios=(0, 4, 128), topk=512, traffic_profile=None,
                step_traffic_profile=None):
    """Decode of a layer stack at 262,144 tokens, batch 4.  The default is V4-Flash's head
    [0, 4, 128]: a window-only layer, a ratio-4 layer (65,536 rows, indexer top-512) and a
    ratio-128 layer (2048 rows, top-512); ratios (128, 128, 4, 128) with topk 1024 is
    V4-Pro's head (no window-only layer, top-1024).  A step is one decode token of every
    sequence through all layers; the K steps are replayed as a HIP graph like the headline
    decode, with each layer's row emission amortized at its natural rate.  The roofline is
    the whole step's (algorithmic bytes of every layer over the summed kernel time of a step);
    the dominant kernel beside it is the ratio-4 layer's indexer scan (every visible indexer
    row is read once per step), whose HBM traffic comes from ``traffic_profile``."""
    B, L = 4, 262144
    steps, warm = min(args.steps, 64), args.warmup
    specs = [LayerSpec(ratio=0, indexer=False, topk=0) if r == 0 else LayerSpec(ratio=r, topk=topk)
             for r in ratios]
    i4 = list(ratios).index(4)
    layers, toks = [], []
    t_setup = time.time()
    for i, spec in enumerate(specs):
        lseed = seed + spec.ratio + 1000 * list(ratios[:i]).count(spec.ratio)
        params = SC.layer_params(spec, lseed, device="cuda")
        layer = CsaLayer(spec, B, L + warm + 3 * steps + 2 * max(ratios) + 8, params, device="cuda",
                         max_chunk=spec.window)
        build_prefix(layer, spec, lseed, L)
        layers.append(layer)
        tl = []
        for j in range(warm + steps):
            t = SC.batch_token_inputs(spec, lseed, [L + j] * B, 1, device="cuda")
            tl.append({k: v[:, 0].contiguous() for k, v in t.items()})
        toks.append(tl)
    log(f"[stack] {list(ratios)} (top-{topk}) at {L} tokens x {B} built in {time.time() - t_setup:.1f}s")

    def step(j, only=None):
        for i, layer in enumerate(layers):
            if only is not None:
                K.dsv4_trace_enable(i == only)
            layer.decode(toks[i][j])

    for j in range(warm):
        step(j)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(warm, warm + steps):
        step(j)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # kernel durations of the whole step, then of the ratio-4 layer alone, back to back
    p_trace = layers[0].lengths[0]

    def reset_trace():
        for l in layers:
            l.lengths = [p_trace] * B

    per_kernel = traced_min(lambda: [step(j) for j in range(warm, warm + steps)], 6 * len(layers) * steps,
                            reset_trace)
    reset_trace()
    per_kernel4 = traced(lambda: [step(j, only=i4) for j in range(warm, warm + steps)],
                         6 * len(layers) * steps)
    # graph replay of the K steps (state restored outside the timed region)
    names = ("ring", "state", "rows", "state_i", "rows_i")
    snap = [{n: getattr(l, n).clone() for n in names if hasattr(l, n)} for l in layers]
    p_graph = layers[0].lengths[0]
    graph = graph_of(lambda: [step(j) for j in range(warm, warm + steps)])

    def restore():
        for l, sn in zip(layers, snap):
            for n, v in sn.items():
                getattr(l, n).copy_(v)
        torch.cuda.synchronize()

    restore()
    graph.replay()
    torch.cuda.synchronize()
    restore()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    g_wall = time.perf_counter() - t0
    del graph
    # each layer's row emissions at their natural rate (the window holds n_e of them, not K/r)
    corr_wall = corr_kernel = 0.0
    emissions = {}
    for i, (spec, layer) in enumerate(zip(specs, layers)):
        if not spec.has_rows:
            continue
        n_g = emission_positions(p_graph, steps, spec.ratio)
        n_t = emission_positions(p_trace, steps, spec.ratio)
        if n_g == steps / spec.ratio and n_t == steps / spec.ratio:
            continue
        layer.lengths = [p_graph + steps] * B
        ew, ek, _ = emission_cost(layer, toks[i][warm])
        corr_wall += (steps / spec.ratio - n_g) * ew * 1e-3
        corr_kernel += (steps / spec.ratio - n_t) * ek
        emissions[f"layer{i}_ratio{spec.ratio}"] = {"extra_us_per_emission": ew * 1e3,
                                                    "extra_kernel_us_per_emission": ek * 1e3,
                                                    "emission_steps_in_window": n_g}
    g_amort = g_wall + corr_wall
    kernel_ms_step = (sum(v[1] for v in per_kernel.values()) + corr_kernel) / steps
    by = defaultdict(float)
    for i, spec in enumerate(specs):
        for k, v in decode_step_bytes(spec, B, range(p_trace, p_trace + steps)).items():
            by[f"layer{i}_ratio{spec.ratio}.{k}" if k != "total" else "total"] += v
    spec4 = specs[i4]
    nv = (p_trace + steps // 2 + 1) // spec4.ratio
    scan = scan_kernel(per_kernel4)
    n_l, ms_l = per_kernel4[scan]
    # algorithmic bytes of one scan: every visible indexer row, the queries and head weights
    bytes_launch = B * (nv * spec4.index_dim * 2 + spec4.index_heads * (spec4.index_dim * 2 + 4))
    achieved = bytes_launch / (ms_l / n_l * 1e-3) / 1e9
    dominant = {"kernel": f"{scan} (ratio-4 layer)", "bound": "hbm", "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": (traffic_from_profile(traffic_profile, scan) if traffic_profile else None),
                "bytes_per_launch": bytes_launch, "avg_us": ms_l / n_l * 1e3}
    dominant["step_traffic"] = (step_traffic_from_profile(step_traffic_profile, per_kernel, steps)
                                if step_traffic_profile else None)
    return {
        "workload": f"decode, {list(ratios)} stack ("
                    + ", ".join("window-only" if r == 0 else
                                f"ratio-{r} with top-{topk} over ~{(L + warm) // r} rows" for r in ratios)
                    + f"), batch {B}, context {L}",
        "tok_s": B * steps / g_amort, "ms_per_step": g_amort / steps * 1e3,
        "mode": f"hip-graph replay of the K captured steps ({len(ratios)} layers per step), row "
                "emissions amortized at their natural rate",
        "raw_ms_per_step": g_wall / steps * 1e3,
        "emission": emissions,
        "eager": {"tok_s": B * steps / wall, "ms_per_step": wall / steps * 1e3},
        "kernels": kernel_table(per_kernel, steps),
        "kernels_ratio4_layer": kernel_table(per_kernel4, steps),
        "bytes_per_step": dict(by),
        "roofline": step_roofline(by["total"], kernel_ms_step, dominant),
    }


def bench_shared(args, seed=71, n_own=2, n_sel=1):
    """Decode of a cross-layer-sharing group at 262,144 tokens, batch 4 (V4.1's layout: one
    ratio-4 layer owns the compressors and index keys; ``n_own`` index-source layers score
    their own queries against its keys and ``n_sel`` layers attend its selection).  A step is
    one token through the owner and every consumer, replayed as a HIP graph.  The roofline is
    the index scan (owner and index-source layers: the same rows, read once per launch)."""
    B, L = 4, 262144
    steps, warm = min(args.steps, 64), args.warmup
    spec = LayerSpec(ratio=4)
    t_setup = time.time()
    owner = CsaLayer(spec, B, L + warm + 3 * steps + 8, SC.layer_params(spec, seed, device="cuda"),
                     device="cuda", max_chunk=spec.window)
    build_prefix(owner, spec, seed, L)
    cons = []
    for i in range(n_own + n_sel):
        c = SharedCsaLayer(spec, owner, SC.layer_params(spec, seed + 1 + i, device="cuda"),
                           index="own" if i < n_own else "owner", max_chunk=spec.window)
        c.ring.copy_(owner.ring)          # the owner's last W token latents
        cons.append(c)
    toks = []
    for j in range(warm + steps):
        to = {k: v[:, 0].contiguous() for k, v in
              SC.batch_token_inputs(spec, seed, [L + j] * B, 1, device="cuda").items()}
        tc = []
        for i in range(len(cons)):
            t = {k: v[:, 0].contiguous() for k, v in
                 SC.batch_token_inputs(spec, seed + 1 + i, [L + j] * B, 1, device="cuda",
                                       fields=["q", "qi", "w"]).items()}
            t["kv"] = to["kv"]
            tc.append(t)
        toks.append((to, tc))
    sel = torch.empty(B, 1, spec.topk, dtype=torch.int32, device="cuda")
    log(f"[shared] owner + {n_own} index-source + {n_sel} selection-sharing layers at {L} tokens x {B} "
        f"built in {time.time() - t_setup:.1f}s")

    def step(j):
        to, tc = toks[j]
        owner.decode(to, sel_out=sel)
        for c, t in zip(cons, tc):
            c.decode(t) if c.index == "own" else c.decode(t, sel=sel[:, 0])

    for j in range(warm):
        step(j)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(warm, warm + steps):
        step(j)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # kernel durations in a second pass, back to back (positions keep advancing, as in
    # bench_stack: the layers hold room for the three passes)
    per_kernel = traced(lambda: [step(j) for j in range(warm, warm + steps)], 12 * steps)
    names = ("ring", "state", "rows", "state_i", "rows_i")
    snap = [{n: getattr(l, n).clone() for n in names if hasattr(l, n)} for l in [owner] + cons]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(warm, warm + steps):
            step(j)

    def restore():
        for l, sn in zip([owner] + cons, snap):
            for n, v in sn.items():
                getattr(l, n).copy_(v)
        torch.cuda.synchronize()

    restore()
    graph.replay()
    torch.cuda.synchronize()
    restore()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    g_wall = time.perf_counter() - t0
    nv = (L + warm) // spec.ratio
    scan = scan_kernel(per_kernel)
    n_l, ms_l = per_kernel[scan]
    bytes_launch = B * (nv * spec.index_dim * 2 + spec.index_heads * (spec.index_dim * 2 + 4))
    achieved = bytes_launch / (ms_l / n_l * 1e-3) / 1e9
    owner_bytes = sum(getattr(owner, n).numel() * getattr(owner, n).element_size() for n in names)
    cons_bytes = cons[0].ring.numel() * cons[0].ring.element_size()
    n_layers = 1 + len(cons)
    return {
        "workload": f"decode, cross-layer KV sharing at context {L}, batch {B}: one ratio-4 owner "
                    f"(compressors, ~{nv} rows, top-512), {n_own} layers scoring their own queries "
                    f"against its index keys, {n_sel} attending its selection",
        "tok_s": B * steps / g_wall, "ms_per_step": g_wall / steps * 1e3,
        "us_per_layer": g_wall / steps / n_layers * 1e6,
        "mode": f"hip-graph replay of the K captured steps ({n_layers} layers per step)",
        "eager": {"tok_s": B * steps / wall, "ms_per_step": wall / steps * 1e3},
        "cache_bytes": {"owner": owner_bytes, "per_sharing_layer": cons_bytes},
        "kernels": kernel_table(per_kernel, steps),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": scan,
                     "bytes_per_launch": bytes_launch},
    }


def _host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def oracle_prefix_rows(spec: LayerSpec, seed: int, b: int, n_tok: int, index_lane: bool = False,
                       device="cpu", block: int = 8192) -> np.ndarray:
    """Compressed rows of sequence ``b`` after ``n_tok`` tokens, by the oracle, block by block
    from the seeded lanes (drawn on ``device`` by the input generator, read on the host)."""
    import oracle
    r = spec.ratio
    fa, fg = ("ai", "gi") if index_lane else ("a", "g")
    P = {k: _host(v) for k, v in SC.layer_params(spec, seed).items()}
    ape, gamma = (P["ape_i"], P["norm_w_i"]) if index_lane else (P["ape"], P["norm_w"])
    dim = spec.index_dim if index_lane else spec.dim
    store = "bf16" if spec.dtype == torch.bfloat16 else "f32"
    end = n_tok - n_tok % r
    block = max(r, block - block % r)
    out = [np.zeros((0, dim))]
    for t0 in range(0, end, block):
        t1 = min(end, t0 + block)
        s0 = max(0, t0 - r) if spec.is_overlap else t0          # the previous window, overlapping
        lanes = SC.token_inputs(spec, seed, b, s0, t1, device=device, fields=[fa, fg])
        out.append(oracle.compressor_rows(_host(lanes[fa]), _host(lanes[fg]), ape, gamma,
                                          P["inv_freq"], ratio=r, overlap=spec.is_overlap,
                                          eps=spec.eps, store=store, rows=range(t0 // r, t1 // r),
                                          token0=s0))
    return np.concatenate(out)


def cpu_baseline_decode(spec: LayerSpec, seed: int, L: int, n_seq: int, steps: int, device="cpu"):
    """The oracle doing the decode work of ``steps`` steps of ``n_seq`` sequences from
    position L on: at each step the row emission when one completes ((p + 1) % r == 0: the
    oracle's compressor over that row's window), then attention over the window and every
    visible row.  The cache it starts from (rows of the first L tokens) is built by the
    oracle from the same seeded inputs before the clock starts; nothing comes from the GPU."""
    import oracle
    r, W = spec.ratio, spec.window
    store = "bf16" if spec.dtype == torch.bfloat16 else "f32"
    P = {k: _host(v) for k, v in SC.layer_params(spec, seed).items()}
    t_lo = max(0, L - W + 1 - spec.coff * r)
    seqs = []
    for b in range(n_seq):
        rows = oracle_prefix_rows(spec, seed, b, L, device=device)
        tok = {k: _host(v) for k, v in SC.token_inputs(spec, seed, b, t_lo, L + steps, device=device,
                                                       fields=["q", "kv", "a", "g"]).items()}
        seqs.append([rows, tok])
    emitted = 0
    t0 = time.perf_counter()
    for i in range(steps):
        p = L + i
        for rows_tok in seqs:
            rows, tok = rows_tok
            if (p + 1) % r == 0:
                j = (p + 1) // r - 1
                s0 = max(0, (j - 1) * r) if spec.is_overlap else j * r
                row = oracle.compressor_rows(tok["a"][s0 - t_lo:p + 1 - t_lo],
                                             tok["g"][s0 - t_lo:p + 1 - t_lo], P["ape"],
                                             P["norm_w"], P["inv_freq"], ratio=r,
                                             overlap=spec.is_overlap, eps=spec.eps, store=store,
                                             rows=[j], token0=s0)
                rows = rows_tok[0] = np.concatenate([rows, row])
                emitted += 1
            lo = max(0, p - W + 1)
            oracle.csa_attention(tok["q"][p - t_lo][None], tok["kv"][lo - t_lo:p + 1 - t_lo],
                                 rows, None, [p], window=W, ratio=r, sinks=P["sinks"],
                                 scale=spec.scale, store=store, kv_offset=lo)
    dt = time.perf_counter() - t0
    done = steps * n_seq
    return {"value": done / dt, "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{steps} decode steps x {n_seq} sequences from position {L} "
                      f"({done} tokens, {emitted} row emissions at the natural rate), window + "
                      f"every visible row per query; oracle in numpy, cache built by the oracle"}


# ------------------------------------------------------------------ prefill @ 64K
def bench_prefill(args, seed=1):
    spec = LayerSpec(ratio=4)
    S, L = args.chunk, args.context
    start = L - S
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, 1, L, params, device="cuda", max_chunk=max(S, spec.window))
    t_setup = time.time()
    build_prefix(layer, spec, seed, start)
    log(f"[prefill] prefix of {start} tokens built in {time.time() - t_setup:.1f}s")
    tok = SC.batch_token_inputs(spec, seed, [start], S, device="cuda")
    snap = {"state": layer.state.clone(), "state_i": layer.state_i.clone(), "ring": layer.ring.clone()}
    sel = torch.empty(1, S, spec.topk, dtype=torch.int32, device="cuda")

    def step():
        layer.state.copy_(snap["state"])
        layer.state_i.copy_(snap["state_i"])
        layer.ring.copy_(snap["ring"])
        layer.lengths = [start]
        return layer.prefill(tok, sel_out=sel)

    reps = max(1, args.prefill_reps)
    for _ in range(max(1, args.warmup // 4)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    per_kernel = traced(lambda: [step() for _ in range(reps)], 10 * reps)
    # algorithmic flops of the chunk: indexer q.k over every visible row, attention QK^T and PV
    fl = prefill_chunk_flops(spec, start, S)
    dom = max(per_kernel, key=lambda n: per_kernel[n][1])
    n_d, ms_d = per_kernel[dom]
    dom_flops = fl["indexer"] if "index" in dom else fl["attention"] if "attn" in dom else 0.0
    achieved = dom_flops / (ms_d / n_d * 1e-3) / 1e12
    total_ms = sum(v[1] for v in per_kernel.values()) / reps
    whole = fl["total"] / (total_ms * 1e-3) / 1e12
    res = {
        "tok_s": S / wall, "ms_per_chunk": wall * 1e3,
        "workload": f"ratio-4 layer, chunk {start}->{L} (S={S}), indexer top-{spec.topk}, "
                    f"64 heads x 512 latent, bf16",
        "flops_per_chunk": fl,
        "kernels": kernel_table(per_kernel, reps),
        "roofline": {"bound": "mfma", "achieved": whole, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": whole / BF16_MFMA_PEAK_TFLOPS,
                     "scope": "whole chunk: algorithmic flops over the summed kernel time of the "
                              "chunk (compressor lanes, indexer, top-k, attention, ring update)",
                     "flops_per_chunk": fl["total"], "kernel_us_per_chunk": total_ms * 1e3,
                     "traffic": None,
                     "dominant_kernel": {"kernel": dom, "bound": "mfma", "achieved": achieved,
                                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                         "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                                         "traffic": traffic_from_profile(TRAFFIC_PREFILL, dom),
                                         "flops_per_launch": dom_flops,
                                         "avg_us": ms_d / n_d * 1e3}},
    }
    return res, (spec, seed, start, S)


def cpu_baseline_prefill(spec: LayerSpec, seed: int, start: int, S: int, n_queries: int,
                         device="cpu"):
    """The oracle on the chunk start .. start+S-1 of one sequence: the chunk's compressed rows
    (both lanes; timed, charged to the sample at n_queries / S of their cost), then for
    ``n_queries`` queries spread over the chunk the indexer scores over every visible row,
    the top-k and attention over window + selected rows.  The rows of the first ``start``
    tokens are built by the oracle before the clock starts."""
    import oracle
    r, W = spec.ratio, spec.window
    store = "bf16" if spec.dtype == torch.bfloat16 else "f32"
    P = {k: _host(v) for k, v in SC.layer_params(spec, seed).items()}
    rows = oracle_prefix_rows(spec, seed, 0, start, device=device)
    rows_i = oracle_prefix_rows(spec, seed, 0, start, index_lane=True, device=device)
    s0 = max(0, start - r) if spec.is_overlap else start
    lanes = {k: _host(v) for k, v in SC.token_inputs(spec, seed, 0, s0, start + S, device=device,
                                                     fields=["a", "g", "ai", "gi"]).items()}
    idx = np.linspace(0, S - 1, n_queries).astype(int)
    qs = []
    for i in idx:
        p = start + int(i)
        lo = max(0, p - W + 1)
        t = {k: _host(v) for k, v in SC.token_inputs(spec, seed, 0, p, p + 1, device=device,
                                                     fields=["q", "qi", "w"]).items()}
        t["kv"] = _host(SC.token_inputs(spec, seed, 0, lo, p + 1, device=device, fields=["kv"])["kv"])
        qs.append((p, lo, t))
    kw = dict(ratio=r, overlap=spec.is_overlap, eps=spec.eps, store=store,
              rows=range(start // r, (start + S) // r), token0=s0)
    t0 = time.perf_counter()
    rows = np.concatenate([rows, oracle.compressor_rows(lanes["a"], lanes["g"], P["ape"], P["norm_w"],
                                                        P["inv_freq"], **kw)])
    rows_i = np.concatenate([rows_i, oracle.compressor_rows(lanes["ai"], lanes["gi"], P["ape_i"],
                                                            P["norm_w_i"], P["inv_freq"], **kw)])
    t_comp = time.perf_counter() - t0
    t0 = time.perf_counter()
    for p, lo, t in qs:
        nv = oracle.visible_rows(p, r)
        sc = oracle.index_scores(t["qi"], t["w"], rows_i[:nv])
        sel = oracle.select_topk(sc, [p], ratio=r, k=spec.topk)
        oracle.csa_attention(t["q"], t["kv"], rows, sel, [p], window=W, ratio=r, sinks=P["sinks"],
                             scale=spec.scale, store=store, kv_offset=lo)
    t_q = time.perf_counter() - t0
    dt = t_q + t_comp * n_queries / S
    return {"value": n_queries / dt, "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{n_queries} of the {S} queries of the chunk {start}->{start + S} (indexer over "
                      f"~{(start + S) // r} rows, top-{spec.topk}, attention) plus {n_queries}/{S} of the "
                      f"chunk's compressor work; oracle in numpy, prefix rows built by the oracle"}


def bench_output_path(args, seed=41):
    """The attention output's way out of a layer at the layer's shapes: inverse RoPE of the
    rotary dims of 64 heads x 512 (in place), then the grouped block-diagonal projection
    (wo_a: 8 groups x 1024 outputs x 4096 inputs).  Decode: one token of each of 8
    sequences (the projection streams wo_a's 64 MiB once: HBM-bound); prefill: one 2048-token
    chunk (MFMA-bound: 2 * 2048 * 8 * 1024 * 4096 flop).  Kernel times from the trace over
    ``reps`` calls; the weights are synthetic (N(0, 1/4096))."""
    spec = LayerSpec(ratio=4)
    G, R = 8, 1024
    Kd = spec.heads // G * spec.dim
    inv = SC.inv_freq(spec.rope_dim).cuda()
    wo_a = synth.normal((G, R, Kd), seed=seed, stream="wo_a", scale=Kd ** -0.5,
                        dtype=torch.bfloat16, device="cuda")
    out = {}
    for name, B, S, pos in (("decode_b8", 8, 1, args.context), ("prefill_2048", 1, args.chunk,
                                                                 args.context - args.chunk)):
        o = synth.normal((B, S, spec.heads, spec.dim), seed=seed, stream="attn_out",
                         dtype=torch.bfloat16, device="cuda")
        y = torch.empty(B, S, G, R, dtype=torch.bfloat16, device="cuda")
        reps = 20
        for _ in range(3):
            output_path(spec, o, [pos] * B, inv, wo_a, y)
        torch.cuda.synchronize()
        K.dsv4_trace_reset()
        K.dsv4_trace_enable(True)
        for _ in range(reps):
            output_path(spec, o, [pos] * B, inv, wo_a, y)
        torch.cuda.synchronize()
        K.dsv4_trace_enable(False)
        times = {n: kernel_time(n) for n in K.dsv4_trace_kernels()}
        T = B * S
        gname = next(n for n in times if n.startswith("gproj") and times[n][0])
        n_g, ms_g = times[gname]
        us_g = ms_g / n_g * 1e3
        n_r, ms_r = times["rope"]
        entry = {"tokens": T, "kernels": {n: {"launches": v[0], "avg_us": v[1] / max(1, v[0]) * 1e3}
                                         for n, v in times.items() if v[0]}}
        if S == 1:
            byts = G * R * Kd * 2 + T * G * Kd * 2 + T * G * R * 2
            ach = byts / (us_g * 1e-6) / 1e9
            entry["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": ach / HBM_PEAK_GBS, "traffic": None, "kernel": gname,
                                 "bytes_per_launch": byts}
        else:
            fl = 2.0 * T * G * R * Kd
            ach = fl / (us_g * 1e-6) / 1e12
            entry["roofline"] = {"bound": "mfma", "achieved": ach, "peak": BF16_MFMA_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": ach / BF16_MFMA_PEAK_TFLOPS,
                                 "traffic": None, "kernel": gname, "flops_per_launch": fl}
        entry["us_per_call"] = us_g + ms_r / n_r * 1e3
        out[name] = entry
        del o, y
    # the ratio-4 compressor's lanes of a 2048-token chunk from hidden states (wkv, wgate
    # [1024, 4096]): both one-group projections in one launch (dsv4_lane_proj)
    T, hid, W = args.chunk, 4096, spec.coff * spec.dim
    x = synth.normal((T, hid), seed=seed, stream="hidden", dtype=torch.bfloat16, device="cuda")
    wkv = synth.normal((W, hid), seed=seed, stream="wkv", scale=hid ** -0.5, dtype=torch.bfloat16,
                       device="cuda")
    wg = synth.normal((W, hid), seed=seed, stream="wgate", scale=hid ** -0.5, dtype=torch.bfloat16,
                      device="cuda")
    for _ in range(3):
        compressor_lanes(x, wkv, wg)
    torch.cuda.synchronize()
    K.dsv4_trace_reset()
    K.dsv4_trace_enable(True)
    calls = 10
    for _ in range(calls):
        compressor_lanes(x, wkv, wg)
    torch.cuda.synchronize()
    K.dsv4_trace_enable(False)
    gname = max((n for n in K.dsv4_trace_kernels() if n.startswith("gproj")),
                key=lambda n: kernel_time(n)[0])
    n_g, ms_g = kernel_time(gname)
    us = ms_g / calls * 1e3                        # kernel time per call (both lanes)
    fl = 2.0 * 2.0 * T * W * hid                   # both products
    ach = fl / (us * 1e-6) / 1e12
    out["lanes_prefill_2048"] = {
        "tokens": T, "us_per_call": us, "launches_per_call": n_g / calls,
        "roofline": {"bound": "mfma", "achieved": ach, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / BF16_MFMA_PEAK_TFLOPS, "traffic": None, "kernel": gname,
                     "flops_per_call": fl}}
    return out


# ------------------------------------------------------------------ profiles
# The summaries under profiles/ are written from rocprofv3 output by the modes below (no GPU
# needed), so each one names commands that run committed files only.  A traffic summary
# records a digest of its kernel's sources; the JSON line reports its traffic only while the
# sources still match (a changed kernel reports null until it is measured again).
CSRC = os.path.join(ROOT, "sparse_attention_dsv4_amd", "csrc")
KERNEL_SOURCES = {"attn": "attention.hip", "ring": "attention.hip", "index": "indexer.hip",
                  "topk": "indexer.hip", "compress": "compress.hip", "frontier": "compress.hip",
                  "gproj": "proj.hip", "rope": "proj.hip"}
COPY_CALIB_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_DECODE = os.path.join(PROFILES, "traffic_attn_decode_ctx65536_b8_ratio128.txt")
TRAFFIC_PREFILL = os.path.join(PROFILES, "traffic_index_score_rs_ctx65536_chunk2048_ratio4.txt")
TRAFFIC_STACK = os.path.join(PROFILES, "traffic_index_score_fused_decode_ctx262144_b4_stack.txt")
TRAFFIC_DECODE_STEP = os.path.join(PROFILES, "traffic_step_decode_ctx65536_b8_ratio128.txt")
TRAFFIC_STACK_STEP = os.path.join(PROFILES, "traffic_step_stack_decode_ctx262144_b4.txt")


def kernel_source_digest(kernel: str) -> str:
    src = next(v for k, v in KERNEL_SOURCES.items() if kernel.startswith(k))
    h = hashlib.sha256()
    for f in (src, "common.hpp", "mfma.hpp", "kernels.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_calibration():
    """A device-to-device copy of COPY_CALIB_BYTES, three times: the reference dispatch that
    scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    a = torch.randn(COPY_CALIB_BYTES // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {COPY_CALIB_BYTES} bytes x 3", flush=True)


def _short_kernel(name: str, with_args: bool = False):
    """Library kernel name without the namespace and the _kernel suffix (with its template
    arguments when asked: one kernel template serves several selection stages)."""
    if "copyBuffer" in name:
        return "copy"
    m = re.search(r"(\w+)_kernel(<[^>(]*>)?", name)
    if not m or "dsv4" not in name:
        return None
    return m.group(1) + (m.group(2).replace(" ", "") if with_args and m.group(2) else "")


def _csv_rows(directory: str, pattern: str):
    for f in sorted(glob.glob(os.path.join(directory, "**", pattern), recursive=True)):
        with open(f) as fh:
            yield from csv.DictReader(fh)


def _grid(r: dict) -> str:
    g = [r[k] for k in ("Grid_Size", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z") if k in r]
    return "x".join(g) if g else "?"


def _pmc(directory: str, counter: str):
    """{(kernel, grid): {dispatch: value}} of one rocprofv3 --pmc pass."""
    out = defaultdict(lambda: defaultdict(float))
    for r in _csv_rows(directory, "*counter_collection.csv"):
        k = _short_kernel(r["Kernel_Name"])
        if k is None or r["Counter_Name"] != counter:
            continue
        out[(k, _grid(r))][r.get("Dispatch_Id", r.get("Correlation_Id"))] += float(r["Counter_Value"])
    return out


def _main_group(groups: dict, kernel: str, largest_grid: bool = False):
    """The (grid, values) of `kernel` with the most dispatches (the timed launches), or, where
    several layers launch the kernel equally often, the largest grid among those launched at
    least 8 times (the timed steps, not the one-off prefix build)."""
    cand = [(len(v), g, list(v.values())) for (k, g), v in groups.items() if k == kernel]
    if largest_grid:
        cand = [c for c in cand if c[0] >= 8]
    if not cand:
        raise SystemExit(f"no dispatches of {kernel}")
    if largest_grid:
        size = lambda g: int(np.prod([int(x) for x in g.split("x")])) if g != "?" else 0
        n, g, vals = max(cand, key=lambda c: size(c[1]))
    else:
        n, g, vals = max(cand)
    return g, vals


def write_traffic_profile(a):
    cf = _main_group(_pmc(a.calib_fetch, "FETCH_SIZE"), "copy")[1]
    cw = _main_group(_pmc(a.calib_write, "WRITE_SIZE"), "copy")[1]
    ff = COPY_CALIB_BYTES / (np.mean(cf) * 1024.0)
    wf = COPY_CALIB_BYTES / (np.mean(cw) * 1024.0)
    g, fv = _main_group(_pmc(a.fetch, "FETCH_SIZE"), a.kernel, a.largest_grid)
    gw, wv = _main_group(_pmc(a.write, "WRITE_SIZE"), a.kernel, a.largest_grid)
    traffic = np.mean(fv) * 1024.0 * ff + np.mean(wv) * 1024.0 * wf
    with open(a.out, "w") as f:
        f.write(f"# HBM traffic of {a.kernel}: {a.title}\n")
        f.write("# commands (run on the MI355X box from the repository root; each --pmc pass its own run):\n")
        for c in a.command:
            f.write(f"#   {c}\n")
        f.write("# FETCH_SIZE / WRITE_SIZE are KiB per dispatch, summed over the counter's instances;\n"
                "# each is scaled by the ratio of known bytes to the counter's reading on the copy.\n")
        f.write(f"kernel: {a.kernel}\n")
        f.write(f"source_digest: {kernel_source_digest(a.kernel)}\n")
        f.write(f"grid: {g}\n")
        f.write(f"dispatches: {len(fv)} fetch, {len(wv)} write\n")
        f.write(f"fetch_kib_per_dispatch: {np.mean(fv):.1f}\n")
        f.write(f"write_kib_per_dispatch: {np.mean(wv):.1f}\n")
        f.write(f"copy_calibration: {COPY_CALIB_BYTES} bytes read and written; FETCH_SIZE {np.mean(cf):.1f} KiB, "
                f"WRITE_SIZE {np.mean(cw):.1f} KiB -> scale {ff:.4f} (fetch), {wf:.4f} (write)\n")
        f.write(f"traffic_bytes_per_launch: {traffic:.0f}\n")
    print(open(a.out).read())


def traffic_from_profile(path: str, kernel: str):
    """Bytes per launch from a committed traffic summary, or None when it is absent or was
    measured on other sources of the kernel."""
    try:
        kv = dict(l.split(": ", 1) for l in open(path).read().splitlines() if not l.startswith("#") and ": " in l)
    except OSError:
        return None
    if kv.get("kernel") != kernel or kv.get("source_digest") != kernel_source_digest(kernel):
        return None
    return float(kv["traffic_bytes_per_launch"])


def write_step_traffic_profile(a):
    """HBM bytes per dispatch of every library kernel launched at least 8 times in the run
    (the timed steps; the one-off prefix build falls below), one line per kernel: the
    per-step traffic of a workload is then the sum over its kernels of launches per step
    times bytes per dispatch."""
    cf = _main_group(_pmc(a.calib_fetch, "FETCH_SIZE"), "copy")[1]
    cw = _main_group(_pmc(a.calib_write, "WRITE_SIZE"), "copy")[1]
    ff = COPY_CALIB_BYTES / (np.mean(cf) * 1024.0)
    wf = COPY_CALIB_BYTES / (np.mean(cw) * 1024.0)
    fetch, write = _pmc(a.fetch, "FETCH_SIZE"), _pmc(a.write, "WRITE_SIZE")
    per = defaultdict(lambda: [[], []])
    for (k, g), v in fetch.items():
        if len(v) >= 8 and k != "copy":
            per[k][0] += list(v.values())
    for (k, g), v in write.items():
        if len(v) >= 8 and k != "copy":
            per[k][1] += list(v.values())
    with open(a.out, "w") as f:
        f.write(f"# HBM traffic per dispatch of each kernel of a step: {a.title}\n")
        f.write("# commands (run on the MI355X box from the repository root; each --pmc pass its own run):\n")
        for c in a.command:
            f.write(f"#   {c}\n")
        f.write(f"# copy_calibration: {COPY_CALIB_BYTES} bytes; FETCH_SIZE {np.mean(cf):.1f} KiB, WRITE_SIZE "
                f"{np.mean(cw):.1f} KiB -> scale {ff:.4f} (fetch), {wf:.4f} (write)\n")
        f.write("# kernel | source_digest | dispatches | fetch_kib | write_kib | bytes_per_dispatch\n")
        for k, (fv, wv) in sorted(per.items()):
            if not fv or not wv:
                continue
            byts = np.mean(fv) * 1024.0 * ff + np.mean(wv) * 1024.0 * wf
            f.write(f"step_kernel: {k} | {kernel_source_digest(k)} | {len(fv)} | {np.mean(fv):.1f} | "
                    f"{np.mean(wv):.1f} | {byts:.0f}\n")
    print(open(a.out).read())


def step_traffic_from_profile(path: str, per_kernel: dict, steps: int):
    """HBM bytes per step: the launches per step of each traced kernel times its bytes per
    dispatch from a committed step-traffic summary; None when the summary is absent, lacks a
    kernel, or was measured on other sources of one."""
    try:
        lines = [l.split(": ", 1)[1] for l in open(path).read().splitlines()
                 if l.startswith("step_kernel: ")]
    except OSError:
        return None
    table = {}
    for l in lines:
        k, digest, _, _, _, byts = [x.strip() for x in l.split("|")]
        table[k] = (digest, float(byts))
    total = 0.0
    for name, (n, _) in per_kernel.items():
        if not n:
            continue
        if name not in table or table[name][0] != kernel_source_digest(name):
            return None
        total += n / steps * table[name][1]
    return total


def write_kernel_profile(a):
    groups = defaultdict(list)
    for r in _csv_rows(a.trace_dir, "*kernel_trace.csv"):
        k = _short_kernel(r["Kernel_Name"], with_args=True)
        if k is None or k == "copy":
            continue
        groups[(k, _grid(r))].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    with open(a.out, "w") as f:
        f.write(f"# rocprofv3 kernel summary: {a.title}\n")
        f.write("# commands (run on the MI355X box from the repository root):\n")
        for c in a.command:
            f.write(f"#   {c}\n")
        f.write("# per (kernel, grid) from kernel_trace.csv of that run; library kernels only (the input\n"
                "# generation and copies of the setup are omitted).  The grid with the most launches is the\n"
                "# timed one; others come from building the prefix cache once per run.\n#\n")
        f.write(f"# {'kernel':<32s} {'grid':<22s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_us':>12s}\n")
        for (k, g), v in sorted(groups.items(), key=lambda x: -sum(x[1])):
            f.write(f"  {k:<32s} {g:<22s} {len(v):6d} {np.mean(v):10.2f} {min(v):10.2f} {max(v):10.2f} {sum(v):12.1f}\n")
    print(open(a.out).read())


def main():
    if len(sys.argv) > 1 and sys.argv[1] in ("--write-traffic-profile", "--write-kernel-profile",
                                              "--write-step-traffic-profile"):
        mode = sys.argv[1]
        pp = argparse.ArgumentParser(prog=f"bench.py {mode}")
        pp.add_argument("--out", required=True)
        pp.add_argument("--title", required=True)
        pp.add_argument("--command", action="append", default=[])
        pp.add_argument("--kernel")
        pp.add_argument("--fetch")
        pp.add_argument("--write")
        pp.add_argument("--calib-fetch")
        pp.add_argument("--calib-write")
        pp.add_argument("--trace-dir")
        pp.add_argument("--largest-grid", action="store_true",
                        help="take the kernel's dispatches of the largest grid launched 8+ times")
        a = pp.parse_args(sys.argv[2:])
        {"--write-traffic-profile": write_traffic_profile, "--write-kernel-profile": write_kernel_profile,
         "--write-step-traffic-profile": write_step_traffic_profile}[mode](a)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--copy-calibration":
        copy_calibration()
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--context", type=int, default=65536)
    ap.add_argument("--decode-batch", type=int, default=8)
    ap.add_argument("--chunk", type=int, default=2048)
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--cpu-decode-steps", type=int, default=512,
                    help="decode steps of the oracle's sample (a multiple of 128: row emissions at their natural rate)")
    ap.add_argument("--cpu-decode-seqs", type=int, default=8)
    ap.add_argument("--cpu-prefill-queries", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-batch-scan", action="store_true",
                    help="leave out the decode batch scan (batch 32 and 128 at the headline shape)")
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-stack", action="store_true",
                    help="leave out the 262,144-token [0, 4, 128] stack decode sub-line")
    ap.add_argument("--only", choices=["decode", "prefill", "stack", "pro", "shared"], default=None,
                    help="run one workload (for per-workload profiler runs); the JSON line "
                         "then carries that workload's numbers only")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the CSA layer here runs on a single MI355X and has no "
              "multi-GPU path; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    K.lib()
    if args.only == "stack":             # stack-only profiler run
        stack = bench_stack(args, traffic_profile=TRAFFIC_STACK, step_traffic_profile=TRAFFIC_STACK_STEP)
        log(f"[stack] graph {stack['tok_s']:.0f} tok/s, {stack['ms_per_step']:.4f} ms/step")
        print(json.dumps({"workload": "stack", "decode_262k_stack": stack}), flush=True)
        return
    if args.only == "pro":               # V4-Pro-stack-only run
        print(json.dumps({"workload": "pro", "decode_262k_pro_stack":
                          bench_stack(args, ratios=(128, 128, 4, 128), topk=1024)}), flush=True)
        return
    if args.only == "shared":            # shared-KV-only run
        print(json.dumps({"workload": "shared", "decode_262k_shared_kv": bench_shared(args)}), flush=True)
        return
    dec = pre = None
    if args.only != "prefill":
        dec, dec_state = bench_decode(args)
        log(f"[decode] graph {dec['tok_s']:.0f} tok/s, {dec['ms_per_step']:.4f} ms/step "
            f"(raw {dec['raw']['ms_per_step']:.4f}); eager {dec['eager']['tok_s']:.0f} tok/s; whole step "
            f"{dec['roofline']['frac'] * 100:.1f}% of HBM ({dec['roofline']['kernel_us_per_step']:.2f} us of "
            f"kernels); {dec['roofline']['dominant_kernel']['kernel']} "
            f"{dec['roofline']['dominant_kernel']['frac'] * 100:.1f}%")
    if not args.skip_prefill and args.only != "decode":
        pre, pre_state = bench_prefill(args)
        log(f"[prefill] {pre['tok_s']:.0f} tok/s, {pre['ms_per_chunk']:.3f} ms/chunk; whole chunk "
            f"{pre['roofline']['frac'] * 100:.1f}% of MFMA ({pre['roofline']['kernel_us_per_chunk']:.0f} us "
            f"of kernels); {pre['roofline']['dominant_kernel']['kernel']} "
            f"{pre['roofline']['dominant_kernel']['frac'] * 100:.1f}%")
    outp = None
    if args.only is None:
        outp = bench_output_path(args)
        log(f"[output path] decode b8 {outp['decode_b8']['us_per_call']:.1f} us "
            f"({outp['decode_b8']['roofline']['frac'] * 100:.0f}% of HBM in the projection); prefill 2048 "
            f"{outp['prefill_2048']['us_per_call']:.1f} us ({outp['prefill_2048']['roofline']['frac'] * 100:.0f}% of MFMA); "
            f"compressor lanes of 2048 tokens {outp['lanes_prefill_2048']['us_per_call']:.1f} us")
    stack = pro = shared = None
    if not args.skip_stack and args.only is None:
        stack = bench_stack(args, traffic_profile=TRAFFIC_STACK, step_traffic_profile=TRAFFIC_STACK_STEP)
        log(f"[stack] graph {stack['tok_s']:.0f} tok/s, {stack['ms_per_step']:.4f} ms/step; whole step "
            f"{stack['roofline']['frac'] * 100:.1f}% of HBM; index scan "
            f"{stack['roofline']['dominant_kernel']['frac'] * 100:.1f}%")
        pro = bench_stack(args, ratios=(128, 128, 4, 128), topk=1024)
        log(f"[pro stack] graph {pro['tok_s']:.0f} tok/s, {pro['ms_per_step']:.4f} ms/step; whole step "
            f"{pro['roofline']['frac'] * 100:.1f}% of HBM")
        shared = bench_shared(args)
        log(f"[shared] graph {shared['tok_s']:.0f} tok/s, {shared['ms_per_step']:.4f} ms/step "
            f"({shared['us_per_layer']:.1f} us per layer); index scan {shared['roofline']['achieved']:.0f} GB/s")
    scan = None
    if args.only is None and dec is not None and not args.skip_batch_scan:
        scan = bench_decode_batch_scan(args)
        log("[decode batch scan] " + "; ".join(
            f"batch {e['batch']}: {e['tok_s']:.0f} tok/s, {e['ms_per_step'] * 1e3:.1f} us/step, whole step "
            f"{e['whole_step_hbm_frac'] * 100:.1f}% of HBM" for e in scan))
    if dec is None:                      # prefill-only profiler run
        print(json.dumps({"workload": "prefill", "prefill": pre}), flush=True)
        return
    cpu = None
    if not args.no_cpu_baseline:
        t_cpu = time.time()
        dspec, dseed = dec_state
        cpu = cpu_baseline_decode(dspec, dseed, args.context, args.cpu_decode_seqs,
                                  args.cpu_decode_steps, device="cuda")
        if pre is not None:
            pspec, pseed, pstart, pS = pre_state
            cpu["prefill"] = cpu_baseline_prefill(pspec, pseed, pstart, pS, args.cpu_prefill_queries,
                                                  device="cuda")
        cpu["host"] = platform.processor() or platform.machine()
        log(f"[cpu baseline] decode {cpu['value']:.1f} tok/s on {cpu['cores']} threads "
            f"({time.time() - t_cpu:.1f}s with setup)")
    line = {
        "metric": "CSA decode tokens/s and prefill tokens/s at 64K ctx; % HBM/MFMA peak",
        "value": dec["tok_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode, ratio-128 layer, batch {args.decode_batch}, context "
                               f"{args.context}, 64 heads x 512 latent, window 128, all rows attended",
                   "global_batch": args.decode_batch, "seq_len": args.context,
                   "parallelism": "single-gpu"},
        "roofline": dec["roofline"],
        "decode_mode": dec["mode"],
        "decode_raw": dec["raw"],
        "decode_emission": dec["emission"],
        "decode_bytes_per_step": dec["bytes_per_step"],
        "eager": dec["eager"],
        "kernels": dec["kernels"],
        "prefill": pre,
        "decode_batch_scan": scan,
        "decode_262k_stack": stack,
        "decode_262k_pro_stack": pro,
        "decode_262k_shared_kv": shared,
        "output_path": outp,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
