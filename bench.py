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
    n, ms = K.dsv4_trace_read(name)
    return n, ms


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max(int(i.get("num_threads", 1)) for i in threadpool_info()) or 1
    except Exception:
        return os.cpu_count() or 1


# ------------------------------------------------------------------ decode @ 64K
def bench_decode(args, seed=0):
    spec = LayerSpec(ratio=128, indexer=False, topk=0)
    B, L = args.decode_batch, args.context
    steps, warm = args.steps, args.warmup
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, L + warm + 3 * steps + 8, params, device="cuda", max_chunk=spec.window)
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
    K.dsv4_trace_reset()
    t0 = time.perf_counter()
    for i in range(warm, warm + steps):
        layer.decode(toks[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # kernel durations, measured in a second identical pass with the event trace on
    K.dsv4_trace_enable(True)
    K.dsv4_trace_reset()
    pos = list(layer.lengths)
    for i in range(warm, warm + steps):
        layer.decode(toks[i])
    torch.cuda.synchronize()
    names = K.dsv4_trace_kernels()
    per_kernel = {n: kernel_time(n) for n in names}
    K.dsv4_trace_enable(False)
    # the same steps captured once as a HIP graph and replayed: every launch and argument of
    # the K steps is recorded, so a replay costs no host work per launch.  The state is
    # restored before each replay (outside the timed region), so the replay recomputes
    # exactly the captured positions.
    snap = {n: getattr(layer, n).clone() for n in ("ring", "state", "rows")}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(warm, warm + steps):
            layer.decode(toks[i])

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
    attn_name = max((n for n in per_kernel if n.startswith("attn")), key=lambda n: per_kernel[n][1])
    n_l, ms_l = per_kernel[attn_name]
    # algorithmic bytes of one decode attention launch: q and out (bf16) + every attended key
    keys = spec.window + (L + warm) // spec.ratio
    bytes_launch = B * (2 * spec.heads * spec.dim * 2 + keys * spec.dim * 2)
    achieved = bytes_launch / (ms_l / n_l * 1e-3) / 1e9
    res = {
        "tok_s": B * steps / g_wall, "ms_per_step": g_wall / steps * 1e3,
        "mode": "hip-graph replay of the K captured steps",
        "graph_events_ms_per_step": g_ev / steps * 1e3,
        "eager": {"tok_s": B * steps / wall, "ms_per_step": wall / steps * 1e3,
                  "mode": "one library call per lane per step from Python"},
        "kernels": {n: {"launches": v[0], "avg_us": v[1] / max(1, v[0]) * 1e3} for n, v in per_kernel.items()},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile(TRAFFIC_DECODE, attn_name), "kernel": attn_name,
                     "bytes_per_launch": bytes_launch},
    }
    layer_state = (layer, toks, spec, params, pos)
    return res, layer_state


def bench_stack(args, seed=23, ratios=(0, 4, 128), topk=512, traffic_profile=None):
    """Decode of a layer stack at 262,144 tokens, batch 4.  The default is V4-Flash's head
    [0, 4, 128]: a window-only layer, a ratio-4 layer (65,536 rows, indexer top-512) and a
    ratio-128 layer (2048 rows, top-512); ratios (128, 128, 4, 128) with topk 1024 is
    V4-Pro's head (no window-only layer, top-1024).  A step is one decode token of every
    sequence through all layers; the K steps are replayed as a HIP graph like the headline
    decode.  The roofline is the ratio-4 layer's indexer scan (HBM-bound: every visible
    indexer row is read once per step); its HBM traffic is read from ``traffic_profile`` (the
    counters of that stack's run), None when no such profile is given."""
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
        layer = CsaLayer(spec, B, L + warm + 3 * steps + 8, params, device="cuda", max_chunk=spec.window)
        build_prefix(layer, spec, lseed, L)
        layers.append(layer)
        tl = []
        for j in range(warm + steps):
            t = SC.batch_token_inputs(spec, lseed, [L + j] * B, 1, device="cuda")
            tl.append({k: v[:, 0].contiguous() for k, v in t.items()})
        toks.append(tl)
    log(f"[stack] {list(ratios)} (top-{topk}) at {L} tokens x {B} built in {time.time() - t_setup:.1f}s")

    def step(j, trace_layer=None):
        for i, layer in enumerate(layers):
            if trace_layer is not None:
                K.dsv4_trace_enable(i == trace_layer)
            layer.decode(toks[i][j])
        if trace_layer is not None:
            K.dsv4_trace_enable(False)

    for j in range(warm):
        step(j)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(warm, warm + steps):
        step(j)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # kernel durations of the ratio-4 layer, in a second identical pass with the trace on
    K.dsv4_trace_reset()
    for j in range(warm, warm + steps):
        step(j, trace_layer=i4)
    torch.cuda.synchronize()
    per_kernel = {n: kernel_time(n) for n in K.dsv4_trace_kernels()}
    # graph replay of the K steps (state restored outside the timed region)
    names = ("ring", "state", "rows", "state_i", "rows_i")
    snap = [{n: getattr(l, n).clone() for n in names if hasattr(l, n)} for l in layers]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(warm, warm + steps):
            step(j)

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
    spec4 = specs[i4]
    nv = (L + warm) // spec4.ratio
    n_l, ms_l = per_kernel["index_score_stream"]
    # algorithmic bytes of one scan: every visible indexer row, the queries and head weights
    bytes_launch = B * (nv * spec4.index_dim * 2 + spec4.index_heads * (spec4.index_dim * 2 + 4))
    achieved = bytes_launch / (ms_l / n_l * 1e-3) / 1e9
    return {
        "workload": f"decode, {list(ratios)} stack ("
                    + ", ".join("window-only" if r == 0 else
                                f"ratio-{r} with top-{topk} over ~{(L + warm) // r} rows" for r in ratios)
                    + f"), batch {B}, context {L}",
        "tok_s": B * steps / g_wall, "ms_per_step": g_wall / steps * 1e3,
        "mode": f"hip-graph replay of the K captured steps ({len(ratios)} layers per step)",
        "eager": {"tok_s": B * steps / wall, "ms_per_step": wall / steps * 1e3},
        "kernels_ratio4_layer": {n: {"launches": v[0], "avg_us": v[1] / max(1, v[0]) * 1e3}
                                 for n, v in per_kernel.items()},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": (traffic_from_profile(traffic_profile, "index_score_stream")
                                                                  if traffic_profile else None),
                     "kernel": "index_score_stream",
                     "bytes_per_launch": bytes_launch},
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
    # kernel durations in a second pass with the trace on (positions keep advancing, as in
    # bench_stack: the layers hold room for the three passes)
    K.dsv4_trace_reset()
    K.dsv4_trace_enable(True)
    for j in range(warm, warm + steps):
        step(j)
    torch.cuda.synchronize()
    K.dsv4_trace_enable(False)
    per_kernel = {n: kernel_time(n) for n in K.dsv4_trace_kernels()}
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
    n_l, ms_l = per_kernel["index_score_stream"]
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
        "kernels": {n: {"launches": v[0], "avg_us": v[1] / max(1, v[0]) * 1e3} for n, v in per_kernel.items()},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "index_score_stream",
                     "bytes_per_launch": bytes_launch},
    }


def cpu_baseline_decode(layer_state, sample_steps):
    """The oracle doing the same decode work (window + all visible rows, per sequence) on
    the host, for ``sample_steps`` steps of every sequence.  Rows and ring are the GPU
    caches copied to the host (the oracle consumes them as inputs)."""
    import oracle
    layer, toks, spec, params, pos = layer_state
    B = layer.batch
    rows = layer.rows.float().cpu().numpy().astype(np.float64)
    sinks = params["sinks"].cpu().numpy()
    n = pos[0]
    kv_hist = np.random.default_rng(0).standard_normal((spec.window, spec.dim))
    t0 = time.perf_counter()
    done = 0
    for i in range(sample_steps):
        for b in range(B):
            q = toks[i]["q"][b].float().cpu().numpy()[None].astype(np.float64)
            p = n + i
            kv = np.concatenate([kv_hist[1:], toks[i]["kv"][b].float().cpu().numpy()[None]])
            nv = min(oracle.visible_rows(p, spec.ratio), rows.shape[1])
            oracle.csa_attention(q, kv, rows[b, :nv], None, [p], window=spec.window,
                                 ratio=spec.ratio, sinks=sinks, scale=spec.scale, store="bf16",
                                 kv_offset=p - spec.window + 1)
            done += 1
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{sample_steps} decode steps x {B} sequences of the 64K ratio-128 layer "
                      f"(window + {rows.shape[1]} rows per query), numpy fp32 oracle"}


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
    K.dsv4_trace_enable(True)
    K.dsv4_trace_reset()
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    names = K.dsv4_trace_kernels()
    per_kernel = {n: kernel_time(n) for n in names}
    K.dsv4_trace_enable(False)
    # algorithmic flops of the chunk: indexer q.k over every visible row, attention QK^T and PV
    idx_pairs = sum(min((p + 1) // 4, L // 4) for p in range(start, L))
    idx_flops = 2.0 * spec.index_heads * spec.index_dim * idx_pairs
    keys = sum(spec.window + min(spec.topk, (p + 1) // 4) for p in range(start, L))
    attn_flops = 4.0 * spec.heads * spec.dim * keys
    dom = max(per_kernel, key=lambda n: per_kernel[n][1])
    n_d, ms_d = per_kernel[dom]
    dom_flops = idx_flops if "index" in dom else attn_flops if "attn" in dom else 0.0
    achieved = dom_flops / (ms_d / n_d * 1e-3) / 1e12
    total_ms = sum(v[1] for v in per_kernel.values()) / reps
    res = {
        "tok_s": S / wall, "ms_per_chunk": wall * 1e3,
        "workload": f"ratio-4 layer, chunk {start}->{L} (S={S}), indexer top-{spec.topk}, "
                    f"64 heads x 512 latent, bf16",
        "flops_per_chunk": idx_flops + attn_flops,
        "tflops_whole_chunk": (idx_flops + attn_flops) / (total_ms * 1e-3) / 1e12,
        "kernels": {n: {"launches": v[0], "avg_us": v[1] / max(1, v[0]) * 1e3} for n, v in per_kernel.items()},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                     "traffic": traffic_from_profile(TRAFFIC_PREFILL, dom),
                     "kernel": dom, "flops_per_launch": dom_flops},
    }
    return res, (layer, tok, spec, params, start, sel)


def cpu_baseline_prefill(state, n_queries):
    """The oracle on ``n_queries`` queries of the same chunk: indexer scores over every
    visible row, top-k, attention over window + selected rows (rows from the GPU cache)."""
    import oracle
    layer, tok, spec, params, start, _ = state
    rows = layer.rows[0].float().cpu().numpy().astype(np.float64)
    rows_i = layer.rows_i[0].float().cpu().numpy().astype(np.float64)
    sinks = params["sinks"].cpu().numpy()
    S = tok["q"].shape[1]
    idx = np.linspace(spec.window - 1, S - 1, n_queries).astype(int)   # windows inside the chunk
    q = tok["q"][0].float().cpu().numpy().astype(np.float64)
    kv = tok["kv"][0].float().cpu().numpy().astype(np.float64)
    qi = tok["qi"][0].float().cpu().numpy()
    w = tok["w"][0].cpu().numpy()
    t0 = time.perf_counter()
    for i in idx:
        p = start + int(i)
        nv = oracle.visible_rows(p, spec.ratio)
        sc = oracle.index_scores(qi[i:i + 1], w[i:i + 1], rows_i[:nv])
        sel = oracle.select_topk(sc, [p], ratio=spec.ratio, k=spec.topk)
        lo = int(i) - spec.window + 1
        oracle.csa_attention(q[i:i + 1], kv[lo:i + 1], rows, sel, [p], window=spec.window,
                             ratio=spec.ratio, sinks=sinks, scale=spec.scale, store="bf16",
                             kv_offset=start + lo)
    dt = time.perf_counter() - t0
    return {"value": n_queries / dt, "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{n_queries} of the {S} queries of the 64K prefill chunk (indexer over "
                      f"~16K rows, top-512, attention), numpy fp32 oracle"}


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
    # [1024, 4096]): two one-group projections of 128 x 128 tiles
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
    for _ in range(10):
        compressor_lanes(x, wkv, wg)
    torch.cuda.synchronize()
    K.dsv4_trace_enable(False)
    n_g, ms_g = kernel_time("gproj")
    us = ms_g / n_g * 1e3
    fl = 2.0 * T * W * hid
    ach = fl / (us * 1e-6) / 1e12
    out["lanes_prefill_2048"] = {
        "tokens": T, "us_per_call": 2 * us,
        "roofline": {"bound": "mfma", "achieved": ach, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / BF16_MFMA_PEAK_TFLOPS, "traffic": None, "kernel": "gproj_tile",
                     "flops_per_launch": fl}}
    return out


# ------------------------------------------------------------------ profiles
# The summaries under profiles/ are written from rocprofv3 output by the modes below (no GPU
# needed), so each one names commands that run committed files only.  A traffic summary
# records a digest of its kernel's sources; the JSON line reports its traffic only while the
# sources still match (a changed kernel reports null until it is measured again).
CSRC = os.path.join(ROOT, "sparse_attention_dsv4_amd", "csrc")
KERNEL_SOURCES = {"attn": "attention.hip", "ring": "attention.hip", "index": "indexer.hip",
                  "topk": "indexer.hip", "compress": "compress.hip"}
COPY_CALIB_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_DECODE = os.path.join(PROFILES, "traffic_attn_decode_ctx65536_b8_ratio128.txt")
TRAFFIC_PREFILL = os.path.join(PROFILES, "traffic_index_score_rs_ctx65536_chunk2048_ratio4.txt")
TRAFFIC_STACK = os.path.join(PROFILES, "traffic_index_score_stream_decode_ctx262144_b4_stack.txt")


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
    if len(sys.argv) > 1 and sys.argv[1] in ("--write-traffic-profile", "--write-kernel-profile"):
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
        (write_traffic_profile if mode == "--write-traffic-profile" else write_kernel_profile)(a)
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
    ap.add_argument("--cpu-decode-steps", type=int, default=64)
    ap.add_argument("--cpu-prefill-queries", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        stack = bench_stack(args, traffic_profile=TRAFFIC_STACK)
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
        log(f"[decode] graph {dec['tok_s']:.0f} tok/s, {dec['ms_per_step']:.4f} ms/step; "
            f"eager {dec['eager']['tok_s']:.0f} tok/s, {dec['eager']['ms_per_step']:.4f} ms/step")
    if not args.skip_prefill and args.only != "decode":
        pre, pre_state = bench_prefill(args)
        log(f"[prefill] {pre['tok_s']:.0f} tok/s, {pre['ms_per_chunk']:.3f} ms/chunk")
    outp = None
    if args.only is None:
        outp = bench_output_path(args)
        log(f"[output path] decode b8 {outp['decode_b8']['us_per_call']:.1f} us "
            f"({outp['decode_b8']['roofline']['frac'] * 100:.0f}% of HBM in the projection); prefill 2048 "
            f"{outp['prefill_2048']['us_per_call']:.1f} us ({outp['prefill_2048']['roofline']['frac'] * 100:.0f}% of MFMA); "
            f"compressor lanes of 2048 tokens {outp['lanes_prefill_2048']['us_per_call']:.1f} us")
    stack = pro = shared = None
    if not args.skip_stack and args.only is None:
        stack = bench_stack(args, traffic_profile=TRAFFIC_STACK)
        log(f"[stack] graph {stack['tok_s']:.0f} tok/s, {stack['ms_per_step']:.4f} ms/step; index scan "
            f"{stack['roofline']['achieved']:.0f} GB/s ({stack['roofline']['frac'] * 100:.1f}% of HBM)")
        pro = bench_stack(args, ratios=(128, 128, 4, 128), topk=1024)
        log(f"[pro stack] graph {pro['tok_s']:.0f} tok/s, {pro['ms_per_step']:.4f} ms/step; index scan "
            f"{pro['roofline']['achieved']:.0f} GB/s ({pro['roofline']['frac'] * 100:.1f}% of HBM)")
        shared = bench_shared(args)
        log(f"[shared] graph {shared['tok_s']:.0f} tok/s, {shared['ms_per_step']:.4f} ms/step "
            f"({shared['us_per_layer']:.1f} us per layer); index scan {shared['roofline']['achieved']:.0f} GB/s")
    if dec is None:                      # prefill-only profiler run
        print(json.dumps({"workload": "prefill", "prefill": pre}), flush=True)
        return
    cpu = None
    if not args.no_cpu_baseline:
        cpu = {"decode": cpu_baseline_decode(dec_state, args.cpu_decode_steps)}
        if pre is not None:
            cpu["prefill"] = cpu_baseline_prefill(pre_state, args.cpu_prefill_queries)
        cpu = dict(cpu["decode"], prefill=cpu.get("prefill"),
                   host=platform.processor() or platform.machine())
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
        "eager": dec["eager"],
        "kernels": dec["kernels"],
        "prefill": pre,
        "decode_262k_stack": stack,
        "decode_262k_pro_stack": pro,
        "decode_262k_shared_kv": shared,
        "output_path": outp,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
