"""Parity at the full sizes the benchmark times, in the same launch configuration (needs a
gfx950 GPU).

The layer is driven exactly as bench.py drives it (same seeds, prefix builder, batch, chunk
and call sequence), and sampled outputs are checked against the oracle one by one:
  * decode, ratio-128 layer, batch 8, context 65,536 (512 rows + 128-token window per query):
    sampled rows against the oracle compressor; every sequence's output of three decode steps
    against the oracle attention over the GPU's rows; the same at batches 32 and 128 (the
    batch scan), on sampled sequences;
  * prefill, ratio-4 layer with the indexer, the 2048-token chunk 63,488 -> 65,536: sampled
    rows of both lanes, then for sampled queries the top-512 over ~16K visible rows (exact up
    to the 1e-5 band) and the attention output.
and at the other stated workload sizes, with the same sampling:
  * ratio-4 decode, batch 1, context 8192 (2048 rows, sparse), 9 steps across row births;
  * chunked prefill of 16,384 tokens in 2048-token chunks on a ratio-4 layer;
  * the [0, 4, 128] stack at 262,144 tokens, batch 4, 256 decode steps (65,536 rows and
    top-512 on the ratio-4 layer; 2048 rows and top-512 on the ratio-128 layer).
Stage isolation as in the other parity tests: each oracle stage consumes the GPU's upstream
result (rows, then the selection), so a bf16 rounding upstream cannot move a later check.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth.csa as SC
from sparse_attention_dsv4_amd.layer import CsaLayer, LayerSpec
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _params64(spec, seed):
    return {k: G.f64(v) for k, v in SC.layer_params(spec, seed).items()}


def _lanes(spec, seed, b, t0, t1, fields):
    return {k: G.f64(v) for k, v in SC.token_inputs(spec, seed, b, t0, t1, fields=fields).items()}


def _check_rows(spec, seed, gpu_rows, b, js, index_lane=False):
    par = _params64(spec, seed)
    r, coff = spec.ratio, spec.coff
    for j in js:
        t0 = max(0, (j - (coff - 1)) * r)
        f = ["ai", "gi"] if index_lane else ["a", "g"]
        ln = _lanes(spec, seed, b, t0, (j + 1) * r, f)
        a, g = ln[f[0]], ln[f[1]]
        ape, gam = (par["ape_i"], par["norm_w_i"]) if index_lane else (par["ape"], par["norm_w"])
        ref = oracle.compressor_rows(a, g, ape, gam, par["inv_freq"], ratio=r, overlap=spec.is_overlap,
                                     eps=spec.eps, store="bf16", rows=[j], token0=t0)
        G.assert_rows_match(G.f64(gpu_rows[b, j])[None], ref, "bf16",
                            f"{'indexer' if index_lane else 'attention'} row {j} of sequence {b}",
                            spec.rope_dim)


@pytest.mark.parametrize("B", [8, 32, 128])
def test_fullsize_decode_64k_ratio128(B):
    """The decode benchmark's layer and context at batch 8 (splits of one LDS chunk) and at
    the batch scan's 32 and 128 (splits of 320 and 640 keys: double-buffered 64-key chunks,
    the head groups of a split grouped on one XCD); sampled sequences against the oracle."""
    spec = LayerSpec(ratio=128, indexer=False, topk=0)
    seed, L, steps = 0, 65536, 3                     # bench_decode's seed and context
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, L + steps + 8, params, device="cuda", max_chunk=spec.window)
    bench.build_prefix(layer, spec, seed, L)
    outs = []
    for i in range(steps):
        t = SC.batch_token_inputs(spec, seed, [L + i] * B, 1, device="cuda", fields=["q", "kv", "a", "g"])
        outs.append(layer.decode({k: v[:, 0].contiguous() for k, v in t.items()}).cpu())
    torch.cuda.synchronize()
    rows = layer.rows.cpu()
    for b in (0, 5, B - 1):
        _check_rows(spec, seed, rows, b, [0, 1, 255, 510, 511])
    par = _params64(spec, seed)
    worst = 0.0
    seqs = range(B) if B <= 8 else sorted({0, 1, B // 2, B - 1})
    for i in range(steps):
        p = L + i
        nv = oracle.visible_rows(p, spec.ratio)
        for b in seqs:
            tk = _lanes(spec, seed, b, p - spec.window + 1, p + 1, ["q", "kv"])
            ref = oracle.csa_attention(tk["q"][-1:], tk["kv"], G.f64(rows[b, :nv]), None, [p],
                                       window=spec.window, ratio=spec.ratio, sinks=par["sinks"],
                                       scale=spec.scale, store="bf16", kv_offset=p - spec.window + 1)
            mr = G.max_rel_rows(G.f64(outs[i][b]), ref[0]).max()
            worst = max(worst, mr)
            assert mr <= 2e-2, f"step {i} sequence {b}: max-rel {mr:.3g}"
    print(f"  decode outputs: worst per-head max-rel {worst:.3g} over {steps * len(seqs)} queries x 64 heads")


def test_fullsize_prefill_chunk_64k_ratio4():
    spec = LayerSpec(ratio=4)
    seed, S, L = 1, 2048, 65536                      # bench_prefill's seed, chunk and context
    start = L - S
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, 1, L, params, device="cuda", max_chunk=max(S, spec.window))
    bench.build_prefix(layer, spec, seed, start)
    tok = SC.batch_token_inputs(spec, seed, [start], S, device="cuda")
    sel = torch.empty(1, S, spec.topk, dtype=torch.int32, device="cuda")
    out = layer.prefill(tok, sel_out=sel).cpu()
    torch.cuda.synchronize()
    rows, rows_i, sel = layer.rows.cpu(), layer.rows_i.cpu(), sel.cpu().numpy()
    js = [0, 1, 8191, start // 4 - 1, start // 4, L // 4 - 2, L // 4 - 1]
    _check_rows(spec, seed, rows, 0, js)
    _check_rows(spec, seed, rows_i, 0, js, index_lane=True)

    par = _params64(spec, seed)
    queries = [0, 1, 127, 128, 777, 1500, 2046, 2047]
    n_exact = n_band = 0
    for s in queries:
        p = start + s
        nv = oracle.visible_rows(p, spec.ratio)
        tk = _lanes(spec, seed, 0, p - spec.window + 1, p + 1, ["q", "kv", "qi", "w"])
        sc = oracle.index_scores(tk["qi"][-1:], tk["w"][-1:], G.f64(rows_i[0, :nv]))
        ref_sel = oracle.select_topk(sc, [p], ratio=spec.ratio, k=spec.topk)
        ne, nb, nbad, bad = G.topk_band_ok(sel[0, s:s + 1], ref_sel, sc, [p], spec)
        assert nbad == 0, f"query {s}: top-k differs outside the band: {bad}"
        n_exact += ne
        n_band += nb
        ref = oracle.csa_attention(tk["q"][-1:], tk["kv"], G.f64(rows[0, :nv]), sel[0, s:s + 1], [p],
                                   window=spec.window, ratio=spec.ratio, sinks=par["sinks"],
                                   scale=spec.scale, store="bf16", kv_offset=p - spec.window + 1)
        mr = G.max_rel_rows(G.f64(out[0, s]), ref[0]).max()
        assert mr <= 2e-2, f"query {s}: attention max-rel {mr:.3g}"
    print(f"  prefill: top-k exact {n_exact}, in band {n_band} of {len(queries)} sampled queries")


def _decode_steps(layer, spec, seed, B, L, steps):
    outs, sels = [], []
    for i in range(steps):
        t = SC.batch_token_inputs(spec, seed, [L + i] * B, 1, device="cuda")
        sel = (torch.empty(B, 1, spec.topk, dtype=torch.int32, device="cuda")
               if spec.has_indexer else None)
        outs.append(layer.decode({k: v[:, 0].contiguous() for k, v in t.items()}, sel_out=sel).cpu())
        sels.append(sel[:, 0].cpu().numpy() if sel is not None else None)
    torch.cuda.synchronize()
    return outs, sels


def _check_decode_queries(spec, seed, layer, outs, sels, L, samples):
    """Oracle per sampled (step, sequence): top-k over the GPU's indexer rows (band rule),
    then attention over the GPU's rows with the GPU's selection."""
    par = _params64(spec, seed)
    rows = layer.rows.cpu() if spec.has_rows else None
    rows_i = layer.rows_i.cpu() if spec.has_indexer else None
    worst, n_exact = 0.0, 0
    for i, b in samples:
        p = L + i
        nv = oracle.visible_rows(p, spec.ratio) if spec.has_rows else 0
        f = ["q", "kv"] + (["qi", "w"] if spec.has_indexer else [])
        tk = _lanes(spec, seed, b, max(0, p - spec.window + 1), p + 1, f)
        sel = None
        if spec.has_indexer:
            sc = oracle.index_scores(tk["qi"][-1:], tk["w"][-1:], G.f64(rows_i[b, :nv]))
            ref_sel = oracle.select_topk(sc, [p], ratio=spec.ratio, k=spec.topk)
            ne, nb, nbad, bad = G.topk_band_ok(sels[i][b:b + 1], ref_sel, sc, [p], spec)
            assert nbad == 0, f"step {i} sequence {b}: top-k differs outside the band: {bad}"
            n_exact += ne
            sel = sels[i][b:b + 1]
        ref = oracle.csa_attention(tk["q"][-1:], tk["kv"], G.f64(rows[b, :nv]) if rows is not None else None,
                                   sel, [p], window=spec.window, ratio=spec.ratio, sinks=par["sinks"],
                                   scale=spec.scale, store="bf16", kv_offset=max(0, p - spec.window + 1))
        mr = G.max_rel_rows(G.f64(outs[i][b]), ref[0]).max()
        worst = max(worst, mr)
        assert mr <= 2e-2, f"step {i} sequence {b}: max-rel {mr:.3g}"
    return worst, n_exact


def test_config_ratio4_decode_8k_batch1():
    """Ratio-4 layer with the indexer, batch 1, context 8192 (2048 rows, sparse regime);
    decode steps across two row births (rows 2048 and 2049)."""
    spec = LayerSpec(ratio=4)
    seed, B, L, steps = 21, 1, 8192, 9
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, L + steps + 8, params, device="cuda", max_chunk=spec.window)
    bench.build_prefix(layer, spec, seed, L)
    outs, sels = _decode_steps(layer, spec, seed, B, L, steps)
    _check_rows(spec, seed, layer.rows.cpu(), 0, [0, 1, 2047, 2048, 2049])
    _check_rows(spec, seed, layer.rows_i.cpu(), 0, [0, 1, 2047, 2048, 2049], index_lane=True)
    worst, ne = _check_decode_queries(spec, seed, layer, outs, sels, L, [(i, 0) for i in range(steps)])
    print(f"  8K ratio-4 decode: worst max-rel {worst:.3g}; top-k exact {ne} of {steps}")


def test_config_chunked_prefill_16k():
    """Chunked prefill of 16,384 tokens on a ratio-4 layer in 2048-token chunks (compressor
    state carried across chunks); sampled queries of the first, a middle and the last chunk."""
    spec = LayerSpec(ratio=4)
    seed, S, n = 22, 2048, 8
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, 1, S * n, params, device="cuda", max_chunk=S)
    outs, sels = [], []
    for c in range(n):
        tok = SC.batch_token_inputs(spec, seed, [c * S], S, device="cuda")
        sel = torch.empty(1, S, spec.topk, dtype=torch.int32, device="cuda")
        outs.append(layer.prefill(tok, sel_out=sel).cpu())
        sels.append(sel.cpu().numpy())
    torch.cuda.synchronize()
    js = [0, 511, 512, 2047, 2048, 4095]
    _check_rows(spec, seed, layer.rows.cpu(), 0, js)
    _check_rows(spec, seed, layer.rows_i.cpu(), 0, js, index_lane=True)
    par = _params64(spec, seed)
    rows, rows_i = layer.rows.cpu(), layer.rows_i.cpu()
    for c, s in [(0, 0), (0, 2047), (3, 5), (3, 1500), (7, 0), (7, 2047)]:
        p = c * S + s
        nv = oracle.visible_rows(p, spec.ratio)
        lo = max(0, p - spec.window + 1)
        tk = _lanes(spec, seed, 0, lo, p + 1, ["q", "kv", "qi", "w"])
        sc = oracle.index_scores(tk["qi"][-1:], tk["w"][-1:], G.f64(rows_i[0, :nv]))
        ref_sel = oracle.select_topk(sc, [p], ratio=spec.ratio, k=spec.topk)
        gsel = sels[c][0, s:s + 1]
        ne, nb, nbad, bad = G.topk_band_ok(gsel, ref_sel, sc, [p], spec)
        assert nbad == 0, f"chunk {c} query {s}: {bad}"
        ref = oracle.csa_attention(tk["q"][-1:], tk["kv"], G.f64(rows[0, :nv]), gsel, [p],
                                   window=spec.window, ratio=spec.ratio, sinks=par["sinks"],
                                   scale=spec.scale, store="bf16", kv_offset=lo)
        mr = G.max_rel_rows(G.f64(outs[c][0, s]), ref[0]).max()
        assert mr <= 2e-2, f"chunk {c} query {s}: max-rel {mr:.3g}"


@pytest.mark.parametrize("ratio", [0, 4, 128])
def test_config_stack_262k_batch4(ratio):
    """The [0, 4, 128] stack at 262,144 tokens, batch 4: a window-only layer, a ratio-4 layer
    (65,536 rows, top-512) and a ratio-128 layer (2048 rows, top-512).  256 decode steps, so
    rows are born on both compressed layers (every 4 and every 128 tokens); sampled steps
    are checked for every sequence."""
    spec = {0: LayerSpec(ratio=0, indexer=False, topk=0), 4: LayerSpec(ratio=4),
            128: LayerSpec(ratio=128)}[ratio]
    seed, B, L, steps = 23 + ratio, 4, 262144, 256
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, L + steps + 8, params, device="cuda", max_chunk=spec.window)
    bench.build_prefix(layer, spec, seed, L)
    outs, sels = _decode_steps(layer, spec, seed, B, L, steps)
    if spec.has_rows:
        n = (L + steps) // spec.ratio
        js = [0, L // spec.ratio - 1, L // spec.ratio, n - 1]
        for b in (0, 3):
            _check_rows(spec, seed, layer.rows.cpu(), b, js)
            _check_rows(spec, seed, layer.rows_i.cpu(), b, js, index_lane=True)
    samples = [(i, b) for i in (0, 3, 127, 255) for b in range(B)]
    worst, ne = _check_decode_queries(spec, seed, layer, outs, sels, L, samples)
    print(f"  262K ratio-{ratio} decode: worst max-rel {worst:.3g}; top-k exact {ne} of {len(samples)}")


@pytest.mark.parametrize("ratio", [4, 128])
def test_pro_stack_262k_batch4(ratio):
    """V4-Pro's head [128, 128, 4, 128] at 262,144 tokens, batch 4, top-1024: its two layer
    kinds, a ratio-128 layer (2048 rows, so the selection is sparse) and a ratio-4 layer
    (65,536 rows).  128 decode steps (a ratio-128 row is born on the way); sampled steps are
    checked for every sequence."""
    spec = LayerSpec(ratio=ratio, topk=1024)
    seed, B, L, steps = 51 + ratio, 4, 262144, 128
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, L + steps + 8, params, device="cuda", max_chunk=spec.window)
    bench.build_prefix(layer, spec, seed, L)
    outs, sels = _decode_steps(layer, spec, seed, B, L, steps)
    n = (L + steps) // spec.ratio
    js = [0, L // spec.ratio - 1, L // spec.ratio, n - 1]
    for b in (0, 3):
        _check_rows(spec, seed, layer.rows.cpu(), b, js)
        _check_rows(spec, seed, layer.rows_i.cpu(), b, js, index_lane=True)
    samples = [(i, b) for i in (0, 127) for b in range(B)]
    worst, ne = _check_decode_queries(spec, seed, layer, outs, sels, L, samples)
    print(f"  262K Pro ratio-{ratio} decode: worst max-rel {worst:.3g}; top-k exact {ne} of {len(samples)}")


@pytest.mark.parametrize("case", ["dense_ratio4_b8", "selected_b16"])
def test_decode_splits_longer_than_one_lds_chunk(case):
    """Decode splits that hold more keys than one LDS chunk (128 keys), so the attention
    workgroup runs several 64-key chunks (two buffers) with the running max carried between
    them: a dense ratio-4 lane at batch 8 (1500 rows + window: 240-key splits, four chunks),
    and the indexer's top-512 at batch 16 (640 keys: 160-key splits, three chunks, the
    selection compacted again for each)."""
    if case == "dense_ratio4_b8":
        spec = LayerSpec(ratio=4, indexer=False, topk=0)
        seed, B, L, steps = 31, 8, 6000, 2
    else:
        spec = LayerSpec(ratio=4)
        seed, B, L, steps = 32, 16, 4096, 2
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, L + steps + 8, params, device="cuda", max_chunk=spec.window)
    bench.build_prefix(layer, spec, seed, L)
    outs, sels = _decode_steps(layer, spec, seed, B, L, steps)
    samples = [(i, b) for i in range(steps) for b in range(B)]
    worst, ne = _check_decode_queries(spec, seed, layer, outs, sels, L, samples)
    print(f"  {case}: worst max-rel {worst:.3g}; top-k exact {ne} of {len(samples)}")
