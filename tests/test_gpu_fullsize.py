"""Parity at the full sizes the benchmark times, in the same launch configuration (needs a
gfx950 GPU).

The layer is driven exactly as bench.py drives it (same seeds, prefix builder, batch, chunk
and call sequence), and sampled outputs are checked against the oracle one by one:
  * decode, ratio-128 layer, batch 8, context 65,536 (512 rows + 128-token window per query):
    sampled rows against the oracle compressor; every sequence's output of three decode steps
    against the oracle attention over the GPU's rows;
  * prefill, ratio-4 layer with the indexer, the 2048-token chunk 63,488 -> 65,536: sampled
    rows of both lanes, then for sampled queries the top-512 over ~16K visible rows (exact up
    to the 1e-5 band) and the attention output.
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


def test_fullsize_decode_64k_batch8_ratio128():
    spec = LayerSpec(ratio=128, indexer=False, topk=0)
    seed, B, L, steps = 0, 8, 65536, 3               # bench_decode's seed, batch and context
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, L + steps + 8, params, device="cuda", max_chunk=spec.window)
    bench.build_prefix(layer, spec, seed, L)
    outs = []
    for i in range(steps):
        t = SC.batch_token_inputs(spec, seed, [L + i] * B, 1, device="cuda", fields=["q", "kv", "a", "g"])
        outs.append(layer.decode({k: v[:, 0].contiguous() for k, v in t.items()}).cpu())
    torch.cuda.synchronize()
    rows = layer.rows.cpu()
    for b in (0, 5, 7):
        _check_rows(spec, seed, rows, b, [0, 1, 255, 510, 511])
    par = _params64(spec, seed)
    worst = 0.0
    for i in range(steps):
        p = L + i
        nv = oracle.visible_rows(p, spec.ratio)
        for b in range(B):
            tk = _lanes(spec, seed, b, p - spec.window + 1, p + 1, ["q", "kv"])
            ref = oracle.csa_attention(tk["q"][-1:], tk["kv"], G.f64(rows[b, :nv]), None, [p],
                                       window=spec.window, ratio=spec.ratio, sinks=par["sinks"],
                                       scale=spec.scale, store="bf16", kv_offset=p - spec.window + 1)
            mr = G.max_rel_rows(G.f64(outs[i][b]), ref[0]).max()
            worst = max(worst, mr)
            assert mr <= 2e-2, f"step {i} sequence {b}: max-rel {mr:.3g}"
    print(f"  decode outputs: worst per-head max-rel {worst:.3g} over {steps * B} queries x 64 heads")


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
