"""Helpers of the GPU parity tests: run the HIP path on seeded inputs, run the oracle on the
same inputs, and compare with the tolerances the tests state.

Comparison bars (from the layer's stated targets; see each function):
  * attention outputs: max-rel per (token, head) row <= 2e-2 in bf16, <= 1e-5 in fp32,
    where max-rel = max|gpu - ref| / max|ref| over the row's latent dims;
  * top-k sets: exact, except rows whose oracle score lies within 1e-5 relative of the
    k-th score (with a floor of 1e-3 * max|score| when the k-th score is ~0);
  * compressed rows: fp32 max-rel <= 1e-5; bf16 every element within 2 ulp of the oracle's,
    where on the rotated dims the ulp is taken of the pair's norm (the rotation preserves
    it), or within 2^-10 of the row's largest magnitude: a pooled value near zero is a sum
    of cancelling fp32 terms and carries their rounding, not its own ulp.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth.csa as SC
from sparse_attention_dsv4_amd.layer import CsaLayer, LayerSpec


def store_of(spec: LayerSpec) -> str:
    return "bf16" if spec.dtype == torch.bfloat16 else "f32"


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


# ------------------------------------------------------------------ the HIP path
def run_gpu(spec: LayerSpec, seed: int, batch: int, chunks, n_decode: int, device="cuda"):
    """Prefill ``chunks`` (token counts) then ``n_decode`` decode steps, for every sequence.

    Returns a dict: out [B, T, H, D] (cpu), sel [B, T, k] int32 (cpu, when indexed),
    rows [B, T//r, D], rows_i [B, T//r, di] (cpu), and the layer."""
    T = sum(chunks) + n_decode
    params = SC.layer_params(spec, seed, device=device)
    layer = CsaLayer(spec, batch, T, params, device=device, max_chunk=max(list(chunks) + [1]))
    out = torch.empty(batch, T, spec.heads, spec.dim, dtype=spec.dtype)
    sel = torch.full((batch, T, spec.topk), -2, dtype=torch.int32) if spec.has_indexer else None
    t = 0
    for S in chunks:
        tok = SC.batch_token_inputs(spec, seed, [t] * batch, S, device=device)
        s_buf = torch.empty(batch, S, spec.topk, dtype=torch.int32, device=device) \
            if spec.has_indexer else None
        o = layer.prefill(tok, sel_out=s_buf)
        out[:, t:t + S] = o.cpu()
        if sel is not None:
            sel[:, t:t + S] = s_buf.cpu()
        t += S
    for _ in range(n_decode):
        tok = SC.batch_token_inputs(spec, seed, [t] * batch, 1, device=device)
        tok = {k: v[:, 0].contiguous() for k, v in tok.items()}
        s_buf = torch.empty(batch, 1, spec.topk, dtype=torch.int32, device=device) \
            if spec.has_indexer else None
        o = layer.decode(tok, sel_out=s_buf)
        out[:, t] = o.cpu()
        if sel is not None:
            sel[:, t] = s_buf[:, 0].cpu()
        t += 1
    torch.cuda.synchronize()
    res = {"out": out, "sel": sel, "layer": layer, "T": T}
    if spec.has_rows:
        n = T // spec.ratio
        res["rows"] = layer.rows[:, :n].cpu()
        if spec.has_indexer:
            res["rows_i"] = layer.rows_i[:, :n].cpu()
    return res


# ------------------------------------------------------------------ the oracle
def oracle_inputs(spec: LayerSpec, seed: int, b: int, T: int):
    tok = SC.token_inputs(spec, seed, b, 0, T)
    par = SC.layer_params(spec, seed)
    return ({k: f64(v) for k, v in tok.items()}, {k: f64(v) for k, v in par.items()})


def oracle_rows(spec, tok, par, index_lane=False):
    if index_lane:
        return oracle.compressor_rows(tok["ai"], tok["gi"], par["ape_i"], par["norm_w_i"],
                                      par["inv_freq"], ratio=spec.ratio, overlap=spec.is_overlap,
                                      eps=spec.eps, store=store_of(spec))
    return oracle.compressor_rows(tok["a"], tok["g"], par["ape"], par["norm_w"], par["inv_freq"],
                                  ratio=spec.ratio, overlap=spec.is_overlap, eps=spec.eps,
                                  store=store_of(spec))


def oracle_scores(spec, tok, rows_i, positions):
    P = np.asarray(positions)
    return oracle.index_scores(tok["qi"][P], tok["w"][P], rows_i)


def oracle_select(spec, scores, positions):
    return oracle.select_topk(scores, positions, ratio=spec.ratio, k=spec.topk)


def oracle_attention(spec, tok, par, rows, sel, positions):
    return oracle.csa_attention(tok["q"][np.asarray(positions)], tok["kv"], rows, sel, positions,
                                window=spec.window, ratio=spec.ratio, sinks=par["sinks"],
                                scale=spec.scale, store=store_of(spec))


# ------------------------------------------------------------------ comparisons
def max_rel_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per row over the last axis: max|a - b| / max|b|."""
    num = np.abs(a - b).max(axis=-1)
    den = np.abs(b).max(axis=-1)
    return num / np.maximum(den, 1e-30)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def assert_rows_match(gpu: np.ndarray, ref: np.ndarray, store: str, what: str, rope_dim: int):
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if store == "f32":
        mr = max_rel_rows(gpu, ref)
        assert mr.max() <= 1e-5, f"{what}: fp32 max-rel {mr.max():.3g}"
    else:
        mag = np.abs(ref).copy()
        if rope_dim:
            D = ref.shape[-1]
            pair = np.sqrt(ref[..., D - rope_dim::2] ** 2 + ref[..., D - rope_dim + 1::2] ** 2)
            mag[..., D - rope_dim::2] = pair
            mag[..., D - rope_dim + 1::2] = pair
        diff = np.abs(gpu - ref)
        ulps = diff / bf16_ulp(mag)
        floor = 2.0 ** -10 * np.abs(ref).max(axis=-1, keepdims=True)
        bad = (ulps > 2.0) & (diff > floor)
        w = np.unravel_index(np.argmax(ulps), ulps.shape)
        worst = (f"worst at {tuple(int(x) for x in w)}: gpu {gpu[w]:.6g} ref {ref[w]:.6g} "
                 f"({ulps[w]:.1f} ulp, row max {np.abs(ref[w[:-1]]).max():.3g})")
        assert not bad.any(), f"{what}: {bad.sum()} elements beyond the bar; {worst}"
        n1 = int((ulps > 0.5).sum())
        return f"{n1}/{ulps.size} elements differ; {worst}"
    return float(np.abs(gpu - ref).max())


def topk_band_ok(sel_gpu: np.ndarray, sel_ref: np.ndarray, scores: np.ndarray, positions,
                 spec: LayerSpec):
    """Check one batch of queries.  Returns (n_exact, n_band, n_bad, bad_queries)."""
    n_exact = n_band = n_bad = 0
    bad = []
    for i, p in enumerate(positions):
        nv = min(oracle.visible_rows(p, spec.ratio), scores.shape[1])
        g = sel_gpu[i]
        chosen = [int(x) for x in g if x >= 0]
        # validity of the GPU row: ascending, unique, visible, right count, -1 padded
        valid = (chosen == sorted(set(chosen)) and len(chosen) == min(spec.topk, nv)
                 and all(0 <= j < nv for j in chosen)
                 and all(int(x) == -1 for x in g[len(chosen):]))
        if not valid:
            n_bad += 1
            bad.append((p, "invalid"))
            continue
        if np.array_equal(g, sel_ref[i]):
            n_exact += 1
            continue
        s = scores[i, :nv].astype(np.float64)
        ref = [int(x) for x in sel_ref[i] if x >= 0]
        sk = min(s[j] for j in ref)                     # the k-th score
        tol = 1e-5 * max(abs(sk), 1e-3 * np.abs(s).max())
        diff = set(chosen) ^ set(ref)
        if all(abs(s[j] - sk) <= tol for j in diff):
            n_band += 1
        else:
            n_bad += 1
            bad.append((p, sorted(diff)[:8]))
    return n_exact, n_band, n_bad, bad


def check_against_oracle(spec: LayerSpec, tok: dict, par: dict, got: dict, b: int, positions,
                         end_to_end: bool = False, label: str = ""):
    """Compare sequence ``b`` of a GPU run (``got``: rows, rows_i [B, n, .], sel [B, T, k],
    out [B, T, H, D], cpu tensors) with the oracle run on the inputs ``tok`` / ``par`` (numpy,
    indexed by absolute position) at the query ``positions``.

    Stage-isolated (default): the rows are compared with the oracle's, then the oracle scores
    and selects over the GPU's index rows and attends over the GPU's rows with the GPU's
    selection, so every query's attention is comparable.  End to end: the oracle runs on its
    own rows and selection throughout; queries whose selection differs from the GPU's (only
    inside the top-k band) are left out of the attention comparison."""
    store = store_of(spec)
    rows = sel = None
    report = {}
    P = np.asarray(positions)
    if spec.has_rows:
        rows_ref = oracle_rows(spec, tok, par)
        rows = f64(got["rows"][b])
        report["rows_maxabs"] = assert_rows_match(rows, rows_ref, store, "attention-lane rows",
                                                  spec.rope_dim)
        if end_to_end:
            rows = rows_ref
    agree = np.ones(len(positions), dtype=bool)
    if spec.has_indexer:
        rows_i_ref = oracle_rows(spec, tok, par, index_lane=True)
        rows_i = f64(got["rows_i"][b])
        report["rows_i_maxabs"] = assert_rows_match(rows_i, rows_i_ref, store, "indexer-lane rows",
                                                    spec.rope_dim)
        if end_to_end:
            rows_i = rows_i_ref
        scores = oracle_scores(spec, tok, rows_i, positions)
        sel_ref = oracle_select(spec, scores, positions)
        sel_gpu = got["sel"][b].numpy()[P]
        ne, nb, nbad, bad = topk_band_ok(sel_gpu, sel_ref, scores, positions, spec)
        report.update(topk_exact=ne, topk_band=nb)
        assert nbad == 0, f"top-k mismatches outside the band: {bad[:5]}"
        if end_to_end:
            sel = sel_ref
            agree = np.array([np.array_equal(sel_gpu[i], sel_ref[i]) for i in range(len(positions))])
        else:
            sel = sel_gpu
    ref = oracle_attention(spec, tok, par, rows, sel, positions)
    gpu = f64(got["out"][b])[P]
    mr = max_rel_rows(gpu, ref)[agree]
    bar = 1e-5 if store == "f32" else 2e-2
    report["attn_maxrel"] = float(mr.max()) if mr.size else 0.0
    report["attn_compared"] = f"{int(agree.sum())}/{len(positions)}"
    assert mr.size == 0 or mr.max() <= bar, f"attention max-rel {mr.max():.3g} > {bar}"
    print(f"  {label}seq {b}: {report}", flush=True)
    return report

