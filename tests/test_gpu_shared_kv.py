"""Cross-layer KV sharing (V4.1: deepseek-v41-mlx "Why this exists", the cross-layer sharing
item) through the C ABI: one owner layer with its compressors and indexer lane, and two
layers that read its caches -- one scores its own queries against the owner's index keys,
the other attends the owner's selection -- each checked against the oracle fed the owner's
rows, index keys and token latents and the layer's own q, qi, w and sinks (needs a gfx950
GPU)."""
import pytest
import torch

import oracle
import synth.csa as SC
from sparse_attention_dsv4_amd.layer import CsaLayer, LayerSpec, SharedCsaLayer
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu

SMALL = LayerSpec(ratio=4, heads=8, dim=64, rope_dim=16, window=16, index_heads=4, index_dim=32,
                  topk=16)
V4 = LayerSpec(ratio=4)


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _tokens(spec, seed, t, S, B, kv=None, squeeze=False):
    tok = SC.batch_token_inputs(spec, seed, [t] * B, S, device="cuda")
    if squeeze:
        tok = {k: v[:, 0].contiguous() for k, v in tok.items()}
    if kv is not None:
        tok["kv"] = kv                     # the owner's token latents
    return tok


def _run(spec, seeds, B, chunks, n_dec):
    """Owner, an index-source layer ("own") and a layer on the owner's selection ("owner"),
    through chunked prefill then decode; returns the owner and every output and selection."""
    so, sa, sb = seeds
    T = sum(chunks) + n_dec
    mc = max(chunks)
    owner = CsaLayer(spec, B, T, SC.layer_params(spec, so, device="cuda"), device="cuda", max_chunk=mc)
    la = SharedCsaLayer(spec, owner, SC.layer_params(spec, sa, device="cuda"), index="own", max_chunk=mc)
    lb = SharedCsaLayer(spec, owner, SC.layer_params(spec, sb, device="cuda"), index="owner", max_chunk=mc)
    outs = {n: torch.zeros(B, T, spec.heads, spec.dim, dtype=spec.dtype) for n in "oab"}
    sels = {n: torch.full((B, T, spec.topk), -2, dtype=torch.int32) for n in "oa"}
    t = 0
    for S in chunks:
        to = _tokens(spec, so, t, S, B)
        so_ = torch.empty(B, S, spec.topk, dtype=torch.int32, device="cuda")
        sa_ = torch.empty_like(so_)
        outs["o"][:, t:t + S] = owner.prefill(to, sel_out=so_).cpu()
        outs["a"][:, t:t + S] = la.prefill(_tokens(spec, sa, t, S, B, kv=to["kv"]), sel_out=sa_).cpu()
        outs["b"][:, t:t + S] = lb.prefill(_tokens(spec, sb, t, S, B, kv=to["kv"]), sel=so_).cpu()
        sels["o"][:, t:t + S], sels["a"][:, t:t + S] = so_.cpu(), sa_.cpu()
        t += S
    for _ in range(n_dec):
        to = _tokens(spec, so, t, 1, B, squeeze=True)
        so_ = torch.empty(B, 1, spec.topk, dtype=torch.int32, device="cuda")
        sa_ = torch.empty_like(so_)
        outs["o"][:, t] = owner.decode(to, sel_out=so_).cpu()
        outs["a"][:, t] = la.decode(_tokens(spec, sa, t, 1, B, kv=to["kv"], squeeze=True), sel_out=sa_).cpu()
        outs["b"][:, t] = lb.decode(_tokens(spec, sb, t, 1, B, kv=to["kv"], squeeze=True), sel=so_[:, 0]).cpu()
        sels["o"][:, t], sels["a"][:, t] = so_[:, 0].cpu(), sa_[:, 0].cpu()
        t += 1
    torch.cuda.synchronize()
    return owner, outs, sels


def _check(spec, seeds, owner, outs, sels, b, positions):
    so, sa, sb = seeds
    rows = G.f64(owner.rows[b].cpu())
    rows_i = G.f64(owner.rows_i[b].cpu())
    worst, n_exact = 0.0, 0
    for p in positions:
        nv = oracle.visible_rows(p, spec.ratio)
        t0 = max(0, p - spec.window + 1)
        kv = G.f64(SC.token_inputs(spec, so, b, t0, p + 1, fields=["kv"])["kv"])
        for name, seed in (("a", sa), ("b", sb)):
            tk = {k: G.f64(v) for k, v in SC.token_inputs(spec, seed, b, p, p + 1, fields=["q", "qi", "w"]).items()}
            if name == "a":
                sc = oracle.index_scores(tk["qi"], tk["w"], rows_i[:nv])
                ref_sel = oracle.select_topk(sc, [p], ratio=spec.ratio, k=spec.topk)
                got = sels["a"][b, p:p + 1].numpy()
                ne, nb, nbad, bad = G.topk_band_ok(got, ref_sel, sc, [p], spec)
                assert nbad == 0, f"layer a, sequence {b}, p {p}: top-k differs outside the band: {bad}"
                n_exact += ne
                sel = got
            else:
                sel = sels["o"][b, p:p + 1].numpy()
            sinks = G.f64(SC.layer_params(spec, seed)["sinks"])
            ref = oracle.csa_attention(tk["q"], kv, rows[:nv], sel, [p], window=spec.window,
                                       ratio=spec.ratio, sinks=sinks, scale=spec.scale, store="bf16",
                                       kv_offset=t0)
            mr = G.max_rel_rows(G.f64(outs[name][b, p]), ref[0]).max()
            worst = max(worst, mr)
            assert mr <= 2e-2, f"layer {name}, sequence {b}, p {p}: max-rel {mr:.3g}"
    return worst, n_exact


@pytest.mark.parametrize("shape", ["small", "v4"])
def test_shared_kv_layers_match_oracle(shape):
    """Small shape (generic kernels; 55 rows, top-16: sparse from p = 67 on) and the V4 shape
    (MFMA kernels; 626 rows, top-512: sparse from p = 2051 on); ragged prefill chunks, then
    decode steps across row births."""
    if shape == "small":
        spec, B, chunks, n_dec = SMALL, 2, [70, 90, 40], 20
        pos = list(range(0, 200, 7)) + list(range(196, 220))
    else:
        spec, B, chunks, n_dec = V4, 2, [1500, 1000], 8
        pos = list(range(0, 2500, 173)) + list(range(2046, 2056)) + list(range(2500, 2508))
    seeds = (61, 62, 63)
    owner, outs, sels = _run(spec, seeds, B, chunks, n_dec)
    for b in range(B):
        worst, ne = _check(spec, seeds, owner, outs, sels, b, sorted(set(pos)))
        print(f"  sequence {b}: worst max-rel {worst:.3g}; top-k exact {ne} of {len(set(pos))}")


def test_shared_layer_rejects_mismatched_owner():
    """A sharing layer must read rows of its own width and ratio, and 'owner' selection needs
    an owner with an indexer of the same top-k."""
    owner = CsaLayer(SMALL, 1, 64, SC.layer_params(SMALL, 1, device="cuda"), device="cuda", max_chunk=64)
    other = LayerSpec(ratio=4, heads=8, dim=32, rope_dim=16, window=16, index_heads=4, index_dim=32, topk=16)
    with pytest.raises(ValueError):
        SharedCsaLayer(other, owner, SC.layer_params(other, 2, device="cuda"))
    k8 = LayerSpec(ratio=4, heads=8, dim=64, rope_dim=16, window=16, index_heads=4, index_dim=32, topk=8)
    with pytest.raises(ValueError):
        SharedCsaLayer(k8, owner, SC.layer_params(k8, 2, device="cuda"), index="owner")
    with pytest.raises(ValueError):
        SharedCsaLayer(SMALL, owner, SC.layer_params(SMALL, 2, device="cuda"), index="bogus")
    lb = SharedCsaLayer(SMALL, owner, SC.layer_params(SMALL, 3, device="cuda"), index="owner")
    to = _tokens(SMALL, 1, 0, 8, 1)
    owner.prefill(to)
    with pytest.raises(ValueError):
        lb.prefill(_tokens(SMALL, 3, 0, 8, 1, kv=to["kv"]))      # no owner selection given
