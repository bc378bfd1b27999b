"""Exact trim for speculative decode on the GPU: decode draft tokens, take some back with
CsaLayer.trim, decode other tokens.  Every output, selection and compressed row must equal,
bit for bit, those of a layer that only ever saw the committed tokens, and must match the
oracle run on the committed token stream (MTPLX PR #216, speculative-decode comment, on
taking draft tokens back without approximation; checked here where a ratio-4 row is
emitted, where a ratio-128 row completes and where the indexer starts to select).  Needs a gfx950 GPU."""
import numpy as np
import pytest
import torch

import synth.csa as SC
from sparse_attention_dsv4_amd.layer import CsaLayer, LayerSpec
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _token(spec, seed, pos, B):
    t = SC.batch_token_inputs(spec, seed, [pos] * B, 1, device="cuda")
    return {k: v[:, 0].contiguous() for k, v in t.items()}


def _bits(t):
    return t.contiguous().view(torch.uint8)


# (spec, prefix, script): ("dec", draft seed, count) decodes tokens of that seed at the next
# positions; ("trim", n) takes n back.  Seeds 1, 2, 3 stand for different drafts.
CASES = {
    # prefix 2045: the drafts cross the emission at 2047 / 2051 and the dense-to-sparse
    # threshold (more than 512 visible rows from position 2048 on)
    "ratio4_threshold": (LayerSpec(ratio=4, rollback=16), 2045,
                         [("dec", 1, 8), ("trim", 5), ("dec", 2, 2), ("trim", 4), ("dec", 3, 7)]),
    # prefix 1020: the drafts cross the ratio-128 emission at 1023; the trim lands before it
    "ratio128_boundary": (LayerSpec(ratio=128, indexer=False, topk=0, rollback=16), 1020,
                          [("dec", 1, 8), ("trim", 6), ("dec", 2, 8)]),
    # capacity exactly used: 8 of 8, across two ratio-4 windows
    "ratio4_full_room": (LayerSpec(ratio=4, rollback=8), 1030,
                         [("dec", 1, 8), ("trim", 8), ("dec", 2, 9)]),
    # the generic kernels (fp32, small shapes): a rollback deeper than the window ring's
    # 16 tokens and than two ratio-4 windows, across the top-8 threshold (36 visible rows)
    "small_fp32_generic": (LayerSpec(ratio=4, heads=4, dim=64, rope_dim=16, window=16,
                                     index_heads=2, index_dim=32, topk=8,
                                     dtype=torch.float32, rollback=20), 29,
                           [("dec", 1, 12), ("trim", 7), ("dec", 2, 3), ("trim", 8),
                            ("dec", 3, 10)]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_trim_equals_never_decoded(name):
    spec, prefix, script = CASES[name]
    B, seed = 2, 61
    params = SC.layer_params(spec, seed, device="cuda")
    cap = prefix + 64
    draft = CsaLayer(spec, B, cap, params, device="cuda", max_chunk=prefix)
    ref_spec = LayerSpec(**{**spec.__dict__, "rollback": 0})
    ref = CsaLayer(ref_spec, B, cap, params, device="cuda", max_chunk=prefix)
    tok = SC.batch_token_inputs(spec, seed, [0] * B, prefix, device="cuda")
    draft.prefill(tok)
    ref.prefill(tok)
    committed = []                                   # (seed, position) of the kept tokens
    outs = {}                                        # position -> draft's output, last decode
    for op in script:
        if op[0] == "trim":
            assert op[1] <= len(committed), "the scripts take back decoded tokens only"
            draft.trim(op[1])
            del committed[len(committed) - op[1]:]
            continue
        _, s, n = op
        for _ in range(n):
            p = draft.lengths[0]
            sel = torch.empty(B, 1, spec.topk, dtype=torch.int32, device="cuda") \
                if spec.has_indexer else None
            o = draft.decode(_token(spec, seed + 100 * s, p, B), sel_out=sel)
            outs[p] = (o.clone(), sel.clone() if sel is not None else None)
            committed.append((s, p))
    # the reference decodes only the committed tokens
    for s, p in committed:
        sel = torch.empty(B, 1, spec.topk, dtype=torch.int32, device="cuda") \
            if spec.has_indexer else None
        o = ref.decode(_token(spec, seed + 100 * s, p, B), sel_out=sel)
        do, dsel = outs[p]
        assert torch.equal(_bits(o), _bits(do)), f"position {p}: output differs"
        if sel is not None:
            assert torch.equal(sel, dsel), f"position {p}: selection differs"
    torch.cuda.synchronize()
    assert draft.lengths == ref.lengths
    n = draft.lengths[0] // spec.ratio
    for lane in ("rows", "rows_i"):
        if hasattr(ref, lane):
            a, b = getattr(draft, lane)[:, :n], getattr(ref, lane)[:, :n]
            assert torch.equal(_bits(a), _bits(b)), f"{lane} differ"
    # the trimmed layer against the oracle on the committed stream: prefix tokens, then the
    # kept draft token at every decoded position
    T = draft.lengths[0]
    positions = [p for _, p in committed]
    got = {"out": torch.zeros(B, T, spec.heads, spec.dim, dtype=spec.dtype),
           "sel": torch.full((B, T, max(1, spec.topk)), -2, dtype=torch.int32)}
    for p in positions:
        got["out"][:, p] = outs[p][0].cpu()
        if spec.has_indexer:
            got["sel"][:, p] = outs[p][1][:, 0].cpu()
    if spec.has_rows:
        got["rows"] = draft.rows[:, :n].cpu()
        if spec.has_indexer:
            got["rows_i"] = draft.rows_i[:, :n].cpu()
    par = {k: G.f64(v) for k, v in SC.layer_params(spec, seed).items()}
    for b in range(B):
        parts = [SC.token_inputs(spec, seed, b, 0, prefix, device="cuda")]
        parts += [SC.token_inputs(spec, seed + 100 * s_, b, p, p + 1, device="cuda")
                  for s_, p in committed]
        tok = {k: np.concatenate([G.f64(x[k]) for x in parts]) for k in parts[0]}
        G.check_against_oracle(spec, tok, par, got, b, positions, label="trimmed ")
        if spec.dtype == torch.float32:
            G.check_against_oracle(spec, tok, par, got, b, positions, end_to_end=True,
                                   label="trimmed, end to end ")


def test_trim_beyond_room_raises_on_a_live_layer():
    spec = LayerSpec(ratio=4, rollback=4)
    B, seed = 1, 62
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, 256, params, device="cuda", max_chunk=100)
    layer.prefill(SC.batch_token_inputs(spec, seed, [0], 100, device="cuda"))
    for i in range(3):
        layer.decode(_token(spec, seed, 100 + i, B))
    with pytest.raises(ValueError):
        layer.trim(5)
    assert layer.lengths == [103]
    layer.trim(4)
    assert layer.lengths == [99]
