"""HIP-graph capture of decode steps (needs a gfx950 GPU).

Every launch of a decode step goes onto the caller's stream with its arguments fixed at
launch time and no allocation, memset or synchronisation, so a sequence of steps can be
captured once and replayed.  A replay from the same starting state must reproduce the eager
steps bit for bit (same kernels, same launch shapes, no atomics).  Each replay is preceded by
an eager restore of the state and followed by a synchronisation, and every replay is checked.
"""
import pytest
import torch

import synth.csa as SC
from sparse_attention_dsv4_amd.layer import CsaLayer, LayerSpec

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _layer_state(layer):
    names = ["ring"] + [n for n in ("state", "rows", "state_i", "rows_i") if hasattr(layer, n)]
    return {n: getattr(layer, n).clone() for n in names}


def _restore(layer, snap):
    for n, v in snap.items():
        getattr(layer, n).copy_(v)


def _bits(t):
    """Raw bit pattern: the buffers hold never-written bytes too (possibly NaN patterns, which
    compare unequal to themselves), and those must survive a replay unchanged as well."""
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("spec", [
    LayerSpec(ratio=4),                                   # both lanes, indexer, sparse attention
    LayerSpec(ratio=128, indexer=False, topk=0),          # dense compressed lane
], ids=["ratio4", "ratio128"])
def test_graph_replay_equals_eager_decode(spec):
    seed, B, prefix, steps = 5, 3, 1024 + 61, 9          # crosses ratio-4 row boundaries
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, prefix + steps + 8, params, device="cuda", max_chunk=prefix)
    tok = SC.batch_token_inputs(spec, seed, [0] * B, prefix, device="cuda")
    layer.prefill(tok)
    toks = []
    for i in range(steps):
        t = SC.batch_token_inputs(spec, seed, [prefix + i] * B, 1, device="cuda")
        toks.append({k: v[:, 0].contiguous() for k, v in t.items()})
    torch.cuda.synchronize()
    snap = _layer_state(layer)

    eager = [layer.decode(t).clone() for t in toks]
    torch.cuda.synchronize()
    eager_state = _layer_state(layer)

    _restore(layer, snap)
    layer.lengths = [prefix] * B
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = [layer.decode(t) for t in toks]
    for rep in range(3):
        _restore(layer, snap)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(steps):
            assert torch.equal(_bits(outs[i]), _bits(eager[i])), f"replay {rep}, step {i}: output differs"
        for n, v in eager_state.items():
            assert torch.equal(_bits(getattr(layer, n)), _bits(v)), f"replay {rep}: {n} differs"
