"""Decode steps with the compressor frontier stores folded into the attention launch
(dsv4_csa_attn_decode_store) against the separate calls (dsv4_compress_step per lane, then
dsv4_csa_attn_decode), bit for bit, across steps that complete rows (which take the separate
calls) and steps that do not (needs a gfx950 GPU).  The bf16 64-head layers take the folded
MFMA kernel; the small fp32 layer takes the frontier-store kernel before the generic
attention."""
import pytest
import torch

import synth.csa as SC
from sparse_attention_dsv4_amd.layer import CsaLayer, LayerSpec

pytestmark = pytest.mark.gpu

SMALL = LayerSpec(ratio=4, heads=4, dim=64, rope_dim=16, window=16, index_heads=2, index_dim=32,
                  topk=8, dtype=torch.float32)


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _buffers(layer):
    names = ["ring"] + [n for n in ("state", "rows", "state_i", "rows_i") if hasattr(layer, n)]
    return {n: getattr(layer, n) for n in names}


@pytest.mark.parametrize("spec,prefix,steps", [
    (LayerSpec(ratio=4), 1024 + 61, 11),                        # rows complete every 4th step
    (LayerSpec(ratio=128, indexer=False, topk=0), 1024 + 120, 12),   # one row completes
    (SMALL, 200 + 3, 11),
], ids=["ratio4_bf16", "ratio128_bf16", "ratio4_fp32_small"])
def test_folded_stores_equal_separate_calls(spec, prefix, steps):
    seed, B = 9, 3
    params = SC.layer_params(spec, seed, device="cuda")
    layers = [CsaLayer(spec, B, prefix + steps + 8, params, device="cuda",
                       max_chunk=prefix, fold_stores=f) for f in (True, False)]
    for layer in layers:
        for t in _buffers(layer).values():
            t.zero_()                      # never-written bytes compare equal too
    tok = SC.batch_token_inputs(spec, seed, [0] * B, prefix, device="cuda")
    for layer in layers:
        layer.prefill(tok)
    folded = 0
    for i in range(steps):
        p = prefix + i
        t = SC.batch_token_inputs(spec, seed, [p] * B, 1, device="cuda")
        t = {k: v[:, 0].contiguous() for k, v in t.items()}
        outs = [layer.decode(t) for layer in layers]
        torch.cuda.synchronize()
        folded += (p + 1) % spec.ratio != 0
        assert torch.equal(outs[0].view(torch.uint8), outs[1].view(torch.uint8)), f"step {i}: out"
        for (n, a), (_, b) in zip(_buffers(layers[0]).items(), _buffers(layers[1]).items()):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"step {i}: {n}"
    assert 0 < folded < steps                 # both kinds of step were taken
