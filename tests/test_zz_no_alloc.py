"""The allocation-free top-k entry point (dsv4_index_topk_noalloc: the library's fixed
per-GPU scratch instead of a caller workspace) against the workspace entry point it shares
its kernels with: the selections must be equal, bit for bit, on two calls in a row (the
second smaller, so the scratch holds the first call's leftovers), at the small generic shape
and at the V4 shapes in decode (split selection over ~65K rows) and a short prefill.  A call
whose workspace would exceed the fixed scratch fails before any launch.  Needs a gfx950 GPU."""
import pytest
import torch

import sparse_attention_dsv4_amd as K
import synth
import synth.csa as SC
from sparse_attention_dsv4_amd.layer import LayerSpec

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _inputs(spec, seed, B, S, n_rows, pos0):
    cap = max(n_rows)
    idx = synth.normal((B, cap, spec.index_dim), seed=seed, stream="noalloc.rows", dtype=spec.dtype,
                       device="cuda")
    tok = SC.batch_token_inputs(spec, seed, pos0, S, device="cuda", fields=["qi", "w"])
    return tok["qi"], tok["w"], idx


def _both(spec, seed, B, S, n_rows, pos0):
    cfg = spec.index_cfg()
    qi, w, idx = _inputs(spec, seed, B, S, n_rows, pos0)
    ws = torch.empty(K.dsv4_index_workspace_bytes(cfg, B, S, max(n_rows)), dtype=torch.uint8,
                     device="cuda")
    ref = torch.full((B, S, spec.topk), -3, dtype=torch.int32, device="cuda")
    got = torch.full((B, S, spec.topk), -4, dtype=torch.int32, device="cuda")
    K.dsv4_index_topk(cfg, qi, w, idx, n_rows, pos0, ref, ws)
    K.dsv4_index_topk_noalloc(cfg, qi, w, idx, n_rows, pos0, got)
    torch.cuda.synchronize()
    return ref.cpu(), got.cpu()


CASES = {
    # V4 shapes: a decode call at long context (split selection), then a shorter one
    "v4_decode": (LayerSpec(ratio=4), [(4, 1, [65540] * 4, [262159] * 4),
                                       (2, 1, [3001, 2500], [12003, 9999])]),
    # V4 shapes: a short prefill over ~8K rows, then a decode call
    "v4_prefill_then_decode": (LayerSpec(ratio=4), [(1, 40, [8200], [32760]),
                                                    (3, 1, [1500, 900, 700], [5999, 3601, 2801])]),
    # generic fp32 kernels at the small shape
    "small_fp32": (LayerSpec(ratio=4, heads=4, dim=64, rope_dim=16, window=16, index_heads=2,
                             index_dim=32, topk=8, dtype=torch.float32),
                   [(3, 17, [90, 60, 75], [340, 220, 280]), (1, 5, [40], [150])]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_equals_workspace_call(name):
    spec, calls = CASES[name]
    for i, (B, S, n_rows, pos0) in enumerate(calls):
        ref, got = _both(spec, 90 + i, B, S, n_rows, pos0)
        assert (ref >= -1).all()
        assert torch.equal(ref, got), f"call {i}: {int((ref != got).sum())} entries differ"


def test_noalloc_rejects_calls_above_the_fixed_scratch():
    spec = LayerSpec(ratio=4)
    cfg = spec.index_cfg()
    B, S, n = 1, 2048, 16384
    assert K.dsv4_index_workspace_bytes(cfg, B, S, n) > K.dsv4_index_topk_noalloc_scratch_bytes()
    qi = torch.zeros(B, S, spec.index_heads, spec.index_dim, dtype=spec.dtype, device="cuda")
    w = torch.zeros(B, S, spec.index_heads, device="cuda")
    idx = torch.zeros(B, n, spec.index_dim, dtype=spec.dtype, device="cuda")
    sel = torch.full((B, S, spec.topk), -5, dtype=torch.int32, device="cuda")
    with pytest.raises(K.Dsv4Error) as e:
        K.dsv4_index_topk_noalloc(cfg, qi, w, idx, [n], [4 * n - S], sel)
    assert e.value.code == -5 and "fixed scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (sel == -5).all()                 # nothing was launched
