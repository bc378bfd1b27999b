"""Indexer top-k through the C ABI at row counts that reach every selection kernel (keys in
registers up to 2048 / 4096 / 8192 / 16,384 / 32,768 / 69,632 rows, in memory beyond), and with massive exact ties
(needs a gfx950 GPU).

The indexer rows are drawn directly (the index call takes them as input), so the oracle only
scores and selects: fp32 scores, the k largest, ties to the lower row, ascending output.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_dsv4_amd as K
from tests import gpu_harness as G
from sparse_attention_dsv4_amd.layer import LayerSpec

pytestmark = pytest.mark.gpu

SPEC = LayerSpec(ratio=4)


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _run(rows_i, qi, w, positions, n_rows, spec=SPEC):
    """rows_i [B, cap, di] bf16, qi [B, S, Hi, di] bf16, w [B, S, Hi] fp32 (GPU tensors)."""
    B, S = qi.shape[0], qi.shape[1]
    cfg = spec.index_cfg()
    sel = torch.full((B, S, spec.topk), -2, dtype=torch.int32, device="cuda")
    nb = K.dsv4_index_workspace_bytes(cfg, B, S, max(n_rows))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    K.dsv4_index_topk(cfg, qi, w, rows_i, n_rows, [p[0] for p in positions], sel, ws)
    torch.cuda.synchronize()
    return sel.cpu().numpy()


def _check(rows_i, qi, w, positions, sel, exact, spec=SPEC):
    for b in range(qi.shape[0]):
        P = positions[b]
        rows = G.f64(rows_i[b])
        scores = oracle.index_scores(G.f64(qi[b]), G.f64(w[b]), rows)
        ref = oracle.select_topk(scores, P, ratio=spec.ratio, k=spec.topk)
        if exact:
            assert np.array_equal(sel[b], ref), f"sequence {b}: selection differs"
        else:
            ne, nb, nbad, bad = G.topk_band_ok(sel[b], ref, scores, P, spec)
            print(f"  seq {b}: exact {ne}, in band {nb}")
            assert nbad == 0, bad[:4]


@pytest.mark.parametrize("queries", ["few", "many"])
@pytest.mark.parametrize("n_vis", [600, 2048, 2049, 4096, 5000, 8192, 12000,
                                   16384, 16684, 20001, 32768, 33001, 65600, 69632, 69633])
def test_topk_large_lanes(n_vis, queries):
    """Few queries (2 sequences x 3) from 4096 rows on take the fused decode indexer (each
    scoring workgroup passes on its m best, m from 128 down to 64 here, then one merge);
    many (65 in one sequence) take one workgroup per query.  Up to 16,384 rows the keys per
    thread follow the row count (4, 8, 16 or 32: the counts below reach each and its edge)."""
    B, S = (2, 3) if queries == "few" else (1, 65)
    cap = n_vis + 8
    g = 11 + n_vis
    rows_i = synth.normal((B, cap, SPEC.index_dim), seed=g, stream="rows_i", dtype=torch.bfloat16,
                          device="cuda")
    qi = synth.normal((B, S, SPEC.index_heads, SPEC.index_dim), seed=g, stream="qi",
                      dtype=torch.bfloat16, device="cuda")
    w = synth.normal((B, S, SPEC.index_heads), seed=g, stream="w", device="cuda")
    # consecutive queries; the last one of sequence 0 sees exactly n_vis rows
    positions = [[4 * n_vis - S - b + i for i in range(S)] for b in range(B)]
    n_rows = [min(cap, (positions[b][-1] + 1) // 4) for b in range(B)]
    sel = _run(rows_i, qi, w, positions, n_rows)
    _check(rows_i, qi, w, positions, sel, exact=False)


@pytest.mark.parametrize("n_vis,S", [(2000, 2), (4000, 2), (7000, 40), (12000, 2), (30000, 2),
                                     (80000, 2), (30000, 40), (60000, 40), (80000, 40)])
def test_topk_exact_ties_take_lower_rows(n_vis, S):
    """Rows repeat with period 7, so the scores take 7 values and the k-th score sits inside
    a block of ~1/7 of the rows: the selection must take the lowest rows of that block.  The
    row counts and query counts (4 or 80 per call) reach each selection kernel, split or not."""
    B = 2
    cap = n_vis
    base = synth.normal((7, SPEC.index_dim), seed=3, stream="base", dtype=torch.bfloat16,
                        device="cuda")
    idx = torch.arange(cap, device="cuda") % 7
    rows_i = base[idx][None].repeat(B, 1, 1).contiguous()
    qi = synth.normal((B, S, SPEC.index_heads, SPEC.index_dim), seed=4, stream="qi",
                      dtype=torch.bfloat16, device="cuda")
    w = synth.normal((B, S, SPEC.index_heads), seed=4, stream="w", device="cuda")
    positions = [[4 * n_vis - S + i for i in range(S)] for _ in range(B)]
    n_rows = [cap] * B
    sel = _run(rows_i, qi, w, positions, n_rows)
    _check(rows_i, qi, w, positions, sel, exact=True)


@pytest.mark.parametrize("queries", ["few", "many"])
@pytest.mark.parametrize("n_vis", [1500, 3000, 20001, 70001])
def test_topk_1024_pro_shape(n_vis, queries):
    """V4-Pro keeps the top-1024 (the indexer shape otherwise as Flash): a selection longer
    than the rows of the smaller kernels' first pass, the split selection with 1024
    candidates per chunk (20,001 rows, few queries) and the in-memory kernel (70,001)."""
    spec = LayerSpec(ratio=4, topk=1024)
    B, S = (2, 3) if queries == "few" else (1, 65)
    cap = n_vis + 8
    g = 41 + n_vis
    rows_i = synth.normal((B, cap, spec.index_dim), seed=g, stream="rows_i", dtype=torch.bfloat16,
                          device="cuda")
    qi = synth.normal((B, S, spec.index_heads, spec.index_dim), seed=g, stream="qi",
                      dtype=torch.bfloat16, device="cuda")
    w = synth.normal((B, S, spec.index_heads), seed=g, stream="w", device="cuda")
    positions = [[4 * n_vis - S - b + i for i in range(S)] for b in range(B)]
    n_rows = [min(cap, (positions[b][-1] + 1) // 4) for b in range(B)]
    sel = _run(rows_i, qi, w, positions, n_rows, spec)
    _check(rows_i, qi, w, positions, sel, exact=False, spec=spec)


@pytest.mark.parametrize("n_vis,lo,cnt", [(65600, 30000, 700), (20001, 0, 600), (16384, 15584, 800)])
def test_topk_clustered_rows(n_vis, lo, cnt):
    """A contiguous run of rows scores far above the rest (those index keys scaled by 4, exact
    in bf16), so one scoring workgroup of the fused decode indexer holds more of the k best
    than it passes on: the merge must notice (a workgroup's cutoff reaches the k-th candidate
    key) and select from every score key instead; the result is the oracle's either way."""
    B, S = 2, 1
    cap = n_vis + 8
    g = 71 + n_vis
    rows_i = synth.normal((B, cap, SPEC.index_dim), seed=g, stream="rows_i", dtype=torch.bfloat16,
                          device="cuda")
    rows_i[:, lo:lo + cnt] *= 4
    qi = synth.normal((B, S, SPEC.index_heads, SPEC.index_dim), seed=g, stream="qi",
                      dtype=torch.bfloat16, device="cuda")
    w = synth.normal((B, S, SPEC.index_heads), seed=g, stream="w", device="cuda").abs()
    positions = [[4 * n_vis - 1 - b] for b in range(B)]
    n_rows = [min(cap, (positions[b][-1] + 1) // 4) for b in range(B)]
    sel = _run(rows_i, qi, w, positions, n_rows)
    _check(rows_i, qi, w, positions, sel, exact=False)
    inside = ((sel >= lo) & (sel < lo + cnt)).sum(axis=-1)
    assert (inside > 200).all(), inside                 # the run does hold much of the top-k


def test_topk_mixed_dense_and_sparse_decode():
    """One decode call over sequences at very different lengths: one still dense (fewer
    visible rows than k), the others sparse at 40,000 and 65,000 rows."""
    B, S = 3, 1
    n_vis = [300, 40000, 65000]
    cap = max(n_vis) + 8
    rows_i = synth.normal((B, cap, SPEC.index_dim), seed=5, stream="rows_i", dtype=torch.bfloat16,
                          device="cuda")
    qi = synth.normal((B, S, SPEC.index_heads, SPEC.index_dim), seed=5, stream="qi",
                      dtype=torch.bfloat16, device="cuda")
    w = synth.normal((B, S, SPEC.index_heads), seed=5, stream="w", device="cuda")
    positions = [[4 * n + 2] for n in n_vis]
    n_rows = [n for n in n_vis]
    sel = _run(rows_i, qi, w, positions, n_rows)
    assert list(sel[0, 0, :300]) == list(range(300)) and (sel[0, 0, 300:] == -1).all()
    _check(rows_i, qi, w, positions, sel, exact=False)


@pytest.mark.parametrize("queries", ["few", "many"])
@pytest.mark.parametrize("n_vis", [2048, 16384, 30000, 70001])
@pytest.mark.parametrize("mode", ["equal", "quantised"])
def test_topk_degenerate_scores(mode, n_vis, queries):
    """Scores both sides compute exactly, with the k-th inside a block of equal scores.
    'equal': a zero query, every score 0, so the k lowest rows are the selection.
    'quantised': one head whose query is the unit vector on dim 0 (weight 1, the other
    heads' weights 0), so a row's score is its first element, one of 128 bf16 values in
    [1, 2) (a multiple of 2^-7, repeating with row index): each value is shared by many
    rows, the selection's digit passes narrow down to one value and split its tie.  Row
    counts and query counts reach each selection kernel (registers, fused, in memory)."""
    B, S = (2, 3) if queries == "few" else (1, 65)
    cap = n_vis + 8
    g = 91 + n_vis
    rows_i = synth.normal((B, cap, SPEC.index_dim), seed=g, stream="rows_i", dtype=torch.bfloat16,
                          device="cuda")
    qi = torch.zeros((B, S, SPEC.index_heads, SPEC.index_dim), dtype=torch.bfloat16, device="cuda")
    w = synth.normal((B, S, SPEC.index_heads), seed=g, stream="w", device="cuda")
    if mode == "quantised":
        j = torch.arange(cap, device="cuda")
        rows_i[:, :, 0] = (1.0 + ((j * 37) % 128).float() / 128.0).to(torch.bfloat16)
        qi[:, :, 0, 0] = 1.0
        w.zero_()
        w[:, :, 0] = 1.0
    positions = [[4 * n_vis - S - b + i for i in range(S)] for b in range(B)]
    n_rows = [min(cap, (positions[b][-1] + 1) // 4) for b in range(B)]
    sel = _run(rows_i, qi, w, positions, n_rows)
    _check(rows_i, qi, w, positions, sel, exact=True)
    if mode == "equal":
        assert (sel == np.arange(SPEC.topk, dtype=np.int32)).all()
