"""Parity of the HIP path against the oracle, through the C ABI (needs a gfx950 GPU).

Stage-isolated checks feed each oracle stage the GPU's own upstream outputs (rows, then the
selection), so an independent bf16 rounding upstream cannot move a later comparison; the
fp32 tiny layer is also checked end to end from the raw inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth.csa as SC
from sparse_attention_dsv4_amd.layer import LayerSpec
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu

TINY = LayerSpec(ratio=4, heads=4, dim=64, rope_dim=16, window=16, index_heads=2, index_dim=32,
                 topk=8, dtype=torch.float32)
SMALL_BF16 = LayerSpec(ratio=4, heads=8, dim=64, rope_dim=16, window=16, index_heads=4,
                       index_dim=32, topk=16)


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _check_layer(spec, res, b, positions, seed, end_to_end=False):
    """Sequence b at the given query positions against the oracle on the same seeded inputs
    (stage-isolated unless ``end_to_end``; see gpu_harness.check_against_oracle)."""
    tok, par = G.oracle_inputs(spec, seed, b, res["T"])
    return G.check_against_oracle(spec, tok, par, res, b, positions, end_to_end=end_to_end)


def test_tiny_fp32_prefill_end_to_end():
    """256-token fp32 layer (4 heads, latent 64, window 16, ratio-4 overlap, indexer 2x32,
    top-8), one-shot prefill; every query against the oracle from the raw inputs."""
    res = G.run_gpu(TINY, 0, 1, [256], 0)
    _check_layer(TINY, res, 0, list(range(256)), 0, end_to_end=True)
    _check_layer(TINY, res, 0, list(range(256)), 0)


def test_tiny_fp32_decode_equals_prefill():
    """Prefill 192 then 64 decode steps equals the one-shot 256-token prefill bit for bit,
    and chunked prefills (1, 3, 7, 16, 64 ...; not aligned to r or W) equal it too."""
    one = G.run_gpu(TINY, 0, 1, [256], 0)
    dec = G.run_gpu(TINY, 0, 1, [192], 64)
    chk = G.run_gpu(TINY, 0, 1, [1, 3, 7, 16, 64, 5, 33, 2, 61], 64)
    for other in (dec, chk):
        assert torch.equal(other["rows"], one["rows"])
        assert torch.equal(other["rows_i"], one["rows_i"])
        assert torch.equal(other["sel"], one["sel"])
        assert torch.equal(other["out"], one["out"])
    _check_layer(TINY, dec, 0, list(range(192, 256)), 0, end_to_end=True)


def test_tiny_fp32_config_prefill_256_then_64_decode():
    """The tiny fp32 configuration as stated: prefill of 256 tokens, then 64 decode steps;
    every position against the oracle from the raw inputs."""
    res = G.run_gpu(TINY, 0, 1, [256], 64)
    _check_layer(TINY, res, 0, list(range(320)), 0, end_to_end=True)


def test_tiny_config_literal_shapes():
    """The tiny fp32 configuration with its stated shapes and recipe: token states
    x ~ N(0, 1) [320, 64] and weights N(0, 1)/sqrt(64) projecting q (64 -> 4 x 64) and kv
    (64 -> 64); the overlapping compressor (window 8, stride 4) whose kv and gate lanes are each
    ONE 64 -> 64 projection feeding both halves of the 128-wide lane, with its (8, 64) APE laid
    out as ape[s, h*64 + c] = APE8[h*4 + s, c] (the previous window's 4 slots take APE8 rows
    0..3, the row's own window rows 4..7); the indexer's qi (64 -> 2 x 32), head weights
    (64 -> 2) and lanes (64 -> 32 into both halves) with an (8, 32) APE; q, kv and qi turned by
    RoPE at their positions inside the library (rope=True).  Prefill of 256 tokens, then 64
    decode steps; every position against the oracle end to end (the oracle rotates q, kv and
    qi itself)."""
    import synth
    T0, ND = 256, 64
    T = T0 + ND

    def nrm(shape, name, scale=1.0):
        return synth.normal(shape, seed=0, stream=f"tiny.{name}", scale=scale, dtype=torch.float64)

    x = nrm((T, 64), "x")

    def proj(out, name):
        return (x @ nrm((out, 64), name, 64 ** -0.5).T).float()

    def both_halves(t):
        return torch.cat([t, t], dim=-1).contiguous()

    def ape_of(a8):                      # [8, D] -> [4, 2D]
        return torch.cat([a8[0:4], a8[4:8]], dim=1).float().contiguous()

    tok = {"q": proj(256, "wq").view(T, 4, 64), "kv": proj(64, "wkv"),
           "a": both_halves(proj(64, "wa")), "g": both_halves(proj(64, "wg")),
           "qi": proj(64, "wqi").view(T, 2, 32), "w": proj(2, "ww"),
           "ai": both_halves(proj(32, "wai")), "gi": both_halves(proj(32, "wgi"))}
    params = {"ape": ape_of(nrm((8, 64), "ape8")), "ape_i": ape_of(nrm((8, 32), "ape8_i")),
              "norm_w": nrm((64,), "gamma").float(), "norm_w_i": nrm((32,), "gamma_i").float(),
              "sinks": nrm((4,), "sinks").float(), "inv_freq": SC.inv_freq(16)}
    from sparse_attention_dsv4_amd.layer import CsaLayer
    layer = CsaLayer(TINY, 1, T, {k: v.cuda() for k, v in params.items()}, device="cuda",
                     max_chunk=T0)
    out = torch.empty(1, T, 4, 64)
    sel = torch.empty(1, T, TINY.topk, dtype=torch.int32)
    s_buf = torch.empty(1, T0, TINY.topk, dtype=torch.int32, device="cuda")
    pre = {k: v[:T0][None].cuda().contiguous() for k, v in tok.items()}
    out[:, :T0] = layer.prefill(pre, sel_out=s_buf, rope=True).cpu()
    sel[:, :T0] = s_buf.cpu()
    for t in range(T0, T):
        s1 = torch.empty(1, 1, TINY.topk, dtype=torch.int32, device="cuda")
        step = {k: v[t:t + 1].cuda().contiguous() for k, v in tok.items()}
        out[:, t] = layer.decode(step, sel_out=s1, rope=True).cpu()
        sel[:, t] = s1[:, 0].cpu()
    torch.cuda.synchronize()
    got = {"out": out, "sel": sel, "rows": layer.rows[:, :T // 4].cpu(),
           "rows_i": layer.rows_i[:, :T // 4].cpu()}
    pos = np.arange(T)
    inv = params["inv_freq"].numpy()
    otok = {k: G.f64(v) for k, v in tok.items()}
    for k, h in (("q", 4), ("kv", None), ("qi", 2)):
        x3 = otok[k] if h else otok[k][:, None]
        r = oracle.round_store(oracle.rope_heads(x3, pos, inv), "f32")
        otok[k] = r if h else r[:, 0]
    par = {k: G.f64(v) for k, v in params.items()}
    G.check_against_oracle(TINY, otok, par, got, 0, list(range(T)), end_to_end=True)
    G.check_against_oracle(TINY, otok, par, got, 0, list(range(T)))


def test_tiny_fp32_dense_to_sparse_crossing():
    """The indexer engages once a query sees more than k = 8 rows (p >= 35 at ratio 4)."""
    res = G.run_gpu(TINY, 1, 1, [30], 20)
    sel = res["sel"][0].numpy()
    for p in range(50):
        nv = oracle.visible_rows(p, 4)
        row = sel[p]
        if nv <= 8:
            assert list(row[:nv]) == list(range(nv)) and (row[nv:] == -1).all()
        else:
            assert (row >= 0).all()
    _check_layer(TINY, res, 0, list(range(50)), 1, end_to_end=True)


def test_small_bf16_ratio4_sparse_chunked():
    """bf16, ratio 4 overlap, sparse regime (100 rows > k = 16), 2 sequences, chunked prefill
    of ragged chunk sizes, then decode steps across window and compress boundaries."""
    res = G.run_gpu(SMALL_BF16, 3, 2, [37, 100, 63], 200)
    for b in range(2):
        _check_layer(SMALL_BF16, res, b, list(range(0, 400, 3)) + list(range(380, 400)), 3)
    dec = G.run_gpu(SMALL_BF16, 3, 2, [400], 0)
    assert torch.equal(dec["rows"], res["rows"]) and torch.equal(dec["rows_i"], res["rows_i"])
    assert torch.equal(dec["sel"], res["sel"])


def test_ratio128_dense_bf16():
    """Plain ratio-128 windows, no indexer (every visible row attended), across row births."""
    spec = LayerSpec(ratio=128, heads=8, dim=64, rope_dim=16, window=16, indexer=False, topk=0)
    res = G.run_gpu(spec, 5, 2, [100, 200], 134)
    for b in range(2):
        _check_layer(spec, res, b, list(range(0, 434, 5)) + list(range(380, 434)), 5)


def test_ratio0_window_only():
    spec = LayerSpec(ratio=0, heads=8, dim=64, rope_dim=16, window=16, indexer=False, topk=0)
    res = G.run_gpu(spec, 6, 3, [9, 40], 30)
    for b in range(3):
        _check_layer(spec, res, b, list(range(79)), 6)


def test_ratio4_overlap_off_and_odd_ratio():
    """A non-overlapping ratio-4 lane and an odd ratio (3) with an indexer."""
    for spec in (LayerSpec(ratio=4, overlap=False, heads=4, dim=64, rope_dim=16, window=8,
                           index_heads=2, index_dim=32, topk=6, dtype=torch.float32),
                 LayerSpec(ratio=3, overlap=True, heads=4, dim=64, rope_dim=16, window=8,
                           index_heads=2, index_dim=32, topk=6, dtype=torch.float32)):
        res = G.run_gpu(spec, 7, 1, [50, 11], 29)
        _check_layer(spec, res, 0, list(range(90)), 7, end_to_end=True)


def test_ragged_batch_positions():
    """Sequences at different positions in one call: each sequence's prefix is built alone
    (batch-1 views of the same buffers), then one batched prefill and decode continue all."""
    import synth.csa as SC
    from sparse_attention_dsv4_amd import layer as LY
    spec = SMALL_BF16
    seed, B = 9, 3
    lens = [5, 130, 61]
    T = max(lens) + 40 + 10
    params = SC.layer_params(spec, seed, device="cuda")
    big = LY.CsaLayer(spec, B, T, params, device="cuda")
    for b, L in enumerate(lens):
        one = LY.CsaLayer(spec, 1, T, params, device="cuda")
        # share buffers with sequence b of the batch
        one.state, one.rows, one.ring = big.state[b:b + 1], big.rows[b:b + 1], big.ring[b:b + 1]
        one.state_i, one.rows_i = big.state_i[b:b + 1], big.rows_i[b:b + 1]
        tok = SC.batch_token_inputs(spec, seed, [0], L, device="cuda")
        tok = {k: v.clone() for k, v in tok.items()}
        # sequence b's own stream: regenerate with b's index
        tok = {k: SC.token_inputs(spec, seed, b, 0, L, device="cuda")[k][None].contiguous()
               for k in tok}
        one.prefill(tok)
    big.lengths = list(lens)
    tok = {k: torch.stack([SC.token_inputs(spec, seed, b, L, L + 40, device="cuda")[k]
                           for b, L in enumerate(lens)]) for k in tok}
    sel = torch.empty(B, 40, spec.topk, dtype=torch.int32, device="cuda")
    out = big.prefill(tok, sel_out=sel).cpu()
    outs = [out]
    sels = [sel.cpu()]
    for i in range(10):
        t = {k: torch.stack([SC.token_inputs(spec, seed, b, L + 40 + i, L + 41 + i,
                                             device="cuda")[k][0] for b, L in enumerate(lens)])
             for k in tok}
        s1 = torch.empty(B, 1, spec.topk, dtype=torch.int32, device="cuda")
        outs.append(big.decode(t, sel_out=s1).cpu()[:, None])
        sels.append(s1.cpu())
    out = torch.cat(outs, 1)
    sel = torch.cat(sels, 1)
    for b, L in enumerate(lens):
        Tb = L + 50
        res = {"T": Tb, "out": torch.zeros(B, Tb, spec.heads, spec.dim),
               "sel": torch.zeros(B, Tb, spec.topk, dtype=torch.int32),
               "rows": big.rows[:, :Tb // 4].cpu(), "rows_i": big.rows_i[:, :Tb // 4].cpu()}
        res["out"][b, L:] = out[b].float()
        res["sel"][b, L:] = sel[b]
        _check_layer(spec, res, b, list(range(L, Tb)), seed)


def test_empty_calls_are_noops():
    import sparse_attention_dsv4_amd as K
    spec = SMALL_BF16
    cfg = spec.comp_cfg()
    rows = torch.full((1, 4, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(1, K.dsv4_comp_state_bytes(cfg, 1), dtype=torch.uint8, device="cuda")
    lane = torch.empty(1, 0, 128, dtype=torch.bfloat16, device="cuda")
    K.dsv4_compress_prefill(cfg, st, lane, lane, [0],
                            torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda"),
                            torch.zeros(64, dtype=torch.bfloat16, device="cuda"),
                            torch.zeros(8, device="cuda"), rows)
    torch.cuda.synchronize()
    assert (rows == 7.0).all()


def test_fails_closed_before_launch():
    """A capacity error leaves the buffers as they were."""
    import sparse_attention_dsv4_amd as K
    spec = SMALL_BF16
    cfg = spec.comp_cfg()
    rows = torch.full((1, 2, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(1, K.dsv4_comp_state_bytes(cfg, 1), dtype=torch.uint8, device="cuda")
    lane = torch.ones(1, 12, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(K.Dsv4Error) as e:
        K.dsv4_compress_prefill(cfg, st, lane, lane, [0],
                                torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda"),
                                torch.ones(64, dtype=torch.bfloat16, device="cuda"),
                                torch.zeros(8, device="cuda"), rows)
    assert e.value.code == -3
    torch.cuda.synchronize()
    assert (rows == 3.0).all() and (st == 0).all()


# ---------------------------------------------------------------- V4-Flash shapes (mfma paths)
V4_R4 = LayerSpec(ratio=4)                                      # 64 x 512, window 128, 64 x 128, top-512
V4_R128 = LayerSpec(ratio=128, indexer=False, topk=0)
V4_R0 = LayerSpec(ratio=0, indexer=False, topk=0)


def test_v4_ratio4_sparse_prefill_and_decode():
    """V4 shapes, ratio-4 overlap with the indexer: 2 sequences, ragged prefill chunks, then
    decode steps (split-key decode attention); 601 rows by the end, so queries from p = 2051
    on are in the sparse regime.  Rows bit-identical between decode and one-shot prefill;
    selections too (the scoring arithmetic does not depend on the chunk)."""
    res = G.run_gpu(V4_R4, 11, 2, [999, 1100, 205], 100)
    pos = sorted(set(list(range(0, 2304, 37)) + list(range(2040, 2060)) + list(range(2304, 2404))))
    for b in range(2):
        _check_layer(V4_R4, res, b, pos, 11)
    one = G.run_gpu(V4_R4, 11, 2, [2404], 0)
    assert torch.equal(one["rows"], res["rows"]) and torch.equal(one["rows_i"], res["rows_i"])
    assert torch.equal(one["sel"], res["sel"])


def test_v4_ratio4_small_prefill_chunks_split_keys():
    """Few queries per call: prefill attention also takes the split-key path."""
    res = G.run_gpu(V4_R4, 12, 1, [2070, 3, 5], 2)
    _check_layer(V4_R4, res, 0, list(range(2060, 2080)), 12)


def test_v4_ratio128_dense():
    res = G.run_gpu(V4_R128, 13, 3, [300, 700], 60)
    for b in range(3):
        _check_layer(V4_R128, res, b, list(range(0, 1000, 17)) + list(range(1000, 1060)), 13)


def test_v4_ratio0_window():
    res = G.run_gpu(V4_R0, 14, 2, [200], 30)
    for b in range(2):
        _check_layer(V4_R0, res, b, list(range(0, 230, 3)), 14)


def test_v4_attention_with_ragged_selection():
    """A caller-made selection with -1 entries in the middle, out-of-range and duplicate-free
    rows: entries outside [0, visible) are skipped, the rest attended in list order."""
    import sparse_attention_dsv4_amd as K
    import synth.csa as SC
    from sparse_attention_dsv4_amd.layer import CsaLayer
    spec = V4_R4
    seed, T = 15, 1200
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, 1, T, params, device="cuda")
    layer.prefill(SC.batch_token_inputs(spec, seed, [0], T - 40, device="cuda"))
    tok = SC.batch_token_inputs(spec, seed, [T - 40], 40, device="cuda")
    K.dsv4_compress_prefill(spec.comp_cfg(), layer.state, tok["a"], tok["g"], [T - 40],
                            params["ape"], params["norm_w"], params["inv_freq"], layer.rows)
    nv_last = T // 4
    rng = np.random.default_rng(0)
    sel = np.full((1, 40, spec.topk), -1, dtype=np.int32)
    for i in range(40):
        p = T - 40 + i
        nv = oracle.visible_rows(p, 4)
        cand = rng.choice(nv, size=200, replace=False)
        row = np.full(spec.topk, -1, dtype=np.int32)
        slots = np.sort(rng.choice(spec.topk, size=260, replace=False))
        row[slots[:200]] = np.sort(cand)
        row[slots[200:230]] = nv + rng.integers(0, 50, size=30)     # not yet visible
        row[slots[230:]] = -7
        sel[0, i] = row
    sel_t = torch.from_numpy(sel).cuda()
    out = torch.empty_like(tok["q"])
    K.dsv4_csa_attn_prefill(spec.attn_cfg(), tok["q"], tok["kv"], layer.ring, layer.rows, sel_t,
                            [nv_last], [T - 40], params["sinks"], out, layer.ws_attn)
    torch.cuda.synchronize()
    tk, par = G.oracle_inputs(spec, seed, 0, T)
    rows = G.f64(layer.rows[0, :nv_last])
    pos = list(range(T - 40, T))
    ref_sel = []
    for i, p in enumerate(pos):
        r = sel[0, i]
        r = r[(r >= 0) & (r < oracle.visible_rows(p, 4))]
        ref_sel.append(np.concatenate([r, np.full(spec.topk - len(r), -1)]))
    ref = G.oracle_attention(spec, tk, par, rows, np.array(ref_sel), pos)
    mr = G.max_rel_rows(G.f64(out[0]), ref)
    assert mr.max() <= 2e-2, mr.max()


@pytest.mark.parametrize("B", [8, 64])
def test_v4_decode_with_ragged_selection(B):
    """Decode over caller-made selections with -1 entries in the middle, rows not yet visible
    and negative codes: 200 attended rows + the 128-token window per query.  At batch 64 a
    query's ~330 keys are one split, several 64-key chunks each compacted from the selection
    (the double-buffered path); at batch 8, one-chunk splits."""
    import sparse_attention_dsv4_amd as K
    import synth.csa as SC
    from sparse_attention_dsv4_amd.layer import CsaLayer
    spec = V4_R4
    seed, T = 16, 1200
    params = SC.layer_params(spec, seed, device="cuda")
    layer = CsaLayer(spec, B, T + 8, params, device="cuda")
    layer.prefill(SC.batch_token_inputs(spec, seed, [0] * B, T, device="cuda"))
    p = T
    nv = oracle.visible_rows(p, 4)
    tok = SC.batch_token_inputs(spec, seed, [p] * B, 1, device="cuda", fields=["q", "kv"])
    rng = np.random.default_rng(1)
    sel = np.full((B, spec.topk), -1, dtype=np.int32)
    for b in range(B):
        row = np.full(spec.topk, -1, dtype=np.int32)
        slots = np.sort(rng.choice(spec.topk, size=260, replace=False))
        row[slots[:200]] = np.sort(rng.choice(nv, size=200, replace=False))
        row[slots[200:230]] = nv + rng.integers(0, 50, size=30)         # not yet visible
        row[slots[230:]] = -7
        sel[b] = row
    out = torch.empty(B, spec.heads, spec.dim, dtype=spec.dtype, device="cuda")
    K.dsv4_csa_attn_decode(spec.attn_cfg(), tok["q"][:, 0].contiguous(), tok["kv"][:, 0].contiguous(),
                           layer.ring, layer.rows, torch.from_numpy(sel).cuda(), [nv] * B, [p] * B,
                           params["sinks"], out, layer.ws_attn)
    torch.cuda.synchronize()
    out = out.cpu()
    for b in (range(B) if B <= 8 else (0, 1, B // 2, B - 1)):
        tk, par = G.oracle_inputs(spec, seed, b, p + 1)
        r = sel[b][(sel[b] >= 0) & (sel[b] < nv)]
        ref_sel = np.concatenate([r, np.full(spec.topk - len(r), -1)])[None]
        ref = G.oracle_attention(spec, tk, par, G.f64(layer.rows[b, :nv]), ref_sel, [p])
        mr = G.max_rel_rows(G.f64(out[b])[None], ref)
        assert mr.max() <= 2e-2, f"sequence {b}: max-rel {mr.max():.3g}"


@pytest.mark.parametrize("spec_name", ["small_bf16", "v4_ratio4", "v4_ratio4_long"])
def test_batch_beyond_one_launch_slice(spec_name):
    """130 sequences: every launcher walks the batch in slices of 128 sequences, so
    sequences 127, 128 and 129 sit on either side of a slice edge (the generic kernels at the
    small shape, sparse regime; the MFMA kernels at the V4 shape, dense regime).  The long
    case's decode steps attend 204 keys: the 128-sequence slice as one split per query (the
    double-buffered 64-key chunks, head groups grouped by XCD), the 2-sequence slice as
    13 one-chunk splits."""
    spec, chunks, n_dec = {"small_bf16": (SMALL_BF16, [120, 50], 30), "v4_ratio4": (V4_R4, [40], 4),
                           "v4_ratio4_long": (V4_R4, [300], 4)}[spec_name]
    res = G.run_gpu(spec, 21, 130, chunks, n_dec)
    T = sum(chunks) + n_dec
    pos = sorted(set(list(range(0, T, 7)) + list(range(T - 6, T))))
    for b in (0, 127, 128, 129):
        _check_layer(spec, res, b, pos, 21)


def test_v4_pro_top1024_sparse():
    """V4-Pro's selection size (top-1024; the layer shape otherwise as Flash's ratio-4 layer):
    1135 rows by the end, so queries from p = 4099 on select 1024 of their rows (chunked
    prefill, then decode steps)."""
    spec = LayerSpec(ratio=4, topk=1024)
    res = G.run_gpu(spec, 31, 1, [2500, 2000], 40)
    pos = sorted(set(list(range(0, 4540, 131)) + list(range(4090, 4110)) + list(range(4520, 4540))))
    _check_layer(spec, res, 0, pos, 31)
