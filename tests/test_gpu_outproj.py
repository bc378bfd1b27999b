"""The layer's neighbours through the C ABI against the oracle (needs a gfx950 GPU):
RoPE of per-head vectors and its inverse (dsv4_rope), the grouped block-diagonal output
projection (dsv4_grouped_proj) on all three of its kernels (up to 32 tokens: weight
streaming; more: LDS-tiled MFMA; fp32 or other shapes: one thread per output), and the
compressor lanes projected from hidden states (dsv4_lane_proj: both lanes in one launch of
the tiled kernel, each equal bit for bit to the one-group projection).

Bars: RoPE as the compressed rows (bf16 within 2 ulp of the pair's norm, fp32 max-rel
1e-5 per head); projection max-rel per (token, group) row 4e-3 in bf16 (two ulps of the
output rounding; the fp32 accumulation of up to 4096 products adds ~1e-6) and 1e-5 in fp32.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_dsv4_amd as K
import synth.csa as SC
from sparse_attention_dsv4_amd.layer import CsaLayer, LayerSpec, compressor_lanes, output_path
from tests import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _inv_freq(rd, theta=160000.0):
    return torch.tensor([theta ** (-2.0 * i / rd) for i in range(rd // 2)], dtype=torch.float32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("inverse", [False, True], ids=["forward", "inverse"])
@pytest.mark.parametrize("H,D,rd", [(64, 512, 64), (1, 512, 64), (64, 128, 64), (3, 20, 6)],
                         ids=["q", "kv", "qi", "odd"])
def test_rope_matches_oracle(H, D, rd, inverse, dtype):
    B, S = 2, 37
    pos0 = [0, (1 << 20) + 13]                          # near zero and far along
    x = synth.normal((B, S, H, D), seed=H + D + rd, stream="rope_x", dtype=dtype, device="cuda")
    inv = _inv_freq(rd)
    y = x.clone()
    K.dsv4_rope(K.RopeCfg(H, D, rd, inverse, dtype), y, pos0, inv.cuda())
    torch.cuda.synchronize()
    for b in range(B):
        pos = np.arange(S) + pos0[b]
        ref = oracle.rope_heads(G.f64(x[b]), pos, inv.numpy(), inverse=inverse)
        G.assert_rows_match(G.f64(y[b]), ref, "bf16" if dtype == torch.bfloat16 else "f32",
                            f"rope seq {b}", rd)
    # the inverse undoes the forward (up to the storage rounding of the two passes)
    z = y.clone()
    K.dsv4_rope(K.RopeCfg(H, D, rd, not inverse, dtype), z, pos0, inv.cuda())
    torch.cuda.synchronize()
    tol = 2 ** -6 if dtype == torch.bfloat16 else 1e-5
    assert G.max_rel_rows(G.f64(z), G.f64(x)).max() <= tol


def _proj_case(T, Gr, Kd, R, dtype, seed, sample=None):
    x = synth.normal((T, Gr, Kd), seed=seed, stream="proj_x", dtype=dtype, device="cuda")
    w = synth.normal((Gr, R, Kd), seed=seed, stream="proj_w", scale=Kd ** -0.5, dtype=dtype,
                     device="cuda")
    y = torch.full((T, Gr, R), float("nan"), dtype=dtype, device="cuda")
    K.dsv4_grouped_proj(K.GprojCfg(Gr, Kd, R, dtype), x, w, y)
    torch.cuda.synchronize()
    rows = np.arange(T) if sample is None else np.unique(np.concatenate(
        [[0, T - 1], np.random.default_rng(seed).integers(0, T, sample)]))
    idx = torch.as_tensor(rows, device=x.device)
    xs = G.f64(x[idx]).reshape(len(rows), Gr, Kd)
    # the oracle takes [tokens, H, D]: here H = G heads of width K
    ref = oracle.grouped_out_proj(xs, G.f64(w)).reshape(len(rows), Gr, R)
    got = G.f64(y[idx])
    assert np.isfinite(got).all(), "outputs left unwritten"
    mr = G.max_rel_rows(got, ref)
    bar = 4e-3 if dtype == torch.bfloat16 else 1e-5
    assert mr.max() <= bar, f"max-rel {mr.max():.3g} (T={T}, G={Gr}, K={Kd}, R={R})"
    return mr.max()


@pytest.mark.parametrize("T", [1, 8, 31, 32])
def test_grouped_proj_streaming(T):
    """Decode shapes (wo_a: 8 groups x 1024 x 4096): the weight-streaming kernel."""
    _proj_case(T, 8, 4096, 1024, torch.bfloat16, seed=100 + T)


@pytest.mark.parametrize("T", [33, 200, 2048])
def test_grouped_proj_tiled(T):
    """Prefill shapes: 128 x 256 tiles; 33 and 200 leave ragged token tiles."""
    _proj_case(T, 8, 4096, 1024, torch.bfloat16, seed=200 + T, sample=None if T < 2048 else 96)


def test_grouped_proj_other_k():
    """Smaller K on both MFMA kernels (K = 512 and 1536), and 128-row tiles (R = 384).  The
    128-row tiles take k blocks of 128 when K allows (K = 128: a single block) and otherwise a
    ring of four blocks of 64, here with fewer blocks than the ring holds (K = 64, 192) and
    more (K = 576)."""
    _proj_case(5, 2, 512, 64, torch.bfloat16, seed=7)
    _proj_case(300, 3, 1536, 256, torch.bfloat16, seed=8)
    _proj_case(40, 2, 512, 384, torch.bfloat16, seed=11)
    for i, kd in enumerate((64, 128, 192, 576)):
        _proj_case(70, 2, kd, 128, torch.bfloat16, seed=20 + i)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_grouped_proj_generic(dtype):
    """Shapes the MFMA kernels do not take (and fp32): one thread per output."""
    _proj_case(9, 3, 40, 24, dtype, seed=9)
    _proj_case(70, 2, 96, 48, dtype, seed=10)


@pytest.mark.parametrize("S", [1, 40], ids=["decode", "prefill"])
def test_output_path_matches_oracle(S):
    """Attention output -> inverse RoPE (rounded to bf16, as the stored activation) -> grouped
    projection, end to end through the layer's output path at the layer's shapes."""
    spec = LayerSpec(ratio=4)
    B, Gr, R = 3, 8, 1024
    Kd = spec.heads // Gr * spec.dim
    pos0 = [7, 4096 + 3, 65536 + 100]
    o = synth.normal((B, S, spec.heads, spec.dim), seed=31 + S, stream="attn_out",
                     dtype=torch.bfloat16, device="cuda")
    wo_a = synth.normal((Gr, R, Kd), seed=31, stream="wo_a", scale=Kd ** -0.5,
                        dtype=torch.bfloat16, device="cuda")
    inv = _inv_freq(spec.rope_dim)
    o_in = G.f64(o)
    y = output_path(spec, o, pos0, inv.cuda(), wo_a)
    torch.cuda.synchronize()
    w64 = G.f64(wo_a)
    for b in range(B):
        pos = np.arange(S) + pos0[b]
        turned = oracle.bf16_round(oracle.rope_heads(o_in[b], pos, inv.numpy(), inverse=True))
        ref = oracle.grouped_out_proj(turned, w64).reshape(S, Gr, R)
        mr = G.max_rel_rows(G.f64(y[b]), ref)
        assert mr.max() <= 4e-3, f"sequence {b}: max-rel {mr.max():.3g}"


@pytest.mark.parametrize("T", [8, 33, 300, 2048, 2049])
def test_lane_proj_equals_two_projections(T):
    """dsv4_lane_proj computes both lanes in one launch from 33 tokens on (up to 32: the
    streaming kernel, one call per lane); either way each lane equals, bit for bit, the
    one-group dsv4_grouped_proj of the same weight (same tiles, same arithmetic)."""
    W, hid = 1024, 4096
    x = synth.normal((T, hid), seed=61 + T, stream="hidden", dtype=torch.bfloat16, device="cuda")
    wkv = synth.normal((W, hid), seed=61, stream="wkv", scale=hid ** -0.5, dtype=torch.bfloat16,
                       device="cuda")
    wg = synth.normal((W, hid), seed=61, stream="wgate", scale=hid ** -0.5, dtype=torch.bfloat16,
                      device="cuda")
    a, g = compressor_lanes(x, wkv, wg)
    cfg = K.GprojCfg(1, hid, W, torch.bfloat16)
    ra = torch.empty(T, 1, W, dtype=torch.bfloat16, device="cuda")
    rg = torch.empty(T, 1, W, dtype=torch.bfloat16, device="cuda")
    K.dsv4_grouped_proj(cfg, x.view(T, 1, hid), wkv.view(1, W, hid), ra)
    K.dsv4_grouped_proj(cfg, x.view(T, 1, hid), wg.view(1, W, hid), rg)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), ra.view(T, W).view(torch.int16))
    assert torch.equal(g.view(torch.int16), rg.view(T, W).view(torch.int16))
    # and against the oracle on sampled tokens (first, last, a middle one)
    for t in sorted({0, T // 2, T - 1}):
        x64 = G.f64(x[t:t + 1])[:, None, :]
        for got, w, n in ((a, wkv, "a"), (g, wg, "g")):
            ref = oracle.grouped_out_proj(x64, G.f64(w)[None])
            mr = G.max_rel_rows(G.f64(got[t:t + 1]), ref)
            assert mr.max() <= 4e-3, f"token {t} lane {n}: max-rel {mr.max():.3g}"


@pytest.mark.parametrize("T", [1, 8, 300], ids=["step", "b8", "chunk300"])
def test_compressor_lanes_from_hidden_states(T):
    """hidden [T, 4096] -> a, g [T, 1024] (wkv, wgate [1024, 4096]) -> rows of the ratio-4
    compressor, against the oracle's matmul (rounded to bf16, the stored lanes) and rows."""
    spec = LayerSpec(ratio=4)
    W, hid = spec.coff * spec.dim, 4096
    x = synth.normal((T, hid), seed=51 + T, stream="hidden", dtype=torch.bfloat16, device="cuda")
    wkv = synth.normal((W, hid), seed=51, stream="wkv", scale=hid ** -0.5, dtype=torch.bfloat16,
                       device="cuda")
    wg = synth.normal((W, hid), seed=51, stream="wgate", scale=hid ** -0.5, dtype=torch.bfloat16,
                      device="cuda")
    a, g = compressor_lanes(x, wkv, wg)
    torch.cuda.synchronize()
    x64 = G.f64(x)[:, None, :]
    ra = oracle.grouped_out_proj(x64, G.f64(wkv)[None])
    rg = oracle.grouped_out_proj(x64, G.f64(wg)[None])
    for got, ref, n in ((a, ra, "a"), (g, rg, "g")):
        mr = G.max_rel_rows(G.f64(got), ref)
        assert mr.max() <= 4e-3, f"lane {n}: max-rel {mr.max():.3g}"
    if T < 2 * spec.ratio:
        return
    # the lanes drive the compressor: rows from the GPU lanes against the oracle's rows from
    # the same (bf16) lanes
    par = SC.layer_params(spec, 51, device="cuda")
    cc = spec.comp_cfg()
    state = torch.empty(1, K.dsv4_comp_state_bytes(cc, 1), dtype=torch.uint8, device="cuda")
    rows = torch.empty(1, T // spec.ratio, spec.dim, dtype=torch.bfloat16, device="cuda")
    K.dsv4_compress_prefill(cc, state, a[None], g[None], [0], par["ape"], par["norm_w"],
                            par["inv_freq"], rows)
    torch.cuda.synchronize()
    ref_rows = oracle.compressor_rows(G.f64(a), G.f64(g), G.f64(par["ape"]), G.f64(par["norm_w"]),
                                      par["inv_freq"].cpu().numpy(), ratio=spec.ratio,
                                      overlap=spec.is_overlap, eps=spec.eps, store="bf16")
    G.assert_rows_match(G.f64(rows[0]), ref_rows, "bf16", "rows from projected lanes", spec.rope_dim)


@pytest.mark.parametrize("spec", [LayerSpec(ratio=4), LayerSpec(ratio=4, heads=4, dim=64, rope_dim=16,
                                  window=16, index_heads=2, index_dim=32, topk=8,
                                  dtype=torch.float32)], ids=["v4_bf16", "small_fp32"])
def test_layer_rotates_its_inputs(spec):
    """A layer given unrotated q / kv / qi (rope=True) equals one given the same inputs
    rotated beforehand (by the oracle's rotation, rounded to storage), through prefill and
    decode: the wiring of the inputs' RoPE (positions, head shapes, which tensors)."""
    B, seed, prefix, steps = 2, 71, 300, 5
    params = SC.layer_params(spec, seed, device="cuda")
    layers = [CsaLayer(spec, B, prefix + steps + 8, params, device="cuda", max_chunk=prefix)
              for _ in range(2)]
    inv = params["inv_freq"].cpu().numpy()
    store = "bf16" if spec.dtype == torch.bfloat16 else "f32"

    def pre_rotated(tok, pos_rows):
        out = {}
        for k, v in tok.items():
            if k in ("q", "kv", "qi"):
                x = G.f64(v)
                shp = x.shape
                x = x.reshape(-1, 1 if k == "kv" else shp[-2], shp[-1])
                r = oracle.rope_heads(x, pos_rows, inv)
                r = oracle.round_store(r, store).reshape(shp)
                out[k] = torch.tensor(r, dtype=spec.dtype, device="cuda")
            else:
                out[k] = v.clone()
        return out

    tok = SC.batch_token_inputs(spec, seed, [0] * B, prefix, device="cuda")
    pos_rows = np.tile(np.arange(prefix), B)
    o_ref = layers[0].prefill(pre_rotated(tok, pos_rows))
    o_rot = layers[1].prefill({k: v.clone() for k, v in tok.items()}, rope=True)
    torch.cuda.synchronize()
    bar = 2e-2 if spec.dtype == torch.bfloat16 else 1e-5
    assert G.max_rel_rows(G.f64(o_rot), G.f64(o_ref)).max() <= bar
    for i in range(steps):
        p = prefix + i
        t = SC.batch_token_inputs(spec, seed, [p] * B, 1, device="cuda")
        t = {k: v[:, 0].contiguous() for k, v in t.items()}
        o_ref = layers[0].decode(pre_rotated(t, np.full(B, p)))
        o_rot = layers[1].decode({k: v.clone() for k, v in t.items()}, rope=True)
        torch.cuda.synchronize()
        assert G.max_rel_rows(G.f64(o_rot), G.f64(o_ref)).max() <= bar, f"decode step {i}"
