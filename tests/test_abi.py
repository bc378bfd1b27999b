"""The C ABI on the CPU: the library loads, exports what include/dsv4.h declares, and every
argument check fails before any launch.  No compute call is made (there is no GPU here):
each call below is rejected by host validation, or is a documented no-op."""
import ctypes
import os
import re

import pytest

import sparse_attention_dsv4_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EINVAL, EUNSUP, ECAP, EHIP, EWS = -1, -2, -3, -4, -5
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: every call using it fails validation


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(K.lib_path):
        pytest.skip("libdsv4.so not built")
    return K.lib()


def _i64(*v):
    return (ctypes.c_int64 * len(v))(*v)


def test_exports_match_header(L):
    header = open(os.path.join(ROOT, "include", "dsv4.h")).read()
    declared = set(re.findall(r"\b(dsv4_[a-z_0-9]+)\s*\(", header))
    assert declared == set(K.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name
    assert "gfx950" in K.dsv4_version()


def test_sizes():
    c = K.CompCfg(ratio=4, overlap=True, dim=512, rope_dim=64)
    assert K.dsv4_comp_state_bytes(c, 3) == 3 * 2 * 2 * 4 * 1024 * 2
    c128 = K.CompCfg(ratio=128, overlap=False, dim=512, rope_dim=64, dtype=K.torch.float32)
    assert K.dsv4_comp_state_bytes(c128, 1) == 2 * 1 * 128 * 512 * 4
    ic = K.IndexCfg(heads=64, dim=128, topk=512, ratio=4)
    assert K.dsv4_index_workspace_bytes(ic, 2, 10, 1000) >= 2 * 10 * 1000 * 4
    bad = K.CompCfg(ratio=0, overlap=False, dim=8, rope_dim=0)
    assert K.dsv4_comp_state_bytes(bad, 1) == 0


def _comp(L, cfg, **kw):
    a = dict(state=FAKE, kv=FAKE, gate=FAKE, batch=1, n_new=4, lb=_i64(0), ape=FAKE, nw=FAKE,
             inv=FAKE, rows=FAKE, cap=100)
    a.update(kw)
    c = cfg.c() if cfg is not None else None
    return L.dsv4_compress_prefill(ctypes.byref(c) if c is not None else None, a["state"], a["kv"],
                                   a["gate"], a["batch"], a["n_new"], a["lb"], a["ape"], a["nw"],
                                   a["inv"], a["rows"], a["cap"], None)


def test_compress_validation(L):
    cfg = K.CompCfg(ratio=4, overlap=True, dim=64, rope_dim=16)
    assert _comp(L, None) == EINVAL
    assert _comp(L, K.CompCfg(ratio=0, overlap=True, dim=64, rope_dim=16)) == EINVAL
    assert _comp(L, K.CompCfg(ratio=4, overlap=True, dim=64, rope_dim=15)) == EINVAL
    assert _comp(L, K.CompCfg(ratio=4, overlap=True, dim=64, rope_dim=80)) == EINVAL
    assert _comp(L, K.CompCfg(ratio=4, overlap=True, dim=5000, rope_dim=16)) == EINVAL
    assert _comp(L, K.CompCfg(ratio=4, overlap=True, dim=64, rope_dim=16, eps=-1.0)) == EINVAL
    assert _comp(L, cfg, n_new=-1) == EINVAL
    assert _comp(L, cfg, batch=-1) == EINVAL
    assert _comp(L, cfg, state=None) == EINVAL
    assert _comp(L, cfg, inv=None) == EINVAL
    assert _comp(L, cfg, lb=_i64(-3)) == EINVAL
    assert _comp(L, cfg, lb=_i64(398), n_new=4, cap=99) == ECAP          # needs 100 rows
    assert "row_cap" in L.dsv4_last_error().decode()
    assert _comp(L, cfg, lb=_i64(2 ** 31), n_new=4, cap=2 ** 40) == ECAP
    # documented no-ops: nothing to do, nothing dereferenced
    assert _comp(L, cfg, n_new=0, state=None, kv=None) == 0
    assert _comp(L, cfg, batch=0, state=None, kv=None, lb=None) == 0


def _index(L, cfg, **kw):
    a = dict(qi=FAKE, w=FAKE, rows=FAKE, cap=1000, n_rows=_i64(600), pos0=_i64(2000), batch=1,
             s=4, sel=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    c = cfg.c()
    return L.dsv4_index_topk(ctypes.byref(c), a["qi"], a["w"], a["rows"], a["cap"], a["n_rows"],
                             a["pos0"], a["batch"], a["s"], a["sel"], a["ws"], a["ws_bytes"], None)


def test_index_validation(L):
    cfg = K.IndexCfg(heads=64, dim=128, topk=512, ratio=4)
    assert _index(L, K.IndexCfg(heads=0, dim=128, topk=512, ratio=4)) == EUNSUP
    assert _index(L, K.IndexCfg(heads=300, dim=128, topk=512, ratio=4)) == EUNSUP
    assert _index(L, K.IndexCfg(heads=64, dim=128, topk=0, ratio=4)) == EINVAL
    assert _index(L, cfg, n_rows=_i64(499)) == EINVAL                   # last query sees 501
    assert _index(L, cfg, n_rows=_i64(1001)) == ECAP
    assert _index(L, cfg, pos0=_i64(-1)) == EINVAL
    assert _index(L, cfg, ws_bytes=16) == EWS
    assert _index(L, cfg, ws=None) == EWS
    assert _index(L, cfg, ws=ctypes.c_void_p(FAKE.value + 4)) == EINVAL    # key rows need 16 B
    assert "aligned" in L.dsv4_last_error().decode()
    # key rows are padded to a multiple of 4 keys, the key block to 256 bytes
    assert K.dsv4_index_workspace_bytes(cfg, 2, 3, 601) == 2 * 3 * 604 * 4 + 96
    # few queries (8 per sequence, past the fused decode indexer) over many rows add k
    # candidate rows and keys per 8192-row chunk (split selection)
    assert K.dsv4_index_workspace_bytes(cfg, 1, 8, 65536) == 8 * 65536 * 4 + 2 * 8 * 8 * 512 * 4
    # a decode call the fused indexer takes: 4 queries over 16,384 rows are scored by 64
    # workgroups of 256 rows each, which pass on up to 128 of their best (key and row) and a
    # cutoff; that candidate area is larger than the split selection's (none at 16,384 rows)
    assert K.dsv4_index_workspace_bytes(cfg, 4, 1, 16384) == 4 * 16384 * 4 + 4 * 64 * (128 * 8 + 4)
    assert K.dsv4_index_workspace_bytes(cfg, 4, 1, 65536) == 4 * 65536 * 4 + 4 * 64 * (128 * 8 + 4)
    assert K.dsv4_index_workspace_bytes(cfg, 65, 1, 65536) == 65 * 65536 * 4
    assert _index(L, cfg, sel=None) == EINVAL
    assert _index(L, cfg, s=70000) == EUNSUP
    assert _index(L, cfg, s=0, qi=None) == 0


def _attn(L, cfg, decode=True, **kw):
    a = dict(q=FAKE, kv=FAKE, ring=FAKE, rows=FAKE, cap=1000, sel=FAKE, n_rows=_i64(600),
             pos=_i64(2000), sinks=FAKE, out=FAKE, batch=1, s=3, ws=None, ws_bytes=0)
    a.update(kw)
    c = cfg.c()
    if decode:
        return L.dsv4_csa_attn_decode(ctypes.byref(c), a["q"], a["kv"], a["ring"], a["rows"], a["cap"],
                                      a["sel"], a["n_rows"], a["pos"], a["sinks"], a["out"],
                                      a["batch"], a["ws"], a["ws_bytes"], None)
    return L.dsv4_csa_attn_prefill(ctypes.byref(c), a["q"], a["kv"], a["ring"], a["rows"], a["cap"],
                                   a["sel"], a["n_rows"], a["pos"], a["sinks"], a["out"],
                                   a["batch"], a["s"], a["ws"], a["ws_bytes"], None)


def test_attention_validation(L):
    cfg = K.AttnCfg(heads=64, dim=512, window=128, ratio=4, topk=512, scale=0.04)
    assert _attn(L, K.AttnCfg(heads=0, dim=512, window=128, ratio=4, topk=512, scale=0.04)) == EINVAL
    assert _attn(L, K.AttnCfg(heads=64, dim=512, window=0, ratio=4, topk=512, scale=0.04)) == EINVAL
    assert _attn(L, K.AttnCfg(heads=64, dim=512, window=128, ratio=4, topk=512,
                              scale=float("nan"))) == EINVAL
    assert _attn(L, cfg, rows=None) == EINVAL
    assert _attn(L, cfg, n_rows=None) == EINVAL
    assert _attn(L, cfg, n_rows=_i64(400)) == EINVAL            # query at 2000 sees 500 rows
    assert _attn(L, cfg, n_rows=_i64(1200)) == ECAP
    assert _attn(L, cfg, pos=_i64(-5)) == EINVAL
    assert _attn(L, cfg, q=None) == EINVAL
    assert _attn(L, cfg, decode=False, s=-1) == EINVAL
    nosel = K.AttnCfg(heads=64, dim=512, window=128, ratio=4, topk=0, scale=0.04)
    assert _attn(L, nosel) == EINVAL                                  # sel with topk 0
    # generic (fp32) path: dense over far more rows than one query's key list can hold
    f32 = K.AttnCfg(heads=64, dim=512, window=128, ratio=4, topk=512, scale=0.04,
                    dtype=K.torch.float32)
    assert _attn(L, f32, sel=None, n_rows=_i64(400000), cap=400000, pos=_i64(1600000)) == EUNSUP
    # bf16 mfma path: decode splits the key list and needs the partials workspace
    assert K.dsv4_attn_workspace_bytes(cfg, 1, 1) > 0
    assert _attn(L, cfg, ws=None, ws_bytes=0) == EWS
    assert _attn(L, cfg, ws=FAKE, ws_bytes=64) == EWS
    assert K.dsv4_attn_workspace_bytes(cfg, 1, 2048) == 0      # one workgroup per query
    win = K.AttnCfg(heads=8, dim=64, window=16, ratio=0, topk=0, scale=0.1)
    assert _attn(L, win, sel=FAKE, rows=None, n_rows=None) == EINVAL    # sel without rows
    assert _attn(L, cfg, batch=0, q=None) == 0


def _store(L, cfg, stores, n=None, **kw):
    """dsv4_csa_attn_decode_store with a valid decode call (ws big enough to pass the size
    check) apart from the frontier stores; every case below fails validation."""
    a = dict(q=FAKE, kv=FAKE, ring=FAKE, rows=FAKE, cap=1000, sel=FAKE, n_rows=_i64(600),
             pos=_i64(2000), sinks=FAKE, out=FAKE, batch=1, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    c = cfg.c()
    keep = [s_cfg.c() for s_cfg, *_ in stores]
    arr = (K._FrontierStore * max(1, len(stores)))()
    for i, (s_cfg, st, kv, g) in enumerate(stores):
        arr[i] = K._FrontierStore(ctypes.pointer(keep[i]), st, kv, g)
    return L.dsv4_csa_attn_decode_store(ctypes.byref(c), a["q"], a["kv"], a["ring"], a["rows"],
                                        a["cap"], a["sel"], a["n_rows"], a["pos"], a["sinks"],
                                        a["out"], a["batch"], a["ws"], a["ws_bytes"],
                                        arr if stores or n is None else None,
                                        len(stores) if n is None else n, None)


def test_decode_store_validation(L):
    cfg = K.AttnCfg(heads=64, dim=512, window=128, ratio=4, topk=512, scale=0.04)
    lane = K.CompCfg(ratio=4, overlap=True, dim=512, rope_dim=64)
    good = (lane, FAKE, FAKE, FAKE)
    # position 2000: token 2000 does not complete a window ((2000 + 1) % 4 != 0), but the
    # FAKE buffers never reach a launch because each case breaks one rule
    assert _store(L, cfg, [good], pos=_i64(2003)) == EINVAL          # completes row 500
    assert "dsv4_compress_step" in L.dsv4_last_error().decode()
    assert _store(L, cfg, [good, good, good]) == EINVAL              # more than two lanes
    assert _store(L, cfg, [], n=1) == EINVAL                         # stores NULL
    assert _store(L, cfg, [(K.CompCfg(ratio=128, overlap=False, dim=512, rope_dim=64),
                            FAKE, FAKE, FAKE)]) == EINVAL            # other ratio
    assert _store(L, cfg, [(K.CompCfg(ratio=4, overlap=True, dim=512, rope_dim=64,
                                      dtype=K.torch.float32), FAKE, FAKE, FAKE)]) == EINVAL
    assert _store(L, cfg, [(lane, None, FAKE, FAKE)]) == EINVAL       # NULL state
    assert _store(L, cfg, [(K.CompCfg(ratio=4, overlap=True, dim=0, rope_dim=0),
                            FAKE, FAKE, FAKE)]) == EINVAL            # bad lane cfg
    win = K.AttnCfg(heads=8, dim=64, window=16, ratio=0, topk=0, scale=0.1)
    assert _store(L, win, [good], rows=None, n_rows=None, sel=None) == EINVAL
    # the attention's own checks come first
    assert _store(L, cfg, [good], q=None) == EINVAL
    assert _store(L, cfg, [good], batch=0, q=None) == 0


def test_rope_and_projection_validation(L):
    def rope(cfg, x=FAKE, pos=_i64(10, 20), batch=2, s=4, inv=FAKE):
        c = cfg.c()
        return L.dsv4_rope(ctypes.byref(c), x, pos, batch, s, inv, None)
    ok_cfg = K.RopeCfg(heads=64, dim=512, rope_dim=64, inverse=True)
    assert rope(K.RopeCfg(heads=0, dim=512, rope_dim=64)) == EINVAL
    assert rope(K.RopeCfg(heads=64, dim=512, rope_dim=63)) == EINVAL      # odd
    assert rope(K.RopeCfg(heads=64, dim=64, rope_dim=80)) == EINVAL       # above dim
    assert rope(ok_cfg, x=None) == EINVAL
    assert rope(ok_cfg, inv=None) == EINVAL
    assert rope(ok_cfg, pos=_i64(10, -1)) == EINVAL
    assert rope(ok_cfg, pos=_i64(10, (1 << 31) - 3)) == ECAP
    assert rope(ok_cfg, s=70000) == EUNSUP
    assert rope(ok_cfg, batch=0, x=None) == 0
    assert rope(K.RopeCfg(heads=64, dim=512, rope_dim=0), x=None) == 0    # nothing turns

    def proj(cfg, x=FAKE, w=FAKE, y=FAKE, t=8):
        c = cfg.c()
        return L.dsv4_grouped_proj(ctypes.byref(c), x, w, y, t, None)
    g = K.GprojCfg(groups=8, in_dim=4096, out_dim=1024)
    assert proj(K.GprojCfg(groups=0, in_dim=4096, out_dim=1024)) == EINVAL
    assert proj(K.GprojCfg(groups=8, in_dim=0, out_dim=1024)) == EINVAL
    assert proj(g, w=None) == EINVAL
    assert proj(g, t=-1) == EINVAL
    assert proj(g, t=1 << 32) == EUNSUP
    assert proj(g, t=0, x=None) == 0

    def lanes(cfg, x=FAKE, wk=FAKE, wg=FAKE, a=FAKE, gl=FAKE, t=8):
        c = cfg.c()
        return L.dsv4_lane_proj(ctypes.byref(c), x, wk, wg, a, gl, t, None)
    lc = K.GprojCfg(groups=1, in_dim=4096, out_dim=1024)
    assert lanes(K.GprojCfg(groups=2, in_dim=4096, out_dim=1024)) == EINVAL   # one group only
    assert lanes(K.GprojCfg(groups=1, in_dim=0, out_dim=1024)) == EINVAL
    assert lanes(lc, wg=None) == EINVAL
    assert lanes(lc, a=None) == EINVAL
    assert lanes(lc, t=-1) == EINVAL
    assert lanes(lc, t=1 << 32) == EUNSUP
    assert lanes(lc, t=0, x=None, wk=None, wg=None, a=None, gl=None) == 0


def test_trace_calls(L):
    K.dsv4_trace_reset()
    assert K.dsv4_trace_read("") == (0, 0.0)
    K.dsv4_trace_enable(True)
    K.dsv4_trace_enable(False)


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    cfg = K.CompCfg(ratio=4, overlap=True, dim=8, rope_dim=4, dtype=torch.float32)
    x = torch.zeros(1, 4, 16)
    with pytest.raises(ValueError):
        K.dsv4_compress_prefill(cfg, torch.zeros(1, 8, dtype=torch.uint8), x, x, [0],
                                torch.zeros(4, 16), torch.zeros(8), torch.zeros(2), torch.zeros(1, 4, 8))
