"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each pin is a plain function that raises AssertionError on failure.  They look the oracle up
through the ``oracle.csa`` module at call time so that the mutation tests can plant a
mistake in the oracle and see which pins catch it.  None of them re-derives an oracle
formula: they use closed forms, special cases that reduce to a textbook or library
routine, invariants, brute-force definitions, and integer facts printed on the pages.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from oracle import csa as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F64 = np.float64


def _rng(seed):
    return np.random.default_rng(seed)


def _inv_freq(rd, theta=160000.0):
    return (theta ** (-np.arange(0, rd, 2, dtype=np.float64) / rd)).astype(np.float32)


# ------------------------------------------------------------------ page facts (golden)
def pin_pool_rows_golden():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    r = facts["pool_rows"]["ratio"]
    for tokens, rows in facts["pool_rows"]["cases"]:
        assert O.rows_completed(tokens, r) == rows, (tokens, rows)


def pin_visibility_golden():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    r = facts["visible_rows"]["ratio"]
    for p, n in facts["visible_rows"]["cases"]:
        assert O.visible_rows(p, r) == n, (p, n)
    # the visible set is exactly the rows whose window ends at or before p
    for p in range(0, 40):
        for rr in (1, 3, 4, 128):
            nv = O.visible_rows(p, rr)
            assert nv * rr <= p + 1 < (nv + 1) * rr, (p, rr, nv)


def pin_window_golden():
    """Window span: probe with a dominant key at distance d from the query."""
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["window"]
    W = facts["window"]
    D, H = 8, 1
    p = 300
    for d, expect_seen in [(d, True) for d in facts["visible_distances"]] + \
                          [(d, False) for d in facts["hidden_distances"]]:
        kv = np.zeros((p + 1, D))
        kv[:, 0] = 1.0
        big = np.zeros(D)
        big[1] = 40.0
        kv[p - d] = big
        q = np.zeros((1, H, D))
        q[0, 0, 1] = 1.0
        o = O.csa_attention(q, kv, None, None, [p], window=W, ratio=0,
                            sinks=np.full(H, -np.inf), scale=1.0, store="f32", work=F64)
        seen = o[0, 0, 1] > 20.0
        assert seen == expect_seen, (d, o[0, 0, :2])


# ------------------------------------------------------------------ storage rounding
def pin_bf16_round_is_library_rne():
    """bf16 rounding of fp32 values equals torch's fp32 -> bfloat16 conversion (nearest,
    ties to even), including exact ties, subnormal-range and large values."""
    rng = _rng(17)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32) * 10.0,
                        np.float32([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8),
                                     2.0 ** -130, 3.0e38, 0.0, -0.0, 65504.0])]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)
    np.testing.assert_array_equal(O.round_store(x, "bf16"), ref)
    np.testing.assert_array_equal(O.round_store(np.float64(1.0) + 2.0 ** -30, "f32"), np.float32(1.0))


# ------------------------------------------------------------------ compressor
def _lanes(rng, T, r, D, overlap):
    coff = 2 if overlap else 1
    a = rng.standard_normal((T, coff * D))
    g = rng.standard_normal((T, coff * D))
    ape = rng.standard_normal((r, coff * D))
    return a, g, ape


def pin_compress_mean_pooling():
    """gate + APE constant over a row's slots -> plain mean of the slot values."""
    rng = _rng(1)
    for overlap, r in [(True, 4), (False, 4), (False, 7), (True, 3)]:
        D, T = 16, 6 * r + 2
        a, _, _ = _lanes(rng, T, r, D, overlap)
        coff = 2 if overlap else 1
        g = np.broadcast_to(rng.standard_normal(coff * D), (T, coff * D)).copy()
        # make the sum constant across slots: ape equal for all slots and both halves
        base = rng.standard_normal(D)
        g[:, :D] = base
        if overlap:
            g[:, D:] = base
        ape = np.zeros((r, coff * D))
        rows = O.compressor_rows(a, g, ape, np.ones(D), np.zeros(2, np.float32), ratio=r,
                                 overlap=overlap, eps=0.0, store="f32", work=F64)
        for j in range(T // r):
            own = a[j * r:(j + 1) * r, (D if overlap else 0):(D if overlap else 0) + D]
            vals = [own]
            if overlap and j >= 1:
                vals.append(a[(j - 1) * r:j * r, :D])
            mean = np.concatenate(vals).mean(axis=0)
            expect = mean / np.linalg.norm(mean) * np.sqrt(D)
            np.testing.assert_allclose(rows[j], expect, rtol=2e-6, atol=2e-6)


def pin_compress_dominant_slot():
    """One slot's logit far above the others -> the row is that slot's (normalised) value."""
    rng = _rng(2)
    for overlap, r in [(True, 4), (False, 4), (False, 5)]:
        D, T = 12, 5 * r
        a, g, _ = _lanes(rng, T, r, D, overlap)
        coff = 2 if overlap else 1
        g *= 0.1
        for half in range(coff):
            for s in range(r):
                ape = np.zeros((r, coff * D))
                ape[s, half * D:(half + 1) * D] = 80.0
                rows = O.compressor_rows(a, g, ape, np.ones(D), np.zeros(2, np.float32),
                                         ratio=r, overlap=overlap, eps=0.0, store="f32",
                                         work=F64)
                for j in range(T // r):
                    if overlap and half == 0:
                        if j == 0:
                            continue            # previous window absent for row 0
                        t = (j - 1) * r + s
                    else:
                        t = j * r + s
                    v = a[t, half * D:(half + 1) * D]
                    expect = v / np.linalg.norm(v) * np.sqrt(D)
                    np.testing.assert_allclose(rows[j], expect, rtol=1e-5, atol=1e-5,
                                               err_msg=f"ov={overlap} half={half} s={s} j={j}")


def pin_compress_ratio1_closed_form():
    """r = 1, no overlap: row t = RoPE(RMSNorm(a_t) * gamma) at position t.

    The expectation uses complex rotation (x0 + i x1) * exp(i t w_i) and the 2-norm.
    """
    rng = _rng(3)
    D, rd, T, eps = 16, 8, 9, 1e-3
    a = rng.standard_normal((T, D))
    g = rng.standard_normal((T, D))
    ape = rng.standard_normal((1, D))
    gamma = rng.standard_normal(D)
    inv = _inv_freq(rd, theta=10.0)
    rows = O.compressor_rows(a, g, ape, gamma, inv, ratio=1, overlap=False, eps=eps,
                             store="f32", work=F64)
    for t in range(T):
        y = a[t] / np.sqrt(np.linalg.norm(a[t]) ** 2 / D + eps) * gamma
        z = y[D - rd::2] + 1j * y[D - rd + 1::2]
        theta = (np.float32(t) * inv).astype(np.float32).astype(np.float64)
        z = z * np.exp(1j * theta)
        expect = y.copy()
        expect[D - rd::2] = z.real
        expect[D - rd + 1::2] = z.imag
        np.testing.assert_allclose(rows[t], expect, rtol=3e-6, atol=3e-6)


def pin_compress_row_purity():
    """A row is a function of its own window (and, overlapping, the previous one) only."""
    rng = _rng(4)
    for overlap, r in [(True, 4), (False, 4), (False, 3)]:
        D, T = 8, 8 * r
        a, g, ape = _lanes(rng, T, r, D, overlap)
        gamma = rng.standard_normal(D)
        inv = _inv_freq(4)
        kw = dict(ratio=r, overlap=overlap, eps=1e-6, store="f32", work=F64)
        base = O.compressor_rows(a, g, ape, gamma, inv, **kw)
        j = 4
        lo = (j - 1) * r if overlap else j * r
        hi = (j + 1) * r
        for t in range(T):
            a2, g2 = a.copy(), g.copy()
            a2[t] += 3.0
            g2[t] -= 2.0
            row = O.compressor_rows(a2, g2, ape, gamma, inv, **kw)[j]
            if lo <= t < hi:
                assert not np.array_equal(row, base[j]), (overlap, t)
            else:
                assert np.array_equal(row, base[j]), (overlap, t)


def pin_compress_prefix_invariance():
    """Rows from a prefix of the lane equal the first rows from the whole lane."""
    rng = _rng(5)
    D, r, T = 8, 4, 41
    a, g, ape = _lanes(rng, T, r, D, True)
    gamma = rng.standard_normal(D)
    inv = _inv_freq(4)
    kw = dict(ratio=r, overlap=True, eps=1e-6, store="bf16")
    full = O.compressor_rows(a, g, ape, gamma, inv, **kw)
    for T2 in (4, 7, 8, 23, 40):
        part = O.compressor_rows(a[:T2], g[:T2], ape, gamma, inv, **kw)
        assert np.array_equal(part, full[:T2 // r])


def pin_compress_lane_slice_with_token0():
    """Rows computed from a slice of the lane that starts at token t0 (``token0=t0`` and a
    ``rows=`` subset) equal the same rows of the whole-lane call, bit for bit: overlapping
    and plain windows, t0 on and off a window boundary, ordered and unordered subsets."""
    rng = _rng(31)
    D = 8
    for overlap, r in [(True, 4), (False, 4), (True, 3), (False, 5)]:
        T = 12 * r + 3
        a, g, ape = _lanes(rng, T, r, D, overlap)
        gamma = rng.standard_normal(D)
        inv = _inv_freq(4)
        kw = dict(ratio=r, overlap=overlap, eps=1e-6, store="bf16")
        full = O.compressor_rows(a, g, ape, gamma, inv, **kw)
        for t0 in (1, r, r + 1, 2 * r - 1, 5 * r + 2):
            first = -(-t0 // r) + (1 if overlap else 0)    # first row with every slot at or after t0
            js = list(range(first, T // r))
            part = O.compressor_rows(a[t0:], g[t0:], ape, gamma, inv, rows=js, token0=t0, **kw)
            assert np.array_equal(part, full[js]), (overlap, r, t0)
            sub = js[::-3]
            part = O.compressor_rows(a[t0:], g[t0:], ape, gamma, inv, rows=sub, token0=t0, **kw)
            assert np.array_equal(part, full[sub]), (overlap, r, t0, sub)


def pin_compress_bf16_rounding_points():
    """bf16 storage at r = 1 (one slot: the pooled value is the token's own value):
    row t = bf16(RoPE_t(bf16(RMSNorm(bf16(a_t)) * gamma))), each rounding torch's
    fp32 -> bfloat16 conversion, at exactly the three points the storage rule names (the
    pooled value before the norm, the normed row, the rotated row).  The norm and the rotation
    are taken in fp64 here (torch), so only the rounding points decide the bits."""
    rng = _rng(33)
    T, D, rd, eps = 24, 32, 16, 1e-6
    a = rng.standard_normal((T, D)) * 3.0
    g = rng.standard_normal((T, D))
    ape = rng.standard_normal((1, D))
    gamma = rng.standard_normal(D)
    inv = _inv_freq(rd, theta=10.0)
    rows = O.compressor_rows(a, g, ape, gamma, inv, ratio=1, overlap=False, eps=eps, store="bf16",
                             work=F64)

    def bf(x):
        return torch.as_tensor(x, dtype=torch.float64).float().bfloat16().double()

    def closed_form(t, round_pooled=True):
        y = bf(a[t]) if round_pooled else torch.as_tensor(a[t], dtype=torch.float64)
        y = bf(y / torch.sqrt(torch.linalg.vector_norm(y) ** 2 / D + eps) * torch.as_tensor(gamma))
        th = torch.as_tensor(np.float32(t) * inv, dtype=torch.float32).double()   # fp32 angle
        z = torch.complex(y[D - rd::2], y[D - rd + 1::2]) * torch.polar(torch.ones_like(th), th)
        out = y.clone()
        out[D - rd::2] = z.real
        out[D - rd + 1::2] = z.imag
        return bf(out).numpy()

    differs = 0
    for t in range(T):
        expect = closed_form(t)
        assert np.array_equal(rows[t], expect), (t, np.abs(rows[t] - expect).max())
        differs += int((closed_form(t, round_pooled=False) != expect).any())
    assert differs > T // 2            # the data is such that the first rounding point shows


def pin_compress_softmax_is_convex():
    """Pooled values lie inside the range of the slot values (softmax weights are a convex
    mix).  A huge eps makes the RMSNorm a fixed scale 1/sqrt(eps), so the pooled value is
    read back from the row; zero frequencies make the RoPE the identity."""
    rng = _rng(6)
    D, r, T, eps = 8, 4, 32, 1e12
    for overlap in (True, False):
        a, g, ape = _lanes(rng, T, r, D, overlap)
        g *= 3.0
        rows = O.compressor_rows(a, g, ape, np.ones(D), np.zeros(2, np.float32), ratio=r,
                                 overlap=overlap, eps=eps, store="f32", work=F64)
        pooled = rows * np.sqrt(eps)
        for j in range(T // r):
            h = D if overlap else 0
            vals = [a[j * r:(j + 1) * r, h:h + D]]
            if overlap and j >= 1:
                vals.append(a[(j - 1) * r:j * r, :D])
            v = np.concatenate(vals)
            assert np.all(pooled[j] <= v.max(0) + 1e-5) and np.all(pooled[j] >= v.min(0) - 1e-5)
            assert not np.allclose(pooled[j], v.mean(0), atol=1e-3)   # gating is not a mean


# ------------------------------------------------------------------ RoPE
def pin_rope_properties():
    rng = _rng(7)
    D, rd, n = 12, 8, 6
    inv = _inv_freq(rd, theta=100.0)
    x = rng.standard_normal((n, D))
    y = rng.standard_normal((n, D))
    pos = np.array([0, 1, 5, 17, 100, 1000], dtype=np.float64)
    rx = O.rope_rows(x, pos, inv, F64)
    # untouched leading dims; pair norms preserved; position 0 is the identity
    assert np.array_equal(rx[:, :D - rd], x[:, :D - rd])
    pn = lambda v: v[:, D - rd::2] ** 2 + v[:, D - rd + 1::2] ** 2
    np.testing.assert_allclose(pn(rx), pn(x), rtol=1e-6)
    np.testing.assert_allclose(rx[0], x[0], rtol=0, atol=0)
    # R(-p) R(p) = I
    back = O.rope_rows(rx, -pos, inv, F64)
    np.testing.assert_allclose(back, x, rtol=1e-6, atol=1e-6)
    # rotated dot products depend on the position difference only
    p, q = 37.0, 11.0
    a = O.rope_rows(x[:1], [p], inv, F64)[0, D - rd:]
    b = O.rope_rows(y[:1], [q], inv, F64)[0, D - rd:]
    c = O.rope_rows(x[:1], [p - q], inv, F64)[0, D - rd:]
    np.testing.assert_allclose(a @ b, c @ y[0, D - rd:], rtol=1e-5)
    # the first pair turns by p * inv[0] radians, counter-clockwise
    e = np.zeros((1, D))
    e[0, D - rd] = 1.0
    r1 = O.rope_rows(e, [0.5], inv, F64)[0]
    th = float(np.float32(0.5) * inv[0])
    np.testing.assert_allclose(r1[D - rd:D - rd + 2], [np.cos(th), np.sin(th)], atol=1e-7)


# ------------------------------------------------------------------ indexer
def pin_index_scale_closed_form():
    for Hi, di in [(1, 16), (2, 32), (4, 8), (64, 128)]:
        qi = np.zeros((1, Hi, di))
        qi[0, :, 0] = 1.0
        K = np.zeros((1, di))
        K[0, 0] = 1.0
        w = np.ones((1, Hi))
        s = O.index_scores(qi, w, K, F64)
        np.testing.assert_allclose(s[0, 0], Hi * di ** -0.5 * Hi ** -0.5, rtol=1e-12)


def pin_index_heads_add():
    """Score with H heads = H^-1/2 * sum of single-head scores (a sum over heads)."""
    rng = _rng(8)
    S, Hi, di, N = 3, 4, 16, 20
    qi = rng.standard_normal((S, Hi, di))
    w = rng.standard_normal((S, Hi))
    K = rng.standard_normal((N, di))
    full = O.index_scores(qi, w, K, F64)
    parts = sum(O.index_scores(qi[:, h:h + 1], w[:, h:h + 1], K, F64) for h in range(Hi))
    np.testing.assert_allclose(full, parts * Hi ** -0.5, rtol=1e-10, atol=1e-12)


def pin_index_relu():
    """A head whose dot product is negative contributes nothing."""
    rng = _rng(9)
    di = 8
    k = rng.standard_normal(di)
    qi = np.stack([k, -k])[None]                 # [1, 2, di]: dot = +|k|^2 and -|k|^2
    w = np.array([[1.0, 5.0]])
    s = O.index_scores(qi, w, k[None], F64)[0, 0]
    np.testing.assert_allclose(s, k @ k * di ** -0.5 * 2 ** -0.5, rtol=1e-10)


def _check_topk_definition(scores, positions, r, k, sel):
    for i, p in enumerate(positions):
        nv = min(O.visible_rows(p, r), scores.shape[1])
        chosen = [int(x) for x in sel[i] if x >= 0]
        assert list(sel[i, len(chosen):]) == [-1] * (k - len(chosen))
        assert chosen == sorted(set(chosen)), "ascending, no duplicates"
        assert len(chosen) == min(k, nv)
        assert all(0 <= j < nv for j in chosen)
        rest = [j for j in range(nv) if j not in set(chosen)]
        for a in chosen:
            for b in rest:
                sa, sb = float(scores[i, a]), float(scores[i, b])
                assert sa > sb or (sa == sb and a < b), (p, a, b, sa, sb)


def pin_topk_definition_bruteforce():
    """Every selected row beats every unselected visible row by (score desc, index asc)."""
    rng = _rng(10)
    N, k, r = 40, 6, 4
    positions = list(range(0, 4 * N, 3))
    scores = np.round(rng.standard_normal((len(positions), N)), 1)    # many exact ties
    scores[:, ::5] = 0.0
    scores[::2, 1::7] = -0.0
    sel = O.select_topk(scores, positions, ratio=r, k=k)
    _check_topk_definition(scores, positions, r, k, sel)


def pin_topk_single_head_is_mips():
    """H_i = 1 with a positive weight: the selection is maximum inner-product search."""
    rng = _rng(11)
    N, di, k = 30, 8, 5
    K = rng.standard_normal((N, di))
    q = rng.standard_normal((1, 1, di))
    w = np.array([[2.0]])
    p = 4 * N - 1                                     # all rows visible at ratio 4
    sel = O.select_topk(O.index_scores(q, w, K, F64), [p], ratio=4, k=k)[0]
    dots = K @ q[0, 0]
    expect = sorted(range(N), key=lambda j: (-max(dots[j], 0.0), j))[:k]
    assert list(sel) == sorted(expect)


def pin_topk_dense_regime():
    scores = np.arange(10, dtype=np.float64)[None, :].repeat(3, 0)
    sel = O.select_topk(scores, [3, 19, 39], ratio=4, k=8)
    assert list(sel[0]) == [0] + [-1] * 7
    assert list(sel[1]) == [0, 1, 2, 3, 4] + [-1] * 3
    assert list(sel[2]) == [2, 3, 4, 5, 6, 7, 8, 9]


# ------------------------------------------------------------------ attention
def pin_attention_is_sdpa_without_sinks():
    """No sinks, window covering everything, no compressed lane: textbook causal attention."""
    rng = _rng(12)
    S, H, D = 9, 3, 16
    q = rng.standard_normal((S, H, D))
    kv = rng.standard_normal((S, D))
    scale = D ** -0.5
    o = O.csa_attention(q, kv, None, None, list(range(S)), window=S + 5, ratio=0,
                        sinks=np.full(H, -np.inf), scale=scale, store="f32", work=F64)
    qt = torch.tensor(q, dtype=torch.float64).permute(1, 0, 2)      # [H, S, D]
    kt = torch.tensor(kv, dtype=torch.float64)[None].expand(H, S, D).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, is_causal=True,
                                                           scale=scale)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-6, atol=1e-6)


def pin_attention_sink_closed_form():
    """All keys equal x: o = (1 - pi) x with pi = 1 / (1 + n e^(l - z))."""
    rng = _rng(13)
    H, D, W = 4, 8, 5
    x = rng.standard_normal(D)
    kv = np.broadcast_to(x, (12, D)).copy()
    q = rng.standard_normal((1, H, D))
    sinks = np.array([-1.0, 0.0, 2.5, 30.0])
    scale = 0.3
    p = 11
    o = O.csa_attention(q, kv, None, None, [p], window=W, ratio=0, sinks=sinks,
                        scale=scale, store="f32", work=F64)[0]
    for h in range(H):
        l = scale * q[0, h] @ x
        pi = 1.0 / (1.0 + W * np.exp(l - sinks[h]))
        np.testing.assert_allclose(o[h], (1 - pi) * x, rtol=1e-6, atol=1e-7)


def pin_attention_sink_scales_output():
    """A sink only rescales the sink-free output by a per-head factor in (0, 1)."""
    rng = _rng(14)
    S, H, D, W, r = 3, 2, 8, 6, 4
    kv = rng.standard_normal((40, D))
    rows = rng.standard_normal((9, D))
    q = rng.standard_normal((S, H, D))
    pos = [20, 30, 39]
    kw = dict(window=W, ratio=r, scale=0.5, store="f32", work=F64)
    a = O.csa_attention(q, kv, rows, None, pos, sinks=np.array([0.7, -0.3]), **kw)
    b = O.csa_attention(q, kv, rows, None, pos, sinks=np.full(H, -np.inf), **kw)
    f = a / b
    for i in range(S):
        for h in range(H):
            assert np.allclose(f[i, h], f[i, h, 0], rtol=1e-6)
            assert 0.0 < f[i, h, 0] < 1.0


def pin_attention_rows_and_sparse_equal_dense():
    """Selecting every visible row (k >= n) equals dense attention over window + rows;
    a dominant invisible row has no effect; a dominant visible row takes over."""
    rng = _rng(15)
    S, H, D, W, r = 4, 2, 8, 5, 4
    kv = rng.standard_normal((64, D))
    rows = rng.standard_normal((16, D))
    q = rng.standard_normal((S, H, D))
    pos = [6, 17, 35, 63]
    kw = dict(window=W, ratio=r, sinks=np.array([0.1, -0.2]), scale=0.4, store="f32",
              work=F64)
    dense = O.csa_attention(q, kv, rows, None, pos, **kw)
    sel = np.full((S, 32), -1)
    for i, p in enumerate(pos):
        nv = O.visible_rows(p, r)
        sel[i, :nv] = np.arange(nv)
    sparse = O.csa_attention(q, kv, rows, sel, pos, **kw)
    np.testing.assert_allclose(sparse, dense, rtol=1e-12, atol=1e-12)
    # the same sets in another order with -1 entries between them
    ragged = np.full((S, 40), -1)
    for i, p in enumerate(pos):
        nv = O.visible_rows(p, r)
        ragged[i, 1:2 * nv + 1:2] = np.arange(nv)[::-1]
    np.testing.assert_allclose(O.csa_attention(q, kv, rows, ragged, pos, **kw), dense,
                               rtol=1e-12, atol=1e-12)
    # dominance probes around the visibility edge of query p = 17 (4 rows visible)
    q1 = np.zeros((1, 1, D))
    q1[0, 0, 0] = 1.0
    kw1 = dict(window=W, ratio=r, sinks=np.full(1, -np.inf), scale=1.0, store="f32",
               work=F64)
    for j, expect in [(3, True), (4, False)]:
        rr = np.zeros((16, D))
        rr[j, 0] = 50.0
        o = O.csa_attention(q1, np.zeros((64, D)), rr, None, [17], **kw1)
        assert (o[0, 0, 0] > 25.0) == expect, (j, o[0, 0, 0])


def pin_attention_kv_slice_with_offset():
    """kv handed over from token lo on (``kv_offset=lo``) equals the call with the whole kv,
    bit for bit, for queries whose window lies inside the slice (including one whose window
    starts exactly at lo)."""
    rng = _rng(32)
    H, D, W, r = 2, 8, 6, 4
    kv = rng.standard_normal((60, D))
    rows = rng.standard_normal((15, D))
    pos = [20, 33, 40, 59, 59]
    q = rng.standard_normal((len(pos), H, D))
    kw = dict(window=W, ratio=r, sinks=np.array([0.3, -1.1]), scale=0.4, store="f32", work=F64)
    for sel in (None, np.array([[0, 2, -1], [1, 6, 7], [-1, 3, 9], [0, 13, 14], [14, -1, -1]])):
        full = O.csa_attention(q, kv, rows, sel, pos, **kw)
        for lo in (1, 7, 15):
            part = O.csa_attention(q, kv[lo:], rows, sel, pos, kv_offset=lo, **kw)
            assert np.array_equal(part, full), lo


def pin_fp32_work_within_rounding_bound():
    """The fp32 working precision (pooling, scoring, softmax) stays within a small multiple of
    fp32 rounding of the same computation in fp64: the error of an fp32 sum of n terms is
    bounded by about n * 2^-24 of the sum of magnitudes."""
    rng = _rng(34)
    D, r, T = 64, 4, 48
    a, g, ape = _lanes(rng, T, r, D, True)
    gamma, inv = rng.standard_normal(D), _inv_freq(16)
    kw = dict(ratio=r, overlap=True, eps=1e-6, store="f32")
    r32 = O.compressor_rows(a, g, ape, gamma, inv, **kw)
    r64 = O.compressor_rows(a, g, ape, gamma, inv, work=F64, **kw)
    assert np.abs(r32 - r64).max() <= 1e-5 * np.abs(r64).max()
    qi, w, Kr = rng.standard_normal((3, 4, 32)), rng.standard_normal((3, 4)), rng.standard_normal((50, 32))
    s32, s64 = O.index_scores(qi, w, Kr), O.index_scores(qi, w, Kr, F64)
    assert np.abs(s32 - s64).max() <= 1e-5 * np.abs(s64).max()
    q, kv = rng.standard_normal((4, 3, D)), rng.standard_normal((40, D))
    pos = [10, 20, 30, 39]
    akw = dict(window=8, ratio=r, sinks=rng.standard_normal(3), scale=D ** -0.5, store="f32")
    o32 = O.csa_attention(q, kv, r64, None, pos, **akw)
    o64 = O.csa_attention(q, kv, r64, None, pos, work=F64, **akw)
    assert (np.abs(o32 - o64).max(-1) / np.abs(o64).max(-1)).max() <= 1e-5


def pin_attention_bruteforce_layer():
    """A tiny layer end to end, top-k covering all rows, against a direct softmax formula
    over the window and every visible compressed row, computed key by key."""
    rng = _rng(16)
    T, H, D, W, r, Hi, di = 24, 2, 8, 4, 4, 2, 4
    kv = rng.standard_normal((T, D))
    a = rng.standard_normal((T, 2 * D))
    g = rng.standard_normal((T, 2 * D))
    ape = rng.standard_normal((r, 2 * D))
    gamma = rng.standard_normal(D)
    inv = _inv_freq(4)
    rows = O.compressor_rows(a, g, ape, gamma, inv, ratio=r, overlap=True, eps=1e-6,
                             store="f32", work=F64)
    qi = rng.standard_normal((T, Hi, di))
    w = rng.standard_normal((T, Hi))
    K = rng.standard_normal((rows.shape[0], di))
    pos = list(range(T))
    sel = O.select_topk(O.index_scores(qi, w, K, F64), pos, ratio=r, k=64)
    q = rng.standard_normal((T, H, D))
    sinks = rng.standard_normal(H)
    out = O.csa_attention(q, kv, rows, sel, pos, window=W, ratio=r, sinks=sinks, scale=0.35,
                          store="f32", work=F64)
    for p in pos:
        keys = [kv[t] for t in range(max(0, p - W + 1), p + 1)]
        keys += [rows[j] for j in range(rows.shape[0]) if (j + 1) * r <= p + 1]
        for h in range(H):
            num = np.zeros(D)
            den = np.exp(sinks[h])
            for x in keys:
                e = np.exp(0.35 * float(q[p, h] @ x))
                num += e * x
                den += e
            np.testing.assert_allclose(out[p, h], num / den, rtol=2e-6, atol=2e-7)


# ------------------------------------------------------------------ output path
def pin_rope_heads_inverse_and_heads():
    """Every head of a token turns by the token's angle; the inverse undoes the forward;
    a one-hot pair turns back clockwise by exactly that angle."""
    rng = _rng(21)
    N, H, D, rd = 5, 3, 10, 6
    inv = _inv_freq(rd, theta=50.0)
    x = rng.standard_normal((N, H, D))
    pos = np.array([0, 3, 9, 40, 1000], dtype=np.float64)
    f = O.rope_heads(x, pos, inv, work=F64)
    for h in range(H):                                   # heads are independent rows
        np.testing.assert_array_equal(f[:, h], O.rope_rows(x[:, h], pos, inv, F64))
    np.testing.assert_allclose(O.rope_heads(f, pos, inv, inverse=True, work=F64), x,
                               rtol=1e-9, atol=1e-9)
    np.testing.assert_array_equal(f[0], x[0])            # position 0
    e = np.zeros((1, 1, D))
    e[0, 0, D - rd + 2] = 1.0                            # pair 1, first component
    th = float(np.float32(7.0) * inv[1])
    b = O.rope_heads(e, [7.0], inv, inverse=True, work=F64)[0, 0, D - rd + 2:D - rd + 4]
    np.testing.assert_allclose(b, [np.cos(th), -np.sin(th)], atol=1e-12)


def pin_grouped_proj_is_block_diagonal():
    """The grouped projection equals one dense matmul with the block-diagonal weight written
    out (zeros off the blocks); one group is a plain matmul; a one-hot input picks one
    weight column of its own group only."""
    rng = _rng(22)
    N, H, D, G, R = 4, 6, 5, 3, 7
    o = rng.standard_normal((N, H, D))
    w = rng.standard_normal((G, R, H // G * D))
    y = O.grouped_out_proj(o, w)
    dense = np.zeros((G * R, H * D))
    for g in range(G):
        dense[g * R:(g + 1) * R, g * (H // G) * D:(g + 1) * (H // G) * D] = w[g]
    np.testing.assert_allclose(y, o.reshape(N, H * D) @ dense.T, rtol=1e-12, atol=1e-12)
    w1 = rng.standard_normal((1, R, H * D))
    np.testing.assert_allclose(O.grouped_out_proj(o, w1), np.matmul(o.reshape(N, H * D), w1[0].T),
                               rtol=1e-12, atol=1e-12)
    e = np.zeros((1, H, D))
    h, d = 3, 2                                          # head 3 is in group 1 (2 heads per group)
    e[0, h, d] = 1.0
    ye = O.grouped_out_proj(e, w)[0]
    np.testing.assert_array_equal(ye[:R], 0.0)
    np.testing.assert_array_equal(ye[2 * R:], 0.0)
    np.testing.assert_array_equal(ye[R:2 * R], w[1][:, (h - 2) * D + d])


ALL_PINS = {name: fn for name, fn in sorted(globals().items())
            if name.startswith("pin_") and callable(fn)}
