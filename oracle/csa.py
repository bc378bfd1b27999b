"""Oracle for the CSA layer: compressor, indexer, sparse MQA attention with sinks.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's CPU baseline.
Never on the product path.

Sources ("the pages"):
  [MTPLX-216]  MTPLX PR #216 "DeepSeek-V4-Flash: native deepseek_v4 AR backend" and its
               follow-up comments (sections: "What V4 adds", "Verification", "Decode path:
               reference-faithful bf16 activation storage", "Decode dispatch reduction").
  [MLXLM-1189] mlx-lm PR #1189 "feat: add DeepSeek-V4 (Pro/Flash) model support" and its
               review thread (Thump604's fix list; OmarB97's RoPE/visibility notes;
               aidiffuser's mask diagnosis; stepnoy's patch; aidiffuser's indexer path;
               stepnoy's index-space fix).
  [V41-MLX]    "deepseek-v41-mlx" (section "Why this exists": the landmines kept from V4).

Readings where the pages leave a step open are marked READING.
Every parity claim of the HIP path is against these functions.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round", "round_store", "rope_rows", "rms_norm", "compressor_rows",
    "rows_completed", "visible_rows", "index_scores", "select_topk", "csa_attention",
    "rope_heads", "grouped_out_proj",
]


# --------------------------------------------------------------------------------------
# Storage rounding
# --------------------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float64.

    The value is first rounded to fp32, then the low 16 bits of the fp32 pattern are
    rounded away (nearest, ties to even).  Finite inputs only.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_store(x, store: str) -> np.ndarray:
    """Round to the storage dtype: ``"bf16"`` or ``"f32"``; returned as float64.

    [MTPLX-216] "Decode path: reference-faithful bf16 activation storage": activations and
    KV are stored at the model dtype (bf16) while pooling, softmax and accumulation run in
    fp32.  In fp32 mode storage is fp32.
    """
    if store == "bf16":
        return bf16_round(x)
    if store == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {store!r}")


# --------------------------------------------------------------------------------------
# Row RoPE and RMSNorm
# --------------------------------------------------------------------------------------
def rope_rows(x: np.ndarray, positions, inv_freq, work=np.float32) -> np.ndarray:
    """Rotate the LAST ``2*len(inv_freq)`` dims of each row of ``x`` at its position.

    [MLXLM-1189] stepnoy's patch, ``apply_positions``: interleaved pairs (x0, x1) = (x[2i],
    x[2i+1]) of the rotary slice, angle theta_i = position * inv_freq[i] formed in fp32,
    result (x0 cos - x1 sin, x0 sin + x1 cos); OmarB97 note 2: the rotary dims are the last
    ``rd`` of the row.  Non-rotary dims pass through.

    x: [N, D]; positions: [N]; inv_freq: [rd/2] fp32.  Returns float64 (not rounded).
    """
    x = np.asarray(x, dtype=np.float64)
    inv = np.asarray(inv_freq, dtype=np.float32)
    rd = 2 * inv.shape[0]
    n, d = x.shape
    assert rd <= d and rd % 2 == 0
    pos = np.asarray(positions, dtype=np.float32).reshape(n, 1)
    theta = (pos * inv[None, :]).astype(np.float32)          # fp32 product, as on the pages
    c = np.cos(theta.astype(work))
    s = np.sin(theta.astype(work))
    out = x.copy()
    x0 = x[:, d - rd + 0::2].astype(work)
    x1 = x[:, d - rd + 1::2].astype(work)
    out[:, d - rd + 0::2] = x0 * c - x1 * s
    out[:, d - rd + 1::2] = x0 * s + x1 * c
    return out


def rms_norm(y: np.ndarray, gamma, eps: float, work=np.float32) -> np.ndarray:
    """y / sqrt(mean(y^2) + eps) * gamma over the last axis, in the working precision.

    [MTPLX-216] "Decode path" comment: the compressor casts the pooled row back to the
    storage dtype before its RMSNorm.
    READING: the standard RMSNorm with a learned per-channel gain; eps is a parameter.
    """
    y = np.asarray(y, dtype=work)
    g = np.asarray(gamma, dtype=work)
    ms = np.mean(y * y, axis=-1, keepdims=True, dtype=work)
    return (y / np.sqrt(ms + work(eps)) * g).astype(np.float64)


# --------------------------------------------------------------------------------------
# Compressor
# --------------------------------------------------------------------------------------
def rows_completed(n_tokens: int, ratio: int) -> int:
    """Rows in a compressed lane after ``n_tokens`` tokens: one per completed window.

    [MLXLM-1189] stepnoy's index-space fix: a 6042-token prompt holds 1510 pool rows at
    ratio 4, and the fixed ladder's pool-row column is floor(tokens / 4).
    """
    return n_tokens // ratio


def compressor_rows(a, g, ape, gamma, inv_freq, *, ratio: int, overlap: bool, eps: float,
                    store: str, work=np.float32, rows=None, token0: int = 0) -> np.ndarray:
    """Compressed rows of one sequence from its kv lane ``a`` and gate lane ``g``.

    [MTPLX-216] "What V4 adds": besides the sliding window, each such layer caches rows that
    each summarise one window of tokens by learned gated pooling; at ratio 4 a window also
    reaches back over its predecessor, at ratio 128 the windows are disjoint.
    [MLXLM-1189] Thump604's fixes: ratio-4 shapes ape (4, 1024), wkv/wgate (1024, 4096), i.e.
    the overlapping compressor's lanes are 2*D wide; aidiffuser's indexer path: with overlap
    a row also pools the window before its own, and the first row's missing predecessor
    counts as logit -inf, value 0.
    [MTPLX-216] "Decode path": pooling runs in fp32 and the row is cast back to the storage
    dtype before the norm; [MLXLM-1189] OmarB97 note 2: each pooled row is RoPE'd at its
    window-start position j*r before it is cached.

    For row j and channel c in [0, D):
      * own window (always): slots s in [0, r) take token t = j*r + s with value
        a[t, h*D + c] and logit g[t, h*D + c] + ape[s, h*D + c], where h = 1 when
        overlapping and h = 0 otherwise;
      * previous window (overlap only): slots s in [0, r) take token t = (j-1)*r + s with
        value a[t, c] and logit g[t, c] + ape[s, c]; absent for j = 0 (logit -inf, value 0).
      READING: half 0 of the 2*D-wide lane feeds the previous window, half 1 the own window.
    pooled[c] = sum_s softmax_s(logit)[s] * value[s]           (work precision)
    y = store(pooled);  y = store(RMSNorm(y) * gamma);  y = store(RoPE_last_rd(y, j*r)).

    a, g: [T, coff*D], entry i holding absolute token ``token0 + i``; ape: [r, coff*D];
    gamma: [D]; inv_freq: [rd/2].  ``rows``: iterable of row indices (default: all
    completed rows when ``token0 == 0``).  Returns float64 [len(rows), D].
    """
    a = np.asarray(a, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    ape = np.asarray(ape, dtype=np.float64)
    r = int(ratio)
    coff = 2 if overlap else 1
    T, width = a.shape
    assert width % coff == 0
    D = width // coff
    assert ape.shape == (r, width)
    if rows is None:
        assert token0 == 0
        rows = range(rows_completed(T, r))
    rows = np.asarray(list(rows), dtype=np.int64)
    assert np.all((rows + 1) * r <= token0 + T), "row needs tokens beyond the lane"
    first = rows * r - (r if overlap else 0)
    assert np.all((first < 0) | (first >= token0)), "row needs tokens before the lane"
    n = rows.shape[0]
    if n == 0:
        return np.zeros((0, D))

    logits, values = [], []
    own = D if overlap else 0
    for s in range(r):                       # own window, half ``own``
        t = rows * r + s - token0
        logits.append(g[t, own:own + D] + ape[s, own:own + D][None, :])
        values.append(a[t, own:own + D])
    if overlap:                               # previous window, half 0
        for s in range(r):
            t = (rows - 1) * r + s - token0
            present = (rows >= 1)[:, None]
            tt = np.where(rows >= 1, t, 0)
            logits.append(np.where(present, g[tt, 0:D] + ape[s, 0:D][None, :], -np.inf))
            values.append(np.where(present, a[tt, 0:D], 0.0))
    L = np.stack(logits).astype(work)        # [slots, n, D]; the gate sum is formed in fp32
    V = np.stack(values).astype(work)
    m = L.max(axis=0)
    e = np.exp(L - m[None])
    w = e / e.sum(axis=0, dtype=work)[None]
    pooled = (w * V).sum(axis=0, dtype=work)
    y = round_store(pooled, store)
    y = round_store(rms_norm(y, gamma, eps, work), store)
    y = round_store(rope_rows(y, rows * r, inv_freq, work), store)
    return y


# --------------------------------------------------------------------------------------
# Visibility and the indexer
# --------------------------------------------------------------------------------------
def visible_rows(p: int, ratio: int) -> int:
    """Number of compressed rows a query at absolute position ``p`` may see.

    [MLXLM-1189] aidiffuser's mask diagnosis / stepnoy's patch: row j pools raw tokens
    [j*r, (j+1)*r - 1] and is visible to the query at p iff (j+1)*r <= p+1.  The visible
    set is therefore the prefix j < (p+1) // r (OmarB97 note 3 states this form).
    """
    return (int(p) + 1) // int(ratio)


def index_scores(qi, w, K, work=np.float32) -> np.ndarray:
    """Indexer scores of every row for every query.

    [MLXLM-1189] stepnoy's patch ("Reference scoring") and aidiffuser's indexer path:
    score(p, j) = sum_h w_h(p) * (d_i^-1/2 * H_i^-1/2) * relu(q_h(p) . K_j), with the raw
    weights_proj output (no sigmoid), the scale folded into the weights, ReLU on the
    logits, a SUM over heads, all in fp32.

    qi: [S, H_i, d_i]; w: [S, H_i]; K: [N, d_i].  Returns [S, N] in ``work`` precision.
    """
    qi = np.asarray(qi, dtype=work)
    w = np.asarray(w, dtype=work)
    K = np.asarray(K, dtype=work)
    S, Hi, di = qi.shape
    scale = work(di) ** work(-0.5) * work(Hi) ** work(-0.5)
    dots = np.matmul(qi, K.T.copy())                         # [S, H_i, N]
    hw = (w * scale)[:, :, None]
    return (hw * np.maximum(dots, work(0))).sum(axis=1, dtype=work)


def select_topk(scores, positions, *, ratio: int, k: int) -> np.ndarray:
    """Per-query selected rows: ascending row indices, padded with -1 to width k.

    [MTPLX-216] "What V4 adds": the top-k filter engages once compressed positions exceed
    index_topk; [MLXLM-1189] stepnoy's patch: causality is applied BEFORE ranking.
    Selected set of query p: all visible rows when there are at most k of them; otherwise
    the first k visible rows in the order (score descending, row index ascending).
    READING: ties go to the lower row index; -0.0 equals +0.0 (compared as numbers).

    scores: [S, N]; positions: [S].  Returns int32 [S, k].
    """
    scores = np.asarray(scores)
    S = scores.shape[0]
    out = np.full((S, k), -1, dtype=np.int32)
    for i in range(S):
        nv = min(visible_rows(positions[i], ratio), scores.shape[1])
        if nv <= k:
            chosen = np.arange(nv)
        else:
            s = scores[i, :nv].astype(np.float64)
            order = np.lexsort((np.arange(nv), -s))          # by -score, then by index
            chosen = np.sort(order[:k])
        out[i, :chosen.shape[0]] = chosen
    return out


# --------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------
def csa_attention(q, kv, rows, sel, positions, *, window: int, ratio: int, sinks,
                  scale: float, store: str, work=np.float32, kv_offset: int = 0) -> np.ndarray:
    """MQA attention of each query over its sliding window plus its compressed rows.

    [MTPLX-216] "What V4 adds" and its opening: 64 heads of queries share a single 512-wide
    latent per key position, used as key and as value; a 128-token sliding window beside the compressed lane; per-head
    sink logits.  "Decode dispatch reduction" (A): the sink is one extra all-zero-V key
    column, so it enters the softmax denominator only.  [MLXLM-1189] stepnoy's patch: the
    selected compressed rows are attended together with the window keys; visibility and
    top-k membership decide which rows.

    For query p and head h, keys X(p) = {kv_t : max(0, p-W+1) <= t <= p} plus the rows
    S(p) (``sel`` row, -1 entries skipped; ``sel=None`` means every visible row):
      l_x = scale * q_h . x;  m = max(z_h, max l);
      o_h = sum_x e^(l_x - m) x / (e^(z_h - m) + sum_x e^(l_x - m)).
    READING: the window is the W tokens ending at p, self included; a token may count both
    as a window key and inside a compressed row (no de-duplication).  The probabilities are
    not rounded before the weighted sum (the bf16 tolerance covers kernels that round them).

    q: [S, H, D]; kv: [T, D] with kv[i] the latent of token kv_offset + i; rows: [N, D] or
    None (ratio 0); sel: [S, k] int or None; positions: [S]; sinks: [H].
    Returns float64 [S, H, D] rounded to ``store``.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    sinks = np.asarray(sinks, dtype=work)
    S, H, D = q.shape
    out = np.zeros((S, H, D))
    for i in range(S):
        p = int(positions[i])
        t0 = max(0, p - window + 1)
        assert t0 - kv_offset >= 0 and p - kv_offset < kv.shape[0], "window outside kv"
        keys = [kv[t0 - kv_offset:p + 1 - kv_offset]]
        if ratio > 0 and rows is not None:
            nv = visible_rows(p, ratio)
            if sel is None:
                js = np.arange(min(nv, rows.shape[0]))
            else:
                js = np.asarray(sel[i])
                js = js[js >= 0]
                assert np.all(js < nv), "selected row not visible"
            keys.insert(0, np.asarray(rows, dtype=np.float64)[js])
        X = np.concatenate(keys, axis=0).astype(work)        # [nk, D]
        qi = q[i].astype(work)                               # [H, D]
        logits = (np.matmul(qi, X.T.copy()) * work(scale)).astype(work)   # [H, nk]
        m = np.maximum(sinks, logits.max(axis=1))
        e = np.exp(logits - m[:, None])
        denom = np.exp(sinks - m) + e.sum(axis=1, dtype=work)
        o = np.matmul(e, X) / denom[:, None]
        out[i] = round_store(o, store)
    return out


# --------------------------------------------------------------------------------------
# The layer's neighbours on either side of the attention: RoPE of the per-head inputs, and
# the output path (inverse rotation of the attention output, grouped output projection)
# --------------------------------------------------------------------------------------
def rope_heads(x, positions, inv_freq, *, inverse: bool = False, work=np.float32) -> np.ndarray:
    """RoPE of every head of every token at the token's position (q, kv, qi), or its inverse
    (the attention output).

    [MLXLM-1189] OmarB97's note 2 and stepnoy's patch: the rotary dims are the last ``rd`` of
    each head, turned in interleaved pairs by position * inv_freq (as ``rope_rows``);
    Thump604's fix list, the item on turning the attention output's rotary dims back;
    [V41-MLX] "Why this exists": the rope inverse on the attention output.  The inverse turns
    each pair back by the same angle: rotating at -position, since the fp32 angle
    fp32(-p) * inv_freq is exactly the negated fp32(p) * inv_freq.

    x: [N, H, D]; positions: [N].  Returns float64 (not rounded).
    """
    x = np.asarray(x, dtype=np.float64)
    n, h, d = x.shape
    pos = np.repeat(np.asarray(positions, dtype=np.float64), h)
    if inverse:
        pos = -pos
    return rope_rows(x.reshape(n * h, d), pos, inv_freq, work).reshape(n, h, d)


def grouped_out_proj(o, wo_a) -> np.ndarray:
    """Grouped (block-diagonal) output projection of the attention output.

    [MTPLX-216] opening ("What V4 adds"): the attention output goes through a low-rank
    projection split into 8 groups, each of rank 1024; "Decode path: reference-faithful bf16 activation
    storage", item 2: wo_a is [8192, 4096] (8 x 1024 outputs, 4096 inputs per group);
    [V41-MLX] "Why this exists": wo_a is block-diagonal.  READING: group g takes heads
    g*H/G .. (g+1)*H/G - 1 (their H/G * D values, head-major) and produces outputs
    g*R .. (g+1)*R - 1.

    o: [N, H, D] (the attention output after the inverse rotation); wo_a: [G, R, H/G * D].
    Returns [N, G * R] float64 (not rounded).
    """
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(wo_a, dtype=np.float64)
    n, h, d = o.shape
    g, r, k = w.shape
    assert h % g == 0 and k == (h // g) * d
    xo = o.reshape(n, g, k)
    return np.stack([xo[:, j] @ w[j].T for j in range(g)], axis=1).reshape(n, g * r)
