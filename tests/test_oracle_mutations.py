"""Negative controls: plant a plausible mistake in the oracle (on the CPU) and require that
at least one pin fails.  This is what makes the pins worth trusting: each mistake below is
one a transcription of the pages could plausibly make.
"""
import inspect

import numpy as np
import pytest

import oracle.csa as C
from tests.oracle_pins import ALL_PINS

_orig = {name: getattr(C, name) for name in C.__all__}


def _visibility_off_by_one(p, ratio):                 # (j+1) r <= p instead of <= p+1
    return int(p) // int(ratio)


def _window_one_longer(*args, **kw):
    kw["window"] = kw["window"] + 1
    return _orig["csa_attention"](*args, **kw)


def _window_one_shorter(*args, **kw):
    kw["window"] = max(1, kw["window"] - 1)
    return _orig["csa_attention"](*args, **kw)


def _sinks_dropped(*args, **kw):
    kw["sinks"] = np.full(np.shape(kw["sinks"]), -np.inf)
    return _orig["csa_attention"](*args, **kw)


def _sink_in_numerator(q, kv, rows, sel, positions, **kw):
    # sink column given the value of the newest token instead of an all-zero value
    o_with = _orig["csa_attention"](q, kv, rows, sel, positions, **kw)
    o_none = _orig["csa_attention"](q, kv, rows, sel, positions,
                                    **{**kw, "sinks": np.full(np.shape(kw["sinks"]), -np.inf)})
    off = kw.get("kv_offset", 0)
    newest = np.stack([np.asarray(kv)[int(p) - off] for p in positions])[:, None, :]
    frac = 1.0 - o_with / np.where(o_none == 0, 1.0, o_none)
    return o_with + frac * newest


def _tiebreak_reversed(scores, positions, *, ratio, k):
    scores = np.asarray(scores)
    out = np.full((scores.shape[0], k), -1, dtype=np.int32)
    for i, p in enumerate(positions):
        nv = min(C.visible_rows(p, ratio), scores.shape[1])
        idx = np.arange(nv)
        if nv > k:
            idx = np.sort(np.lexsort((-np.arange(nv), -scores[i, :nv]))[:k])
        out[i, :idx.shape[0]] = idx
    return out


def _causal_after_ranking(scores, positions, *, ratio, k):
    scores = np.asarray(scores)
    out = np.full((scores.shape[0], k), -1, dtype=np.int32)
    n = scores.shape[1]
    for i, p in enumerate(positions):
        nv = min(C.visible_rows(p, ratio), n)
        top = np.lexsort((np.arange(n), -scores[i]))[:min(k, n)]
        idx = np.sort(top[top < nv])
        out[i, :idx.shape[0]] = idx
    return out


def _overlap_history_lost(a, g, ape, gamma, inv_freq, **kw):
    if kw.get("overlap"):
        g = np.array(g, dtype=np.float64, copy=True)
        D = g.shape[1] // 2
        g[:, :D] = -1e30                                # previous-window slots never win
    return _orig["compressor_rows"](a, g, ape, gamma, inv_freq, **kw)


def _ape_halves_swapped(a, g, ape, gamma, inv_freq, **kw):
    if kw.get("overlap"):
        ape = np.asarray(ape)
        D = ape.shape[1] // 2
        ape = np.concatenate([ape[:, D:], ape[:, :D]], axis=1)
    return _orig["compressor_rows"](a, g, ape, gamma, inv_freq, **kw)


def _ape_slots_reversed(a, g, ape, gamma, inv_freq, **kw):
    return _orig["compressor_rows"](a, g, np.asarray(ape)[::-1], gamma, inv_freq, **kw)


def _rope_at_previous_window(x, positions, inv_freq, work=np.float32):
    return _orig["rope_rows"](x, np.asarray(positions) - 1, inv_freq, work)


def _rope_first_dims(x, positions, inv_freq, work=np.float32):
    x = np.asarray(x, dtype=np.float64)
    rd = 2 * len(inv_freq)
    flipped = x[:, ::-1].copy()
    return _orig["rope_rows"](flipped, positions, inv_freq, work)[:, ::-1]


def _norm_without_gain(y, gamma, eps, work=np.float32):
    return _orig["rms_norm"](y, np.ones_like(np.asarray(gamma)), eps, work)


def _mean_over_heads(qi, w, K, work=np.float32):
    Hi = np.shape(qi)[1]
    return _orig["index_scores"](qi, w, K, work) * (Hi ** -0.5)


def _no_relu(qi, w, K, work=np.float32):
    qi = np.asarray(qi, dtype=np.float64)
    Hi, di = qi.shape[1], qi.shape[2]
    dots = np.einsum("shd,nd->shn", qi, np.asarray(K, dtype=np.float64))
    return ((np.asarray(w)[:, :, None] * di ** -0.5 * Hi ** -0.5) * dots).sum(1)


def _sigmoid_weights(qi, w, K, work=np.float32):
    return _orig["index_scores"](qi, 1.0 / (1.0 + np.exp(-np.asarray(w))), K, work)


def _inverse_turns_forward(x, positions, inv_freq, *, inverse=False, work=np.float32):
    return _orig["rope_heads"](x, positions, inv_freq, inverse=False, work=work)


def _groups_interleaved(o, wo_a):              # head h to group h mod G
    o = np.asarray(o, dtype=np.float64)
    n, h, d = o.shape
    g = np.shape(wo_a)[0]
    perm = np.concatenate([np.arange(j, h, g) for j in range(g)])
    return _orig["grouped_out_proj"](o[:, perm], wo_a)


def _groups_reversed(o, wo_a):                 # group g takes the weight of group G-1-g
    return _orig["grouped_out_proj"](o, np.asarray(wo_a)[::-1])


def _planted(name, old, new):
    """The oracle function ``name`` compiled from its own source with one text substitution
    (the text must be there, so a planted mistake cannot silently stop applying)."""
    src = inspect.getsource(_orig[name])
    assert old in src, (name, old)
    ns = dict(vars(C))
    exec(compile(src.replace(old, new), f"<planted {name}>", "exec"), ns)
    return ns[name]


def _token0_off_by_one(a, g, ape, gamma, inv_freq, **kw):
    # a lane handed over from token t0 > 0 read one token early: entry i taken as token t0 + i - 1
    if kw.get("token0", 0):
        a, g = np.asarray(a), np.asarray(g)
        a, g = np.concatenate([a[:1], a[:-1]]), np.concatenate([g[:1], g[:-1]])
    return _orig["compressor_rows"](a, g, ape, gamma, inv_freq, **kw)


def _kv_offset_off_by_one(q, kv, rows, sel, positions, **kw):
    # kv handed over from token lo > 0 read one token late: entry i taken as token lo + i + 1
    if kw.get("kv_offset", 0):
        kv = np.asarray(kv)
        kv = np.concatenate([kv[1:], kv[-1:]])
    return _orig["csa_attention"](q, kv, rows, sel, positions, **kw)


_round_after_the_norm = _planted("compressor_rows", "y = round_store(pooled, store)",
                                 "y = np.asarray(pooled, dtype=np.float64)")


MUTATIONS = {
    "visibility (j+1)r <= p": ("visible_rows", _visibility_off_by_one),
    "window one token longer": ("csa_attention", _window_one_longer),
    "window one token shorter": ("csa_attention", _window_one_shorter),
    "sinks dropped": ("csa_attention", _sinks_dropped),
    "sink carries a value": ("csa_attention", _sink_in_numerator),
    "tie-break to the higher index": ("select_topk", _tiebreak_reversed),
    "causality applied after ranking": ("select_topk", _causal_after_ranking),
    "overlap history lost": ("compressor_rows", _overlap_history_lost),
    "APE halves swapped": ("compressor_rows", _ape_halves_swapped),
    "APE slots reversed": ("compressor_rows", _ape_slots_reversed),
    "row RoPE one position early": ("rope_rows", _rope_at_previous_window),
    "RoPE on the leading dims": ("rope_rows", _rope_first_dims),
    "RMSNorm gain dropped": ("rms_norm", _norm_without_gain),
    "indexer averages heads": ("index_scores", _mean_over_heads),
    "indexer without ReLU": ("index_scores", _no_relu),
    "indexer sigmoid on weights": ("index_scores", _sigmoid_weights),
    "inverse rotation turns forward": ("rope_heads", _inverse_turns_forward),
    "output groups interleaved": ("grouped_out_proj", _groups_interleaved),
    "output groups reversed": ("grouped_out_proj", _groups_reversed),
    "lane slice read one token early (token0 - 1)": ("compressor_rows", _token0_off_by_one),
    "kv slice read one token late (kv_offset + 1)": ("csa_attention", _kv_offset_off_by_one),
    "pooled row rounded after the norm, not before": ("compressor_rows", _round_after_the_norm),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(C, attr, fn)
    caught = []
    for pin_name, pin in ALL_PINS.items():
        try:
            pin()
        except Exception:                   # an assertion, or the oracle's own guard
            caught.append(pin_name)
    assert caught, f"no pin catches the mutation '{name}'"
    print(f"{name}: caught by {', '.join(caught)}")
