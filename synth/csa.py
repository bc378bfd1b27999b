"""Seeded inputs of one CSA layer: boundary tensors of every token and the layer parameters.

Shapes only; no layer arithmetic.  ``spec`` is any object with the attributes ratio, heads,
dim, rope_dim, coff, index_heads, index_dim, has_rows, has_indexer and dtype.

Recipe (all draws from ``synth.token_lane`` / ``synth.normal``, seeded, per named stream):
  per token t of sequence b:  q [H, D], kv [D], a, g [coff*D], ai, gi [coff*d_i],
                              qi [H_i, d_i]  ~ N(0, 1) in the storage dtype;
                              w [H_i] ~ N(0, 1) fp32;
  per layer: ape [r, coff*D], ape_i [r, coff*d_i], norm_w [D], norm_w_i [d_i] ~ N(0, 1)
             (storage dtype); sinks [H] ~ N(0, 1) fp32;
             inv_freq[i] = theta^(-2i/rd), theta = 160000 (fp32).
N(0, 1) is the law of a projection x W^T with x ~ N(0, 1)^fan_in and W ~ N(0, 1)/sqrt(fan_in),
so drawing the projected tensors directly keeps the statistics of that recipe.
"""
from __future__ import annotations

import numpy as np
import torch

from . import normal, token_lane

ROPE_THETA = 160000.0


def inv_freq(rope_dim: int, theta: float = ROPE_THETA) -> torch.Tensor:
    i = np.arange(0, rope_dim, 2, dtype=np.float64)
    return torch.from_numpy((theta ** (-i / rope_dim)).astype(np.float32))


def layer_params(spec, seed: int, layer: int = 0, device="cpu") -> dict:
    dt = spec.dtype
    p = {"sinks": normal((spec.heads,), seed=seed, stream=f"L{layer}.sinks", device=device),
         "inv_freq": inv_freq(spec.rope_dim).to(device)}
    if spec.has_rows:
        W = spec.coff * spec.dim
        p["ape"] = normal((spec.ratio, W), seed=seed, stream=f"L{layer}.ape", dtype=dt, device=device)
        p["norm_w"] = normal((spec.dim,), seed=seed, stream=f"L{layer}.norm_w", dtype=dt, device=device)
    if spec.has_indexer:
        Wi = spec.coff * spec.index_dim
        p["ape_i"] = normal((spec.ratio, Wi), seed=seed, stream=f"L{layer}.ape_i", dtype=dt,
                            device=device)
        p["norm_w_i"] = normal((spec.index_dim,), seed=seed, stream=f"L{layer}.norm_w_i", dtype=dt,
                               device=device)
    return p


def _fields(spec):
    f = {"q": (spec.heads * spec.dim, spec.dtype, (spec.heads, spec.dim)),
         "kv": (spec.dim, spec.dtype, (spec.dim,))}
    if spec.has_rows:
        f["a"] = (spec.coff * spec.dim, spec.dtype, (spec.coff * spec.dim,))
        f["g"] = (spec.coff * spec.dim, spec.dtype, (spec.coff * spec.dim,))
    if spec.has_indexer:
        f["ai"] = (spec.coff * spec.index_dim, spec.dtype, (spec.coff * spec.index_dim,))
        f["gi"] = (spec.coff * spec.index_dim, spec.dtype, (spec.coff * spec.index_dim,))
        f["qi"] = (spec.index_heads * spec.index_dim, spec.dtype, (spec.index_heads, spec.index_dim))
        f["w"] = (spec.index_heads, torch.float32, (spec.index_heads,))
    return f


def token_inputs(spec, seed: int, b: int, t0: int, t1: int, layer: int = 0, device="cpu",
                 fields=None) -> dict:
    """Tensors of tokens t0..t1-1 of sequence b, each [t1-t0, *shape]."""
    out = {}
    for name, (width, dt, shape) in _fields(spec).items():
        if fields is not None and name not in fields:
            continue
        x = token_lane(seed=seed, stream=f"L{layer}.{name}", b=b, t0=t0, t1=t1, width=width,
                       dtype=dt, device=device)
        out[name] = x.reshape((t1 - t0,) + shape)
    return out


def batch_token_inputs(spec, seed: int, t0s, S: int, layer: int = 0, device="cpu",
                       fields=None) -> dict:
    """Stacked tensors [B, S, *shape] of tokens t0s[b] .. t0s[b]+S-1 of each sequence b."""
    per = [token_inputs(spec, seed, b, t0, t0 + S, layer, device, fields) for b, t0 in enumerate(t0s)]
    return {k: torch.stack([p[k] for p in per]) for k in per[0]}
