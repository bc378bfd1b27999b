"""One CSA layer's device state and the call order of the C ABI for prefill and decode.

A ``CsaLayer`` owns, for a batch of sequences, every buffer the layer carries between calls:
the two compressor frontiers (attention lane and indexer lane), the two compressed lanes,
the sliding-window ring and the indexer workspace.  Per step it calls, in order (MTPLX PR
#216 "What V4 adds": both prefill and decode maintain the lanes incrementally; mlx-lm PR
#1189 stepnoy's index-space fix: the indexer lane is accumulated unconditionally, so its
row count always equals the attention lane's):

    compress (attention lane) -> compress (indexer lane) -> index_topk -> attention

A decode step at which no sequence completes a compressed row only stores the token's
lanes in the compressor frontiers, which neither the selection nor the attention reads: it
goes as index_topk -> attention with the two frontier stores folded into the attention
launch (``dsv4_csa_attn_decode_store``).  Host-side lengths are plain integers; nothing here
computes any part of the layer.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (AttnCfg, CompCfg, GprojCfg, IndexCfg, RopeCfg, dsv4_comp_state_bytes,
               dsv4_compress_prefill, dsv4_compress_step, dsv4_csa_attn_decode,
               dsv4_csa_attn_decode_store, dsv4_csa_attn_prefill, dsv4_grouped_proj, dsv4_lane_proj,
               dsv4_index_topk, dsv4_index_workspace_bytes, dsv4_attn_workspace_bytes, dsv4_rope)


@dataclass(frozen=True)
class LayerSpec:
    """Shapes of one layer.  ratio 0 = pure sliding-window layer; overlap applies to ratio 4."""
    ratio: int
    heads: int = 64
    dim: int = 512
    rope_dim: int = 64
    window: int = 128
    index_heads: int = 64
    index_dim: int = 128
    topk: int = 512
    indexer: bool = True          # score and select rows (else every visible row is attended)
    overlap: bool | None = None   # default: ratio == 4
    eps: float = 1e-6
    dtype: torch.dtype = torch.bfloat16
    rollback: int = 0             # tokens a trim may take back exactly (speculative decode)

    @property
    def coff(self) -> int:
        return 2 if self.is_overlap else 1

    @property
    def is_overlap(self) -> bool:
        return (self.ratio == 4) if self.overlap is None else bool(self.overlap)

    @property
    def has_rows(self) -> bool:
        return self.ratio > 0

    @property
    def has_indexer(self) -> bool:
        return self.ratio > 0 and self.indexer

    @property
    def scale(self) -> float:
        return self.dim ** -0.5

    def comp_cfg(self) -> CompCfg:
        return CompCfg(self.ratio, self.is_overlap, self.dim, self.rope_dim, self.eps, self.dtype,
                       self.rollback)

    def index_comp_cfg(self) -> CompCfg:
        return CompCfg(self.ratio, self.is_overlap, self.index_dim, self.rope_dim, self.eps,
                       self.dtype, self.rollback)

    def index_cfg(self) -> IndexCfg:
        return IndexCfg(self.index_heads, self.index_dim, self.topk, self.ratio, self.dtype)

    def attn_cfg(self) -> AttnCfg:
        return AttnCfg(self.heads, self.dim, self.window, self.ratio, self.topk, self.scale,
                       self.dtype, self.rollback)


class CsaLayer:
    """Device state of one layer for ``batch`` sequences of up to ``max_tokens`` tokens."""

    def __init__(self, spec: LayerSpec, batch: int, max_tokens: int, params: dict,
                 device="cuda", max_chunk: int = 2048, fold_stores: bool = True):
        self.spec, self.batch, self.device = spec, batch, device
        self.fold_stores = fold_stores        # decode: frontier stores ride in the attention
        self.params = params                  # ape, norm_w, ape_i, norm_w_i, inv_freq, sinks
        self.lengths = [0] * batch
        self.max_lengths = [0] * batch        # furthest position each sequence has written
        dt = spec.dtype
        self.ring = torch.zeros(batch, spec.window + spec.rollback, spec.dim, dtype=dt,
                                device=device)
        self.row_cap = max_tokens // spec.ratio if spec.has_rows else 0
        if spec.has_rows:
            cc = spec.comp_cfg()
            self.state = torch.empty(batch, dsv4_comp_state_bytes(cc, 1), dtype=torch.uint8,
                                     device=device)
            self.rows = torch.empty(batch, max(1, self.row_cap), spec.dim, dtype=dt, device=device)
        if spec.has_indexer:
            ic = spec.index_comp_cfg()
            self.state_i = torch.empty(batch, dsv4_comp_state_bytes(ic, 1), dtype=torch.uint8,
                                       device=device)
            self.rows_i = torch.empty(batch, max(1, self.row_cap), spec.index_dim, dtype=dt,
                                      device=device)
            nb = dsv4_index_workspace_bytes(spec.index_cfg(), batch, max_chunk, max(1, self.row_cap))
            self.ws_index = torch.empty(nb, dtype=torch.uint8, device=device)
        # the split-key partials depend on batch * S: size for every chunk length up to max_chunk
        ac = spec.attn_cfg()
        nb = max(dsv4_attn_workspace_bytes(ac, batch, s) for s in range(1, min(max_chunk, 1024) + 1))
        self.ws_attn = torch.empty(max(1, nb), dtype=torch.uint8, device=device)

    # ------------------------------------------------------------------ state views
    def n_rows(self, extra: int = 0):
        r = self.spec.ratio
        return [(n + extra) // r for n in self.lengths] if r > 0 else None

    # ------------------------------------------------------------------ steps
    def rope_inputs(self, tok: dict, pos0, S: int):
        """RoPE of the per-head inputs of S tokens at positions pos0[b] + t, in place: q
        [B,S,H,D] and kv [B,S,D] (the last rope_dim dims of every head), and the indexer's qi
        [B,S,Hi,di] -- the rotation the boundary otherwise expects the caller to have applied
        (q, kv and qi turn at the token's absolute position with the layer's inv_freq, the
        same frequencies the compressed rows use: [MLXLM-1189] OmarB97's RoPE notes)."""
        sp, inv = self.spec, self.params["inv_freq"]
        B = len(pos0)
        dsv4_rope(RopeCfg(sp.heads, sp.dim, sp.rope_dim, False, sp.dtype),
                  tok["q"].view(B, S, sp.heads, sp.dim), pos0, inv)
        dsv4_rope(RopeCfg(1, sp.dim, sp.rope_dim, False, sp.dtype),
                  tok["kv"].view(B, S, 1, sp.dim), pos0, inv)
        if sp.has_indexer:
            dsv4_rope(RopeCfg(sp.index_heads, sp.index_dim, sp.rope_dim, False, sp.dtype),
                      tok["qi"].view(B, S, sp.index_heads, sp.index_dim), pos0, inv)

    def prefill(self, tok: dict, sel_out=None, rope: bool = False) -> torch.Tensor:
        """Process S new tokens of every sequence.  ``tok`` holds q [B,S,H,D], kv [B,S,D],
        a, g [B,S,coff*D], and with an indexer ai, gi [B,S,coff*di], qi [B,S,Hi,di],
        w [B,S,Hi].  Returns out [B,S,H,D]; writes the selection into ``sel_out`` if given.
        With ``rope``, q, kv and qi arrive unrotated and are rotated in place first."""
        sp, P = self.spec, self.params
        S = tok["q"].shape[1]
        pos0 = list(self.lengths)
        if rope:
            self.rope_inputs(tok, pos0, S)
        out = torch.empty_like(tok["q"])
        sel = None
        if sp.has_rows:
            dsv4_compress_prefill(sp.comp_cfg(), self.state, tok["a"], tok["g"], pos0, P["ape"],
                                  P["norm_w"], P["inv_freq"], self.rows)
        if sp.has_indexer:
            dsv4_compress_prefill(sp.index_comp_cfg(), self.state_i, tok["ai"], tok["gi"], pos0,
                                  P["ape_i"], P["norm_w_i"], P["inv_freq"], self.rows_i)
            sel = sel_out if sel_out is not None else torch.empty(
                self.batch, S, sp.topk, dtype=torch.int32, device=self.device)
            dsv4_index_topk(sp.index_cfg(), tok["qi"], tok["w"], self.rows_i, self.n_rows(S),
                            pos0, sel, self.ws_index)
        dsv4_csa_attn_prefill(sp.attn_cfg(), tok["q"], tok["kv"], self.ring,
                              self.rows if sp.has_rows else None, sel, self.n_rows(S), pos0,
                              P["sinks"], out, self.ws_attn)
        self._advance(S)
        return out

    def decode(self, tok: dict, sel_out=None, rope: bool = False) -> torch.Tensor:
        """One token per sequence; ``tok`` tensors have no S axis (q [B,H,D], kv [B,D], ...).
        With ``rope``, q, kv and qi arrive unrotated and are rotated in place first."""
        sp, P = self.spec, self.params
        pos = list(self.lengths)
        if rope:
            self.rope_inputs(tok, pos, 1)
        out = torch.empty_like(tok["q"])
        sel = None
        fold = (self.fold_stores and sp.has_rows and
                all((p + 1) % sp.ratio != 0 for p in pos))   # no row completes at this step
        stores = []
        if sp.has_rows:
            if fold:
                stores.append((sp.comp_cfg(), self.state, tok["a"], tok["g"]))
            else:
                dsv4_compress_step(sp.comp_cfg(), self.state, tok["a"], tok["g"], pos, P["ape"],
                                   P["norm_w"], P["inv_freq"], self.rows)
        if sp.has_indexer:
            if fold:
                stores.append((sp.index_comp_cfg(), self.state_i, tok["ai"], tok["gi"]))
            else:
                dsv4_compress_step(sp.index_comp_cfg(), self.state_i, tok["ai"], tok["gi"], pos,
                                   P["ape_i"], P["norm_w_i"], P["inv_freq"], self.rows_i)
            sel = sel_out if sel_out is not None else torch.empty(
                self.batch, 1, sp.topk, dtype=torch.int32, device=self.device)
            dsv4_index_topk(sp.index_cfg(), tok["qi"][:, None], tok["w"][:, None], self.rows_i,
                            self.n_rows(1), pos, sel, self.ws_index)
            sel = sel[:, 0]
        if fold:
            dsv4_csa_attn_decode_store(sp.attn_cfg(), tok["q"], tok["kv"], self.ring, self.rows,
                                       sel, self.n_rows(1), pos, P["sinks"], out, stores,
                                       self.ws_attn)
        else:
            dsv4_csa_attn_decode(sp.attn_cfg(), tok["q"], tok["kv"], self.ring,
                                 self.rows if sp.has_rows else None, sel, self.n_rows(1), pos,
                                 P["sinks"], out, self.ws_attn)
        self._advance(1)
        return out

    def _advance(self, n: int):
        self.lengths = [x + n for x in self.lengths]
        self.max_lengths = [max(m, x) for m, x in zip(self.max_lengths, self.lengths)]

    # ------------------------------------------------------------------ rollback
    def rollback_room(self):
        """Tokens each sequence can take back exactly: the retained depth (spec.rollback)
        less what earlier trims not yet re-decoded already used."""
        return [max(0, min(x, self.spec.rollback - (max(m, x) - x)))
                for x, m in zip(self.lengths, self.max_lengths)]

    def trim(self, n):
        """Take back the last n[b] tokens of each sequence (an int applies to all), exactly:
        afterwards every call behaves as if those tokens had never been processed (MTPLX PR
        #216 speculative-decode comment: emitted rows truncate, the compressor frontiers and
        the window keep what a rewind needs, and a trim past that bound raises rather than
        clamps).  Nothing on the device changes: rows past the new count are never read, and
        the window ring (W + rollback slots) and the frontier states (coff + ceil(rollback / r)
        windows) still hold every entry the shorter sequences read; re-decoded positions
        overwrite the stale ones.  Raises ValueError, changing nothing, if any n[b] exceeds
        rollback_room()[b]."""
        ns = [int(n)] * self.batch if isinstance(n, int) else [int(v) for v in n]
        if len(ns) != self.batch:
            raise ValueError(f"trim takes {self.batch} counts, got {len(ns)}")
        room = self.rollback_room()
        for b, (v, r) in enumerate(zip(ns, room)):
            if v < 0:
                raise ValueError(f"sequence {b}: negative trim {v}")
            if v > r:
                raise ValueError(f"sequence {b}: trim of {v} tokens exceeds the rollback room "
                                 f"{r} (capacity {self.spec.rollback})")
        self.lengths = [x - v for x, v in zip(self.lengths, ns)]


class SharedCsaLayer:
    """A layer that owns no compressor (V4.1 cross-layer KV sharing: [V41-MLX] "Why this
    exists", the cross-layer sharing item: only some layers run the compressors and build
    index keys; each of the others reads what the last such layer before it built, and the
    index-source layers among them score their own queries against those keys).

    ``owner`` is the CsaLayer whose compressed lanes this layer reads; ``spec`` gives this
    layer's own attention shape (heads, window, top-k) and must match the owner's latent
    width, ratio and dtype.  Each token, after the owner's call for it:
      * index="own" (an index-source layer): its own qi, w scored against the owner's index
        keys (the rows visible to the token, as for the owner) -> its own top-k;
      * index="owner": the selection the owner's indexer made for the same token, passed as
        ``sel`` (or, when the owner has no indexer, every visible row).
    The window holds the owner's token latents (the caller passes the owner's kv): the layer
    keeps them in a ring of its own, because a prefill call advances the ring it is given
    after attending, so two layers cannot take turns on one ring within a chunk.  Lengths
    follow the owner's: from a sequence's first token on, call ``prefill``/``decode`` with
    the same tokens right after the owner's call, while ``owner.lengths`` already counts
    them.  Every step runs in the library (index_topk, attention), as for the owner."""

    def __init__(self, spec: LayerSpec, owner: CsaLayer, params: dict, index: str = "own",
                 device="cuda", max_chunk: int = 2048):
        o = owner.spec
        if spec.ratio != o.ratio or spec.dim != o.dim or spec.dtype != o.dtype:
            raise ValueError("a sharing layer reads the owner's rows: ratio, dim and dtype must match")
        if index not in ("own", "owner"):
            raise ValueError(f"index must be 'own' or 'owner', not {index!r}")
        if index == "own" and spec.has_indexer and not (
                o.has_indexer and (spec.index_heads, spec.index_dim) == (o.index_heads, o.index_dim)):
            raise ValueError("index='own' scores against the owner's index keys: the owner needs "
                             "an indexer of the same width")
        if index == "owner" and spec.has_indexer and not o.has_indexer:
            raise ValueError("index='owner' needs an owner with an indexer")
        if index == "owner" and o.has_indexer and spec.topk != o.topk:
            raise ValueError("index='owner' attends the owner's selection: top-k must match")
        self.spec, self.owner, self.params, self.index = spec, owner, params, index
        self.batch, self.device = owner.batch, device
        self.ring = torch.zeros(owner.batch, spec.window + spec.rollback, spec.dim, dtype=spec.dtype,
                                device=device)
        if index == "own" and spec.has_indexer:
            nb = dsv4_index_workspace_bytes(spec.index_cfg(), owner.batch, max_chunk, max(1, owner.row_cap))
            self.ws_index = torch.empty(nb, dtype=torch.uint8, device=device)
        ac = spec.attn_cfg()
        nb = max(dsv4_attn_workspace_bytes(ac, owner.batch, s) for s in range(1, min(max_chunk, 1024) + 1))
        self.ws_attn = torch.empty(max(1, nb), dtype=torch.uint8, device=device)

    def _positions(self, S: int):
        # the owner has already advanced past these S tokens
        return [n - S for n in self.owner.lengths]

    def _select(self, tok: dict, pos0, S: int, sel, sel_out):
        sp, ow = self.spec, self.owner
        if not (sp.has_indexer and ow.spec.has_indexer):
            return None
        if self.index == "owner":
            if sel is None:
                raise ValueError("index='owner': pass the owner's selection for these tokens")
            return sel
        out = sel_out if sel_out is not None else torch.empty(
            self.batch, S, sp.topk, dtype=torch.int32, device=self.device)
        dsv4_index_topk(sp.index_cfg(), tok["qi"], tok["w"], ow.rows_i, ow.n_rows(), pos0, out,
                        self.ws_index)
        return out

    def prefill(self, tok: dict, sel=None, sel_out=None) -> torch.Tensor:
        """S tokens of every sequence: q [B,S,H,D], kv [B,S,D] (the owner's), and for
        index='own' qi [B,S,Hi,di], w [B,S,Hi]; for index='owner' ``sel`` [B,S,k] is the
        owner's selection of these tokens.  Returns out [B,S,H,D]."""
        sp, ow = self.spec, self.owner
        S = tok["q"].shape[1]
        pos0 = self._positions(S)
        chosen = self._select(tok, pos0, S, sel, sel_out)
        out = torch.empty_like(tok["q"])
        dsv4_csa_attn_prefill(sp.attn_cfg(), tok["q"], tok["kv"], self.ring,
                              ow.rows if sp.has_rows else None, chosen, ow.n_rows(), pos0,
                              self.params["sinks"], out, self.ws_attn)
        return out

    def decode(self, tok: dict, sel=None, sel_out=None) -> torch.Tensor:
        """One token per sequence (no S axis: q [B,H,D], kv [B,D], qi [B,Hi,di], w [B,Hi];
        ``sel`` [B,k] for index='owner')."""
        sp, ow = self.spec, self.owner
        pos = self._positions(1)
        chosen = None
        if sp.has_indexer and ow.spec.has_indexer:
            if self.index == "owner":
                if sel is None:
                    raise ValueError("index='owner': pass the owner's selection for this token")
                chosen = sel
            else:
                s3 = sel_out if sel_out is not None else torch.empty(
                    self.batch, 1, sp.topk, dtype=torch.int32, device=self.device)
                dsv4_index_topk(sp.index_cfg(), tok["qi"][:, None], tok["w"][:, None], ow.rows_i,
                                ow.n_rows(), pos, s3, self.ws_index)
                chosen = s3[:, 0]
        out = torch.empty_like(tok["q"])
        dsv4_csa_attn_decode(sp.attn_cfg(), tok["q"], tok["kv"], self.ring,
                             ow.rows if sp.has_rows else None, chosen, ow.n_rows(), pos,
                             self.params["sinks"], out, self.ws_attn)
        return out


def output_path(spec: LayerSpec, o: torch.Tensor, pos0, inv_freq: torch.Tensor,
                wo_a: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """The attention output's way out of the layer: the rotary dims of every head turned back
    (inverse RoPE at the token's position, in place on ``o``), then the grouped block-diagonal
    projection by ``wo_a`` [G, R, H/G * D].  o: [B, S, H, D] (decode: S = 1); returns
    y [B, S, G, R].  Two library calls: dsv4_rope (inverse) and dsv4_grouped_proj."""
    B, S = o.shape[0], o.shape[1]
    G, R, Kd = wo_a.shape
    dsv4_rope(RopeCfg(spec.heads, spec.dim, spec.rope_dim, True, spec.dtype), o, pos0, inv_freq)
    if y is None:
        y = torch.empty(B, S, G, R, dtype=spec.dtype, device=o.device)
    dsv4_grouped_proj(GprojCfg(G, Kd, R, spec.dtype), o.view(B * S, G, Kd), wo_a, y.view(B * S, G, R))
    return y


def compressor_lanes(x: torch.Tensor, w_kv: torch.Tensor, w_gate: torch.Tensor):
    """A compressor's two lanes from the layer's hidden states: a = x w_kv^T and
    g = x w_gate^T (the ratio-4 layer's wkv and wgate are [1024, 4096]: [MLXLM-1189]
    Thump604's fix list).  x [T, hidden]; w_kv, w_gate [coff*D, hidden]; returns a, g
    [T, coff*D], ready for dsv4_compress_prefill (one sequence's chunk) or, with one token
    per sequence, dsv4_compress_step.  One dsv4_lane_proj call (both products in one launch
    from 33 tokens on)."""
    T, Kd = x.shape
    W = w_kv.shape[0]
    cfg = GprojCfg(1, Kd, W, x.dtype)
    a = torch.empty(T, W, dtype=x.dtype, device=x.device)
    g = torch.empty(T, W, dtype=x.dtype, device=x.device)
    dsv4_lane_proj(cfg, x, w_kv, w_gate, a, g)
    return a, g
