"""Python binding of libdsv4.so, the MI355X CSA layer (compressor, indexer, sparse attention).

Argument marshalling only: each function checks that the torch tensors it is given have the
shapes, dtypes and device the C call expects (the C layer sees raw pointers and cannot),
then calls the C entry point of the same name on torch's current HIP stream.  Every step of
the layer runs in the library's kernels; there is no fallback path.  If the library is not
built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # imported before the library so both share torch's HIP runtime

__all__ = [
    "Dsv4Error", "CompCfg", "IndexCfg", "AttnCfg", "lib", "lib_path",
    "dsv4_version", "dsv4_comp_state_bytes", "dsv4_index_workspace_bytes",
    "dsv4_attn_workspace_bytes", "dsv4_compress_prefill", "dsv4_compress_step",
    "dsv4_index_topk", "dsv4_index_topk_noalloc", "dsv4_index_topk_noalloc_scratch_bytes",
    "dsv4_csa_attn_decode", "dsv4_csa_attn_decode_store",
    "dsv4_csa_attn_prefill", "dsv4_rope", "dsv4_grouped_proj", "dsv4_lane_proj", "RopeCfg", "GprojCfg",
    "dsv4_trace_enable", "dsv4_trace_reset", "dsv4_trace_read", "dsv4_trace_kernels",
    "EXPORTED_SYMBOLS",
]

BF16, F32 = 0, 1
_DTYPES = {torch.bfloat16: BF16, torch.float32: F32}
lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsv4.so")

EXPORTED_SYMBOLS = (
    "dsv4_version", "dsv4_last_error", "dsv4_comp_state_bytes", "dsv4_index_workspace_bytes",
    "dsv4_attn_workspace_bytes", "dsv4_compress_prefill", "dsv4_compress_step",
    "dsv4_index_topk", "dsv4_index_topk_noalloc", "dsv4_index_topk_noalloc_scratch_bytes",
    "dsv4_csa_attn_decode", "dsv4_csa_attn_decode_store",
    "dsv4_csa_attn_prefill", "dsv4_rope", "dsv4_grouped_proj", "dsv4_lane_proj", "dsv4_trace_enable",
    "dsv4_trace_reset", "dsv4_trace_read", "dsv4_trace_kernel_name",
)


class Dsv4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dsv4 error {code}: {msg}")
        self.code = code


class _CompCfg(ctypes.Structure):
    _fields_ = [("ratio", ctypes.c_int32), ("overlap", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("eps", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("retain", ctypes.c_int32)]


class _IndexCfg(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("dim", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("ratio", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class _AttnCfg(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("ratio", ctypes.c_int32), ("topk", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("retain", ctypes.c_int32)]


class _RopeCfg(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("inverse", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class _GprojCfg(ctypes.Structure):
    _fields_ = [("groups", ctypes.c_int32), ("in_dim", ctypes.c_int32), ("out_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class _FrontierStore(ctypes.Structure):
    _fields_ = [("cfg", ctypes.POINTER(_CompCfg)), ("state", ctypes.c_void_p),
                ("kv_lane", ctypes.c_void_p), ("gate_lane", ctypes.c_void_p)]


@dataclass(frozen=True)
class CompCfg:
    ratio: int
    overlap: bool
    dim: int
    rope_dim: int
    eps: float = 1e-6
    dtype: torch.dtype = torch.bfloat16
    retain: int = 0               # tokens of rollback the frontier state keeps

    @property
    def coff(self) -> int:
        return 2 if self.overlap else 1

    def c(self):
        return _CompCfg(self.ratio, int(self.overlap), self.dim, self.rope_dim, self.eps,
                        _DTYPES[self.dtype], self.retain)


@dataclass(frozen=True)
class IndexCfg:
    heads: int
    dim: int
    topk: int
    ratio: int
    dtype: torch.dtype = torch.bfloat16

    def c(self):
        return _IndexCfg(self.heads, self.dim, self.topk, self.ratio, _DTYPES[self.dtype])


@dataclass(frozen=True)
class RopeCfg:
    heads: int
    dim: int
    rope_dim: int
    inverse: bool = False
    dtype: torch.dtype = torch.bfloat16

    def c(self):
        return _RopeCfg(self.heads, self.dim, self.rope_dim, int(self.inverse), _DTYPES[self.dtype])


@dataclass(frozen=True)
class GprojCfg:
    groups: int
    in_dim: int
    out_dim: int
    dtype: torch.dtype = torch.bfloat16

    def c(self):
        return _GprojCfg(self.groups, self.in_dim, self.out_dim, _DTYPES[self.dtype])


@dataclass(frozen=True)
class AttnCfg:
    heads: int
    dim: int
    window: int
    ratio: int
    topk: int
    scale: float
    dtype: torch.dtype = torch.bfloat16
    retain: int = 0               # tokens of rollback the window ring keeps (W + retain slots)

    @property
    def ring_slots(self) -> int:
        return self.window + self.retain

    def c(self):
        return _AttnCfg(self.heads, self.dim, self.window, self.ratio, self.topk, self.scale,
                        _DTYPES[self.dtype], self.retain)


_lib = None
_P = ctypes.c_void_p
_I64P = ctypes.POINTER(ctypes.c_int64)


def lib():
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is not built: run `python -m sparse_attention_dsv4_amd.build`")
        L = ctypes.CDLL(lib_path)
        L.dsv4_version.restype = ctypes.c_char_p
        L.dsv4_last_error.restype = ctypes.c_char_p
        L.dsv4_trace_kernel_name.restype = ctypes.c_char_p
        L.dsv4_trace_kernel_name.argtypes = [ctypes.c_int32]
        for n in ("dsv4_comp_state_bytes", "dsv4_index_workspace_bytes", "dsv4_attn_workspace_bytes",
                  "dsv4_index_topk_noalloc_scratch_bytes"):
            getattr(L, n).restype = ctypes.c_size_t
        L.dsv4_comp_state_bytes.argtypes = [ctypes.POINTER(_CompCfg), ctypes.c_int32]
        L.dsv4_index_workspace_bytes.argtypes = [ctypes.POINTER(_IndexCfg), ctypes.c_int32,
                                                 ctypes.c_int64, ctypes.c_int64]
        L.dsv4_attn_workspace_bytes.argtypes = [ctypes.POINTER(_AttnCfg), ctypes.c_int32, ctypes.c_int64]
        L.dsv4_compress_prefill.argtypes = [ctypes.POINTER(_CompCfg), _P, _P, _P, ctypes.c_int32,
                                            ctypes.c_int64, _I64P, _P, _P, _P, _P, ctypes.c_int64, _P]
        L.dsv4_compress_step.argtypes = [ctypes.POINTER(_CompCfg), _P, _P, _P, ctypes.c_int32,
                                         _I64P, _P, _P, _P, _P, ctypes.c_int64, _P]
        L.dsv4_index_topk.argtypes = [ctypes.POINTER(_IndexCfg), _P, _P, _P, ctypes.c_int64, _I64P,
                                      _I64P, ctypes.c_int32, ctypes.c_int64, _P, _P, ctypes.c_size_t, _P]
        L.dsv4_index_topk_noalloc.argtypes = [ctypes.POINTER(_IndexCfg), _P, _P, _P, ctypes.c_int64,
                                              _I64P, _I64P, ctypes.c_int32, ctypes.c_int64, _P, _P]
        L.dsv4_csa_attn_decode.argtypes = [ctypes.POINTER(_AttnCfg), _P, _P, _P, _P, ctypes.c_int64,
                                           _P, _I64P, _I64P, _P, _P, ctypes.c_int32, _P,
                                           ctypes.c_size_t, _P]
        L.dsv4_csa_attn_decode_store.argtypes = [
            ctypes.POINTER(_AttnCfg), _P, _P, _P, _P, ctypes.c_int64, _P, _I64P, _I64P, _P, _P,
            ctypes.c_int32, _P, ctypes.c_size_t, ctypes.POINTER(_FrontierStore), ctypes.c_int32, _P]
        L.dsv4_csa_attn_prefill.argtypes = [ctypes.POINTER(_AttnCfg), _P, _P, _P, _P, ctypes.c_int64,
                                            _P, _I64P, _I64P, _P, _P, ctypes.c_int32, ctypes.c_int64,
                                            _P, ctypes.c_size_t, _P]
        L.dsv4_rope.argtypes = [ctypes.POINTER(_RopeCfg), _P, _I64P, ctypes.c_int32, ctypes.c_int64,
                                _P, _P]
        L.dsv4_grouped_proj.argtypes = [ctypes.POINTER(_GprojCfg), _P, _P, _P, ctypes.c_int64, _P]
        L.dsv4_lane_proj.argtypes = [ctypes.POINTER(_GprojCfg), _P, _P, _P, _P, _P, ctypes.c_int64, _P]
        L.dsv4_trace_enable.argtypes = [ctypes.c_int32]
        L.dsv4_trace_read.argtypes = [ctypes.c_char_p, _I64P, ctypes.POINTER(ctypes.c_double)]
        _lib = L
    return _lib


def _check(code: int):
    if code != 0:
        raise Dsv4Error(code, lib().dsv4_last_error().decode())


def _host_i64(vals, n: int, what: str):
    vals = [int(v) for v in vals]
    if len(vals) != n:
        raise ValueError(f"{what}: expected {n} entries, got {len(vals)}")
    return (ctypes.c_int64 * n)(*vals)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, shape, dtype, what: str):
    if t is None:
        raise ValueError(f"{what} is required")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ sizes
def dsv4_version() -> str:
    return lib().dsv4_version().decode()


def dsv4_comp_state_bytes(cfg: CompCfg, batch: int) -> int:
    c = cfg.c()
    return int(lib().dsv4_comp_state_bytes(ctypes.byref(c), batch))


def dsv4_index_workspace_bytes(cfg: IndexCfg, batch: int, s: int, n_max: int) -> int:
    c = cfg.c()
    return int(lib().dsv4_index_workspace_bytes(ctypes.byref(c), batch, s, n_max))


def dsv4_attn_workspace_bytes(cfg: AttnCfg, batch: int, s: int) -> int:
    c = cfg.c()
    return int(lib().dsv4_attn_workspace_bytes(ctypes.byref(c), batch, s))


# ------------------------------------------------------------------ the layer
def dsv4_compress_prefill(cfg: CompCfg, state, kv_lane, gate_lane, len_before, ape, norm_w,
                          inv_freq, rows, stream=None):
    """kv_lane, gate_lane [B, n, coff*D]; state: uint8 [B, state_bytes]; rows [B, cap, D]."""
    B, n = kv_lane.shape[0], kv_lane.shape[1]
    W = cfg.coff * cfg.dim
    _need(kv_lane, (B, n, W), cfg.dtype, "kv_lane")
    _need(gate_lane, (B, n, W), cfg.dtype, "gate_lane")
    _need(state, (B, dsv4_comp_state_bytes(cfg, 1)), torch.uint8, "state")
    _need(ape, (cfg.ratio, W), cfg.dtype, "ape")
    _need(norm_w, (cfg.dim,), cfg.dtype, "norm_w")
    _need(inv_freq, (cfg.rope_dim // 2,), torch.float32, "inv_freq")
    if rows.dim() != 3 or rows.shape[0] != B:
        raise ValueError("rows must be [B, cap, D]")
    _need(rows, (B, rows.shape[1], cfg.dim), cfg.dtype, "rows")
    c = cfg.c()
    _check(lib().dsv4_compress_prefill(
        ctypes.byref(c), _ptr(state), _ptr(kv_lane), _ptr(gate_lane), B, n,
        _host_i64(len_before, B, "len_before"), _ptr(ape), _ptr(norm_w), _ptr(inv_freq),
        _ptr(rows), rows.shape[1], _stream(stream)))


def dsv4_compress_step(cfg: CompCfg, state, kv_lane, gate_lane, len_before, ape, norm_w,
                       inv_freq, rows, stream=None):
    """One token per sequence: kv_lane, gate_lane [B, coff*D]."""
    B = kv_lane.shape[0]
    W = cfg.coff * cfg.dim
    _need(kv_lane, (B, W), cfg.dtype, "kv_lane")
    _need(gate_lane, (B, W), cfg.dtype, "gate_lane")
    _need(state, (B, dsv4_comp_state_bytes(cfg, 1)), torch.uint8, "state")
    _need(ape, (cfg.ratio, W), cfg.dtype, "ape")
    _need(norm_w, (cfg.dim,), cfg.dtype, "norm_w")
    _need(inv_freq, (cfg.rope_dim // 2,), torch.float32, "inv_freq")
    if rows.dim() != 3 or rows.shape[0] != B:
        raise ValueError("rows must be [B, cap, D]")
    _need(rows, (B, rows.shape[1], cfg.dim), cfg.dtype, "rows")
    c = cfg.c()
    _check(lib().dsv4_compress_step(
        ctypes.byref(c), _ptr(state), _ptr(kv_lane), _ptr(gate_lane), B,
        _host_i64(len_before, B, "len_before"), _ptr(ape), _ptr(norm_w), _ptr(inv_freq),
        _ptr(rows), rows.shape[1], _stream(stream)))


def dsv4_index_topk(cfg: IndexCfg, qi, w, idx_rows, n_rows, pos0, sel, ws, stream=None):
    """qi [B, S, Hi, di]; w [B, S, Hi] fp32; idx_rows [B, cap, di]; sel [B, S, k] int32;
    ws: uint8 workspace of at least dsv4_index_workspace_bytes(cfg, B, S, max(n_rows))."""
    B, S = qi.shape[0], qi.shape[1]
    _need(qi, (B, S, cfg.heads, cfg.dim), cfg.dtype, "qi")
    _need(w, (B, S, cfg.heads), torch.float32, "w")
    if idx_rows.dim() != 3:
        raise ValueError("idx_rows must be [B, cap, di]")
    _need(idx_rows, (B, idx_rows.shape[1], cfg.dim), cfg.dtype, "idx_rows")
    _need(sel, (B, S, cfg.topk), torch.int32, "sel")
    if ws is None or ws.dtype != torch.uint8 or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous uint8 GPU tensor")
    c = cfg.c()
    _check(lib().dsv4_index_topk(
        ctypes.byref(c), _ptr(qi), _ptr(w), _ptr(idx_rows), idx_rows.shape[1],
        _host_i64(n_rows, B, "n_rows"), _host_i64(pos0, B, "pos0"), B, S, _ptr(sel), _ptr(ws),
        ws.numel(), _stream(stream)))


def dsv4_index_topk_noalloc_scratch_bytes() -> int:
    return int(lib().dsv4_index_topk_noalloc_scratch_bytes())


def dsv4_index_topk_noalloc(cfg: IndexCfg, qi, w, idx_rows, n_rows, pos0, sel, stream=None):
    """dsv4_index_topk with the library's fixed per-GPU scratch instead of a workspace (no
    allocation; calls that overlap on one GPU race)."""
    B, S = qi.shape[0], qi.shape[1]
    _need(qi, (B, S, cfg.heads, cfg.dim), cfg.dtype, "qi")
    _need(w, (B, S, cfg.heads), torch.float32, "w")
    if idx_rows.dim() != 3:
        raise ValueError("idx_rows must be [B, cap, di]")
    _need(idx_rows, (B, idx_rows.shape[1], cfg.dim), cfg.dtype, "idx_rows")
    _need(sel, (B, S, cfg.topk), torch.int32, "sel")
    c = cfg.c()
    _check(lib().dsv4_index_topk_noalloc(
        ctypes.byref(c), _ptr(qi), _ptr(w), _ptr(idx_rows), idx_rows.shape[1],
        _host_i64(n_rows, B, "n_rows"), _host_i64(pos0, B, "pos0"), B, S, _ptr(sel),
        _stream(stream)))


def _attn_common_checks(cfg: AttnCfg, rows, sel, n_rows, B, sel_shape):
    if cfg.ratio > 0:
        if rows is None or rows.dim() != 3:
            raise ValueError("rows must be [B, cap, D] when ratio > 0")
        _need(rows, (B, rows.shape[1], cfg.dim), cfg.dtype, "rows")
        if n_rows is None:
            raise ValueError("n_rows is required when ratio > 0")
    if sel is not None:
        _need(sel, sel_shape, torch.int32, "sel")


def dsv4_csa_attn_decode(cfg: AttnCfg, q, kv_new, win_ring, rows, sel, n_rows, pos, sinks, out,
                         ws=None, stream=None):
    """q [B, H, D]; kv_new [B, D]; win_ring [B, W, D]; rows [B, cap, D] or None; sel [B, k]
    int32 or None; sinks [H] fp32; out [B, H, D]."""
    B = q.shape[0]
    _need(q, (B, cfg.heads, cfg.dim), cfg.dtype, "q")
    _need(kv_new, (B, cfg.dim), cfg.dtype, "kv_new")
    _need(win_ring, (B, cfg.ring_slots, cfg.dim), cfg.dtype, "win_ring")
    _need(sinks, (cfg.heads,), torch.float32, "sinks")
    _need(out, (B, cfg.heads, cfg.dim), cfg.dtype, "out")
    _attn_common_checks(cfg, rows, sel, n_rows, B, (B, cfg.topk))
    c = cfg.c()
    _check(lib().dsv4_csa_attn_decode(
        ctypes.byref(c), _ptr(q), _ptr(kv_new), _ptr(win_ring),
        _ptr(rows) if cfg.ratio > 0 else None, rows.shape[1] if cfg.ratio > 0 else 0,
        _ptr(sel), _host_i64(n_rows, B, "n_rows") if cfg.ratio > 0 else None,
        _host_i64(pos, B, "pos"), _ptr(sinks), _ptr(out), B, _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dsv4_csa_attn_decode_store(cfg: AttnCfg, q, kv_new, win_ring, rows, sel, n_rows, pos, sinks,
                               out, stores, ws=None, stream=None):
    """dsv4_csa_attn_decode, plus the compressor steps of the same token for the lanes in
    ``stores``: a list of up to two (CompCfg, state, kv_lane [B, coff*D], gate_lane) -- for a
    step at which no sequence completes a compressed row ((pos + 1) % ratio != 0)."""
    B = q.shape[0]
    _need(q, (B, cfg.heads, cfg.dim), cfg.dtype, "q")
    _need(kv_new, (B, cfg.dim), cfg.dtype, "kv_new")
    _need(win_ring, (B, cfg.ring_slots, cfg.dim), cfg.dtype, "win_ring")
    _need(sinks, (cfg.heads,), torch.float32, "sinks")
    _need(out, (B, cfg.heads, cfg.dim), cfg.dtype, "out")
    _attn_common_checks(cfg, rows, sel, n_rows, B, (B, cfg.topk))
    ccfgs = []
    arr = (_FrontierStore * max(1, len(stores)))()
    for i, (ccfg, state, kv_lane, gate_lane) in enumerate(stores):
        W = ccfg.coff * ccfg.dim
        _need(kv_lane, (B, W), ccfg.dtype, "kv_lane")
        _need(gate_lane, (B, W), ccfg.dtype, "gate_lane")
        _need(state, (B, dsv4_comp_state_bytes(ccfg, 1)), torch.uint8, "state")
        ccfgs.append(ccfg.c())
        arr[i] = _FrontierStore(ctypes.pointer(ccfgs[-1]), _ptr(state), _ptr(kv_lane), _ptr(gate_lane))
    c = cfg.c()
    _check(lib().dsv4_csa_attn_decode_store(
        ctypes.byref(c), _ptr(q), _ptr(kv_new), _ptr(win_ring),
        _ptr(rows) if cfg.ratio > 0 else None, rows.shape[1] if cfg.ratio > 0 else 0,
        _ptr(sel), _host_i64(n_rows, B, "n_rows") if cfg.ratio > 0 else None,
        _host_i64(pos, B, "pos"), _ptr(sinks), _ptr(out), B, _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), arr, len(stores), _stream(stream)))


def dsv4_csa_attn_prefill(cfg: AttnCfg, q, kv_new, win_ring, rows, sel, n_rows, pos0, sinks,
                          out, ws=None, stream=None):
    """q [B, S, H, D]; kv_new [B, S, D]; win_ring [B, W, D]; sel [B, S, k] int32 or None;
    out [B, S, H, D]."""
    B, S = q.shape[0], q.shape[1]
    _need(q, (B, S, cfg.heads, cfg.dim), cfg.dtype, "q")
    _need(kv_new, (B, S, cfg.dim), cfg.dtype, "kv_new")
    _need(win_ring, (B, cfg.ring_slots, cfg.dim), cfg.dtype, "win_ring")
    _need(sinks, (cfg.heads,), torch.float32, "sinks")
    _need(out, (B, S, cfg.heads, cfg.dim), cfg.dtype, "out")
    _attn_common_checks(cfg, rows, sel, n_rows, B, (B, S, cfg.topk))
    c = cfg.c()
    _check(lib().dsv4_csa_attn_prefill(
        ctypes.byref(c), _ptr(q), _ptr(kv_new), _ptr(win_ring),
        _ptr(rows) if cfg.ratio > 0 else None, rows.shape[1] if cfg.ratio > 0 else 0,
        _ptr(sel), _host_i64(n_rows, B, "n_rows") if cfg.ratio > 0 else None,
        _host_i64(pos0, B, "pos0"), _ptr(sinks), _ptr(out), B, S, _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


# ------------------------------------------------------------------ kernel trace
def dsv4_trace_enable(on: bool = True):
    _check(lib().dsv4_trace_enable(int(bool(on))))


def dsv4_trace_reset():
    _check(lib().dsv4_trace_reset())


def dsv4_trace_read(name_substr: str = ""):
    """(launches, total_ms) of traced kernels whose name contains ``name_substr`` (or, for
    "=name", of the kernel of exactly that name)."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(lib().dsv4_trace_read(name_substr.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def dsv4_trace_kernels():
    out, i = [], 0
    while True:
        n = lib().dsv4_trace_kernel_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


def dsv4_rope(cfg: RopeCfg, x, pos0, inv_freq, stream=None):
    """RoPE in place on x [B, S, H, D] (token t of sequence b at position pos0[b] + t), or its
    inverse when cfg.inverse; inv_freq [rd/2] fp32."""
    if x is None or x.dim() != 4:
        raise ValueError("x must be [B, S, H, D]")
    B, S = x.shape[0], x.shape[1]
    _need(x, (B, S, cfg.heads, cfg.dim), cfg.dtype, "x")
    _need(inv_freq, (cfg.rope_dim // 2,), torch.float32, "inv_freq")
    c = cfg.c()
    _check(lib().dsv4_rope(ctypes.byref(c), _ptr(x), _host_i64(pos0, B, "pos0"), B, S,
                           _ptr(inv_freq), _stream(stream)))


def dsv4_grouped_proj(cfg: GprojCfg, x, w, y, stream=None):
    """y [T, G, R] = per group g: x [T, G, K][:, g] @ w [G, R, K][g].T (fp32 accumulation)."""
    if x is None or x.dim() != 3:
        raise ValueError("x must be [T, G, K]")
    T = x.shape[0]
    _need(x, (T, cfg.groups, cfg.in_dim), cfg.dtype, "x")
    _need(w, (cfg.groups, cfg.out_dim, cfg.in_dim), cfg.dtype, "w")
    _need(y, (T, cfg.groups, cfg.out_dim), cfg.dtype, "y")
    c = cfg.c()
    _check(lib().dsv4_grouped_proj(ctypes.byref(c), _ptr(x), _ptr(w), _ptr(y), T, _stream(stream)))


def dsv4_lane_proj(cfg: GprojCfg, x, w_kv, w_gate, a, g, stream=None):
    """a [T, W] = x [T, K] @ w_kv [W, K].T and g [T, W] = x @ w_gate.T (one group; one launch
    where the tiled kernel applies)."""
    if x is None or x.dim() != 2:
        raise ValueError("x must be [T, K]")
    if cfg.groups != 1:
        raise ValueError("the lane projection takes one group")
    T = x.shape[0]
    _need(x, (T, cfg.in_dim), cfg.dtype, "x")
    _need(w_kv, (cfg.out_dim, cfg.in_dim), cfg.dtype, "w_kv")
    _need(w_gate, (cfg.out_dim, cfg.in_dim), cfg.dtype, "w_gate")
    _need(a, (T, cfg.out_dim), cfg.dtype, "a")
    _need(g, (T, cfg.out_dim), cfg.dtype, "g")
    c = cfg.c()
    _check(lib().dsv4_lane_proj(ctypes.byref(c), _ptr(x), _ptr(w_kv), _ptr(w_gate), _ptr(a), _ptr(g), T,
                                _stream(stream)))
