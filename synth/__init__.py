"""Seeded synthetic inputs for the CSA layer, shared by the tests, the bench and the
oracle-side checks.

This module draws numbers and nothing else: it holds none of the layer's arithmetic.

Construction (counter-based, so any slice can be regenerated on its own):
  * a table of 2**20 standard-normal draws comes from a seeded torch CPU generator;
  * element ``i`` of a named stream reads ``table[h(seed, stream, i) >> 12]`` where ``h`` is
    a 32-bit integer mixer (Wellons' "lowbias32" finaliser applied in a chain);
  * the table is scaled and cast to the storage dtype once, on the CPU, before the gather.

Integer hashing and a gather are exact on every device, so a tensor generated on the GPU is
bit-identical to the same tensor generated on the CPU.  Each value is marginally N(0, scale^2)
(a 2**20-point empirical normal), independent across elements up to hash quality.

Token lanes are indexed by absolute position: element (b, t, c) of a lane of width ``w`` has
flat index ``(b * T_MAX + t) * w + c``, so a sequence's lane is the same whatever chunking
produced it, and the oracle can rebuild just the tokens one compressed row needs.
"""
from __future__ import annotations

import zlib

import torch

__all__ = ["T_MAX", "TABLE_BITS", "stream_id", "normal", "token_lane", "value_table"]

T_MAX = 1 << 22          # positions per sequence addressable in a token lane
TABLE_BITS = 20
_M32 = 0xFFFFFFFF
_tables: dict = {}


def stream_id(name: str) -> int:
    """Stable 32-bit id of a named stream."""
    return zlib.crc32(name.encode("utf-8")) & _M32


def _mul32(x: torch.Tensor, m: int) -> torch.Tensor:
    # (x * m) mod 2**32 for x < 2**32, with every int64 intermediate below 2**49.
    lo = x * (m & 0xFFFF)
    hi = ((x * (m >> 16)) & 0xFFFF) << 16
    return (lo + hi) & _M32


def _mix(x: torch.Tensor) -> torch.Tensor:
    # lowbias32 (C. Wellons, "Hash function prospector"): xorshift-multiply finaliser.
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix_int(v: int) -> int:
    return int(_mix(torch.tensor([v & _M32], dtype=torch.int64))[0])


def value_table(seed: int) -> torch.Tensor:
    """The 2**20 standard-normal draws behind every stream of ``seed`` (fp32, CPU)."""
    if seed not in _tables:
        g = torch.Generator().manual_seed(0x5EED0000 + int(seed))
        _tables[seed] = torch.randn(1 << TABLE_BITS, generator=g, dtype=torch.float32)
    return _tables[seed]


def _scaled_table(seed: int, scale: float, dtype, device) -> torch.Tensor:
    t = value_table(seed)
    if scale != 1.0:
        t = t * torch.tensor(scale, dtype=torch.float32)
    return t.to(dtype).to(device)


def _gather(flat_idx: torch.Tensor, seed: int, stream: str, scale: float, dtype, device):
    s = _mix_int(_mix_int(int(seed) * 0x9E3779B1) ^ stream_id(stream))
    lo = flat_idx & _M32
    hi = flat_idx >> 32
    h = _mix(_mix(_mix(hi ^ s) ^ lo) ^ ((s * 0x2545F491) & _M32))
    table = _scaled_table(seed, scale, dtype, device)
    return table[h >> (32 - TABLE_BITS)]


def normal(shape, *, seed: int, stream: str, scale: float = 1.0,
           dtype=torch.float32, device="cpu", offset: int = 0) -> torch.Tensor:
    """A tensor of ``shape`` whose flat element i is stream element ``offset + i``."""
    n = 1
    for s in shape:
        n *= int(s)
    idx = torch.arange(offset, offset + n, dtype=torch.int64, device=device)
    return _gather(idx, seed, stream, scale, dtype, device).reshape(tuple(shape))


def token_lane(*, seed: int, stream: str, b: int, t0: int, t1: int, width: int,
               scale: float = 1.0, dtype=torch.float32, device="cpu",
               chunk_tokens: int = 8192) -> torch.Tensor:
    """Rows ``t0 .. t1-1`` of sequence ``b`` of a token lane of ``width`` channels: [t1-t0, width]."""
    assert 0 <= t0 <= t1 <= T_MAX
    out = torch.empty((t1 - t0, width), dtype=dtype, device=device)
    c = torch.arange(width, dtype=torch.int64, device=device)
    for s0 in range(t0, t1, chunk_tokens):
        s1 = min(t1, s0 + chunk_tokens)
        t = torch.arange(s0, s1, dtype=torch.int64, device=device)
        idx = (b * T_MAX + t)[:, None] * width + c[None, :]
        out[s0 - t0:s1 - t0] = _gather(idx, seed, stream, scale, dtype, device)
    return out
