"""Exact trim for speculative decode: the host-side rules (CPU).  A layer retains, for a
trim of up to ``rollback`` tokens, the window ring (W + rollback slots) and the compressor
frontier windows (coff + ceil(rollback / r)); a trim beyond what is still retained raises and
changes nothing.  The bit-exactness of a trim is tested on the GPU (test_gpu_rollback.py)."""
import pytest
import torch

import sparse_attention_dsv4_amd as K
from sparse_attention_dsv4_amd.layer import CsaLayer, LayerSpec

SMALL = LayerSpec(ratio=4, heads=4, dim=64, rope_dim=16, window=16, index_heads=2, index_dim=32,
                  topk=8, dtype=torch.float32, rollback=6)


def _layer(spec=SMALL, batch=2):
    from synth.csa import layer_params
    return CsaLayer(spec, batch, 256, layer_params(spec, 1), device="cpu", max_chunk=16)


def test_state_and_ring_sizes_follow_the_capacity():
    c0 = K.CompCfg(ratio=4, overlap=True, dim=512, rope_dim=64)
    c16 = K.CompCfg(ratio=4, overlap=True, dim=512, rope_dim=64, retain=16)
    c1 = K.CompCfg(ratio=128, overlap=False, dim=512, rope_dim=64, retain=1)
    esz = 2
    assert K.dsv4_comp_state_bytes(c0, 1) == 2 * 2 * 4 * 1024 * esz
    assert K.dsv4_comp_state_bytes(c16, 1) == 2 * (2 + 4) * 4 * 1024 * esz
    assert K.dsv4_comp_state_bytes(c1, 1) == 2 * (1 + 1) * 128 * 512 * esz
    assert K.dsv4_comp_state_bytes(K.CompCfg(4, True, 512, 64, retain=-1), 1) == 0
    layer = _layer()
    assert layer.ring.shape[1] == SMALL.window + SMALL.rollback


def test_trim_room_and_errors():
    layer = _layer()
    layer._advance(10)
    assert layer.rollback_room() == [6, 6]
    layer.trim([2, 6])
    assert layer.lengths == [8, 4] and layer.rollback_room() == [4, 0]
    with pytest.raises(ValueError, match="rollback room"):
        layer.trim([1, 1])                       # sequence 1 has nothing left to take back
    assert layer.lengths == [8, 4]               # a refused trim changes nothing
    layer._advance(1)                            # re-decoding a trimmed position restores room
    assert layer.rollback_room() == [5, 1]
    layer._advance(5)                            # back to (and past) the furthest position
    assert layer.rollback_room() == [6, 6]
    with pytest.raises(ValueError):
        layer.trim(7)
    with pytest.raises(ValueError):
        layer.trim([-1, 0])
    with pytest.raises(ValueError):
        layer.trim([1, 1, 1])


def test_no_capacity_means_no_trim():
    spec = LayerSpec(ratio=128, heads=4, dim=64, rope_dim=16, window=16, indexer=False, topk=0,
                     dtype=torch.float32)
    layer = _layer(spec)
    layer._advance(3)
    assert layer.rollback_room() == [0, 0]
    with pytest.raises(ValueError):
        layer.trim(1)
    layer.trim(0)
    assert layer.lengths == [3, 3]
