"""Host-side checks of cross-layer KV sharing (no GPU): a sharing layer refuses an owner whose
rows it cannot read, and takes its positions from the owner's lengths."""
import pytest

import synth.csa as SC
from sparse_attention_dsv4_amd.layer import CsaLayer, LayerSpec, SharedCsaLayer

SMALL = LayerSpec(ratio=4, heads=8, dim=64, rope_dim=16, window=16, index_heads=4, index_dim=32,
                  topk=16)


def _owner(spec=SMALL):
    return CsaLayer(spec, 2, 64, SC.layer_params(spec, 1), device="cpu", max_chunk=64)


def test_owner_mismatches_raise():
    owner = _owner()
    for bad in (LayerSpec(ratio=4, heads=8, dim=32, rope_dim=16, window=16, index_heads=4,
                          index_dim=32, topk=16),                        # other latent width
                LayerSpec(ratio=128, heads=8, dim=64, rope_dim=16, window=16, index_heads=4,
                          index_dim=32, topk=16)):                      # other ratio
        with pytest.raises(ValueError):
            SharedCsaLayer(bad, owner, SC.layer_params(bad, 2), device="cpu")
    other_idx = LayerSpec(ratio=4, heads=8, dim=64, rope_dim=16, window=16, index_heads=2,
                          index_dim=32, topk=16)
    with pytest.raises(ValueError):                                      # other index width
        SharedCsaLayer(other_idx, owner, SC.layer_params(other_idx, 2), index="own", device="cpu")
    k8 = LayerSpec(ratio=4, heads=8, dim=64, rope_dim=16, window=16, index_heads=4, index_dim=32,
                   topk=8)
    with pytest.raises(ValueError):                                      # other top-k
        SharedCsaLayer(k8, owner, SC.layer_params(k8, 2), index="owner", device="cpu")
    with pytest.raises(ValueError):
        SharedCsaLayer(SMALL, owner, SC.layer_params(SMALL, 2), index="bogus", device="cpu")
    no_idx = LayerSpec(ratio=4, heads=8, dim=64, rope_dim=16, window=16, indexer=False, topk=0)
    with pytest.raises(ValueError):                                      # owner has no indexer
        SharedCsaLayer(SMALL, _owner(no_idx), SC.layer_params(SMALL, 2), index="owner", device="cpu")


def test_positions_follow_the_owner():
    owner = _owner()
    layer = SharedCsaLayer(SMALL, owner, SC.layer_params(SMALL, 2), index="own", device="cpu")
    assert layer.ring.shape == (2, SMALL.window, SMALL.dim)
    owner.lengths = [40, 17]                    # the owner has taken these tokens already
    assert layer._positions(8) == [32, 9]
    assert layer._positions(1) == [39, 16]
