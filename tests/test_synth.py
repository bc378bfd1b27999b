"""The seeded input generator: slices regenerate exactly; streams differ; moments are sane."""
import torch

import synth


def test_token_lane_slices_agree():
    full = synth.token_lane(seed=3, stream="a", b=1, t0=0, t1=50, width=24, dtype=torch.bfloat16)
    part = synth.token_lane(seed=3, stream="a", b=1, t0=17, t1=33, width=24, dtype=torch.bfloat16,
                            chunk_tokens=5)
    assert torch.equal(full[17:33], part)


def test_streams_and_sequences_differ():
    a = synth.token_lane(seed=3, stream="a", b=0, t0=0, t1=8, width=16)
    b = synth.token_lane(seed=3, stream="b", b=0, t0=0, t1=8, width=16)
    c = synth.token_lane(seed=3, stream="a", b=1, t0=0, t1=8, width=16)
    d = synth.token_lane(seed=4, stream="a", b=0, t0=0, t1=8, width=16)
    assert not torch.equal(a, b) and not torch.equal(a, c) and not torch.equal(a, d)


def test_normal_offsets_and_moments():
    x = synth.normal((1000, 100), seed=0, stream="x", scale=0.5)
    y = synth.normal((100,), seed=0, stream="x", scale=0.5, offset=500 * 100)
    assert torch.equal(x[500], y)
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 0.5) < 0.01
    # few repeats beyond what a 2**20-entry table implies
    u = torch.unique(x.flatten()).numel()
    assert u > 0.9 * x.numel() * (1 - x.numel() / 2 ** 21)
