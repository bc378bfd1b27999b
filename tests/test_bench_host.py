"""Host-side logic of bench.py (no GPU): the one-GPU guard, and the traffic lookup that
reports an HBM-traffic summary only for the kernel and kernel sources it was measured on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr


def test_traffic_lookup_follows_the_sources(tmp_path):
    """A summary counts only for the kernel it names and the sources it was measured on."""
    for kernel in ("index_score_rs", "index_score_stream", "attn_decode"):
        digest = bench.kernel_source_digest(kernel)
        prof = tmp_path / f"traffic_{kernel}.txt"
        prof.write_text("# header line: ignored\n"
                        f"kernel: {kernel}\nsource_digest: {digest}\n"
                        "traffic_bytes_per_launch: 12345\n")
        assert bench.traffic_from_profile(str(prof), kernel) == 12345.0
        other = "compress_rows" if kernel != "compress_rows" else "attn_decode"
        assert bench.traffic_from_profile(str(prof), other) is None        # another kernel
        prof.write_text(prof.read_text().replace(digest, "0" * 16))
        assert bench.traffic_from_profile(str(prof), kernel) is None       # other sources
    assert bench.traffic_from_profile(str(tmp_path / "absent.txt"), "index_score_rs") is None


def test_source_digest_per_kernel_family():
    d = {k: bench.kernel_source_digest(k) for k in ("attn_decode", "index_score_rs",
                                                   "index_score_stream", "compress_rows")}
    assert d["index_score_rs"] == d["index_score_stream"]     # one source file
    assert len({d["attn_decode"], d["index_score_rs"], d["compress_rows"]}) == 3
    assert all(len(v) == 16 for v in d.values())


# ------------------------------------------------------------------ CPU-baseline legs
TINY4 = dict(ratio=4, heads=4, dim=64, rope_dim=16, window=16, index_heads=2, index_dim=32, topk=8)


def _tiny(**kw):
    import torch
    from sparse_attention_dsv4_amd.layer import LayerSpec
    return LayerSpec(**{**TINY4, **kw}, dtype=torch.float32)


def test_cpu_baseline_decode_runs_the_sampled_steps():
    """Any step and warm-up count: the decode sample builds its own inputs and cache, so it
    does not depend on how many steps the GPU part ran (the driver's --steps 20 --warmup 5
    made an earlier version index past its inputs).  The sample holds one row emission per
    sequence per r steps."""
    spec = _tiny(ratio=8, indexer=False, topk=0)
    res = bench.cpu_baseline_decode(spec, 0, 70, n_seq=2, steps=9, device="cpu")
    assert res["kind"] == "oracle" and res["unit"] == "tokens/s" and res["value"] > 0
    assert res["cores"] >= 1
    assert "9 decode steps x 2 sequences" in res["sample"]
    assert "2 row emissions" in res["sample"]          # p = 71 completes row 8 in each sequence


def test_cpu_baseline_prefill_runs_the_sampled_queries():
    spec = _tiny()
    res = bench.cpu_baseline_prefill(spec, 1, 96, 32, n_queries=5, device="cpu")
    assert res["kind"] == "oracle" and res["value"] > 0
    assert "5 of the 32 queries" in res["sample"]


def test_oracle_prefix_rows_blocks_equal_one_pass():
    """Building the prefix rows block by block (with the overlap's previous window carried
    into each block) gives the one-pass rows."""
    import numpy as np
    import oracle
    import synth.csa as SC
    for spec in (_tiny(), _tiny(ratio=8, overlap=False)):
        n = 75
        blk = bench.oracle_prefix_rows(spec, 3, 1, n, block=16)
        tok = {k: v.double().numpy() for k, v in SC.token_inputs(spec, 3, 1, 0, n).items()}
        par = {k: v.double().numpy() for k, v in SC.layer_params(spec, 3).items()}
        one = oracle.compressor_rows(tok["a"][:n - n % spec.ratio], tok["g"][:n - n % spec.ratio],
                                     par["ape"], par["norm_w"], par["inv_freq"], ratio=spec.ratio,
                                     overlap=spec.is_overlap, eps=spec.eps, store="f32")
        assert np.array_equal(blk, one)


def test_decode_step_bytes_of_the_headline_layer():
    """Batch 8 at 64K on the ratio-128 layer: q and out 64 KiB each, 640 keys of 1 KiB, the
    ring store, the lane stores and 1/128 of an emission per sequence: about 6.35 MB."""
    import torch
    from sparse_attention_dsv4_amd.layer import LayerSpec
    spec = LayerSpec(ratio=128, indexer=False, topk=0)
    by = bench.decode_step_bytes(spec, 8, [65536])
    per_seq_attn = 2 * 64 * 512 * 2 + 640 * 1024 + 1024
    assert by["attention"] == 8 * per_seq_attn
    assert by["compressor"] == 8 * (2 * 1024 * 2 + (2 * 128 * 512 * 2 + 1024) / 128)
    assert abs(by["total"] - 6.35e6) < 0.05e6
    assert torch.bfloat16 == spec.dtype


def test_prefill_flops_of_the_headline_chunk():
    from sparse_attention_dsv4_amd.layer import LayerSpec
    fl = bench.prefill_chunk_flops(LayerSpec(ratio=4), 63488, 2048)
    assert abs(fl["total"] - 0.713e12) < 0.01e12
    assert abs(fl["indexer"] - 0.541e12) < 0.01e12


def test_emission_positions():
    assert bench.emission_positions(65536, 20, 128) == 0
    assert bench.emission_positions(65536, 128, 128) == 1
    assert bench.emission_positions(65535, 1, 128) == 1
    assert bench.emission_positions(0, 20, 4) == 5
    assert bench.emission_positions(5, 10, 0) == 0
