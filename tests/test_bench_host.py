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
