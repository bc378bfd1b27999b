"""Code-generation guards checked on the CPU (hipcc cross-compiles for gfx950 here).

The attention and indexer kernels issue their direct-to-LDS tile loads as inline assembly
that writes m0.  m0 is a register the compiler reserves, so such a kernel is only correct
while the compiler itself uses m0 nowhere in it: every m0 reference must be one of those
writes, followed by its load.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_dsv4_amd", "csrc")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


@pytest.mark.parametrize("src,kernel", [
    ("attention.hip", "attn_prefill_kernel"),
    ("attention.hip", "attn_decode_kernel"),
    ("indexer.hip", "index_score_mfma_kernel"),
    ("indexer.hip", "index_score_rs_kernel"),
    ("proj.hip", "gproj_tile_kernel"),
])
def test_m0_only_feeds_lds_dma(tmp_path, src, kernel):
    out = tmp_path / "k.s"
    SRC = os.path.join(CSRC, src)
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-x", "hip",
           "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    starts = [m.start() for m in re.finditer(r"\n(_Z\w*" + kernel + r"\w*):", asm)]
    assert starts, f"{kernel} not found"
    code = []
    for st in starts:
        body = asm[st:asm.index(".Lfunc_end", st)].split("\n")
        code += [l.strip() for l in body if l.strip() and not l.strip().startswith((";", "."))]
    uses = [i for i, l in enumerate(code) if re.search(r"\bm0\b", l)]
    assert uses, "expected the direct-to-LDS loads"
    for i in uses:
        assert code[i].startswith("s_mov_b32 m0,"), f"compiler uses m0: {code[i]}"
        follow = code[i + 1:i + 3]
        assert any(l.startswith("global_load_lds_dwordx4") for l in follow), (code[i], follow)


@pytest.mark.parametrize("kernel", ["attn_prefill_kernel", "attn_decode_kernel"])
def test_dma_base_is_not_sign_extended(tmp_path, kernel):
    """The key-row copies rebuild a 64-bit scalar base from two 32-bit lane reads.  A signed
    widening of the low half (s_bfe_i64 ... 0x200000) would set the upper word of any address
    whose bit 31 is set; no such widening may feed a copy's base registers."""
    out = tmp_path / "k.s"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-x", "hip",
           "--cuda-device-only", "-S", os.path.join(CSRC, "attention.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    st = re.search(r"\n(_Z\w*" + kernel + r"\w*):", asm).start()
    body = asm[st:asm.index(".Lfunc_end", st)].split("\n")
    code = [l.strip() for l in body if l.strip() and not l.strip().startswith((";", "."))]
    dmas = [i for i, l in enumerate(code) if l.startswith("global_load_lds_dwordx4")]
    assert dmas
    for i in dmas:
        m = re.match(r"global_load_lds_dwordx4 v\d+, (s\[\d+:\d+\])", code[i])
        assert m, f"copy without a scalar base: {code[i]}"
        window = code[max(0, i - 16):i]
        assert not any(l.startswith("s_bfe_i64") for l in window), (code[i], window)
        assert code[i - 1].startswith("s_nop 4"), (code[i - 1], code[i])
