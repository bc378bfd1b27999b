"""Code-generation guards checked on the CPU (hipcc cross-compiles for gfx950 here).

The attention kernel issues its direct-to-LDS key loads as inline assembly that writes m0.
m0 is a register the compiler reserves, so the kernel is only correct while the compiler
itself uses m0 nowhere in that kernel: every m0 reference must be one of those writes,
followed by its load.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "sparse_attention_dsv4_amd", "csrc", "attention.hip")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


def test_attention_kernel_m0_only_feeds_lds_dma(tmp_path):
    out = tmp_path / "attention.s"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-x", "hip",
           "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    m = re.search(r"\n(_Z\w*attn_mfma_kernel\w*):", asm)
    assert m, "attention kernel not found"
    body = asm[m.start():asm.index(".Lfunc_end", m.start())].split("\n")
    code = [l.strip() for l in body if l.strip() and not l.strip().startswith((";", "."))]
    uses = [i for i, l in enumerate(code) if re.search(r"\bm0\b", l)]
    assert uses, "expected the direct-to-LDS loads"
    for i in uses:
        assert code[i].startswith("s_mov_b32 m0,"), f"compiler uses m0: {code[i]}"
        follow = code[i + 1:i + 3]
        assert any(l.startswith("global_load_lds_dwordx4") for l in follow), (code[i], follow)
