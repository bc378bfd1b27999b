"""CPU oracle for the DeepSeek-V4-Flash compressed sparse attention (CSA) layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it.  It shares no code with the HIP path.

Plain numpy, one function per step of the layer, written from the pages' statement of what
each step computes (see the docstrings for the passage each follows).  Working precision is
a parameter: ``np.float32`` (default; the pages fix fp32 pooling, softmax and scoring) or
``np.float64`` (used by the closed-form pins).
"""
from .csa import (  # noqa: F401
    bf16_round,
    round_store,
    rope_rows,
    rms_norm,
    compressor_rows,
    rows_completed,
    visible_rows,
    index_scores,
    select_topk,
    rope_heads,
    grouped_out_proj,
    csa_attention,
)
