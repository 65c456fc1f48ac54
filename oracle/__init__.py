"""fp64 CPU oracle for exact softmax attention -- test infrastructure only.

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the product path never touches it.
"""
from .attention import (  # noqa: F401
    attention_bwd,
    attention_bwd_gqa,
    attention_bwd_varlen,
    attention_gqa,
    attention_varlen,
    attention_from_scores,
    combine_partials,
    naive_attention,
    scores,
    split_kv_partials,
    tiled_attention,
)
from .fp8 import attention_fp8, e4m3_to_f64  # noqa: F401
