"""fp64 CPU oracle for exact attention — test infrastructure, never the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. See ``oracle/attention.py`` for what it computes
and which passages of the pages each step follows.
"""
from .attention import (  # noqa: F401
    allowed_pairs,
    attention_backward,
    attention_forward,
    dropout_keep,
    forward_rows,
    kvcache_forward,
    philox4x32_10,
    varlen_backward,
    varlen_forward,
)
