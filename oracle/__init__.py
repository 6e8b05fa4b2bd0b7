"""CPU float64 oracle (test infrastructure only; see oracle/attention.py)."""
from .attention import (  # noqa: F401
    attention_bwd,
    attention_bwd_key_rows,
    attention_bwd_query_rows,
    attention_fwd,
    attention_fwd_partial,
    attention_fwd_rows,
    merge_partials,
    row_stats,
)
