"""CPU oracle (test infrastructure): see clsa_oracle.py for what it defines."""
from .clsa_oracle import (  # noqa: F401
    attend_head,
    kv_head_of,
    route,
    route_scores,
    route_threshold,
    sparse_attn,
    threshold_select,
    topk_select,
    visible_count,
)
