"""CPU oracle of PISA's forward path and of the attention backward — test
infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The product package never does.
"""
from .pisa_oracle import (  # noqa: F401
    LevelTrace, RowSelection, attend_row, attend_row_grad, attended_tokens, attention_backward,
    build_pyramid, decode_row, forced_nodes, key_block_grad, last_eligible_node, logsumexp,
    node_children, node_score, padded, pyramid_level_sizes, reduce_logits, select_bsa_row, select_exhaustive_row, select_pisa_row, select_rows,
    top_by_score,
)
from .metrics import selection_quality  # noqa: F401
