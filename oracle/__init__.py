"""CPU oracle for the HCA layer forward: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never does.
"""
from .hca_oracle import (  # noqa: F401
    BLOCK,
    attend_decode,
    attend_prefill,
    blocks_per_sequence,
    cache_entries,
    compress,
    cu_blocks_from_cu_seqlens,
    head_mix_and_gate,
    pooling_weights,
    visible_sets,
)
from .hca_backward import attend_prefill_backward, loss_for_gradcheck  # noqa: F401,E402
from .dsa_oracle import attend_selected, dsa_decode, index_scores, select_topk  # noqa: F401,E402
