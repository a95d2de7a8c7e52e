"""fp64 CPU oracle of the QSA sparse-prefill operator.

TEST INFRASTRUCTURE ONLY: used by the test suite, the package smoke check and
the benchmark's CPU-baseline leg; never by the product path. It imports
nothing from the GPU package or the input generators.
"""
from .qsa_oracle import (
    D,
    attend,
    bf16_to_f64,
    expand_blocks,
    kv_head_of,
    pool_selected_slots,
    row_probabilities,
    selected_positions,
    sparse_prefill,
    sparse_prefill_blocks,
    sparse_prefill_pool,
)

__all__ = [
    "D",
    "attend",
    "bf16_to_f64",
    "expand_blocks",
    "kv_head_of",
    "pool_selected_slots",
    "row_probabilities",
    "selected_positions",
    "sparse_prefill",
    "sparse_prefill_blocks",
    "sparse_prefill_pool",
]
