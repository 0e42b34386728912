"""CPU oracle for the HySparse MQA sparse-attention path (forward and gradients).

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, float64 statement of
what the path computes. Only the tests, the smoke entry point and the
benchmark's CPU-baseline leg may import it; the library and its Python binding
never do. It shares no code with the HIP path and imports nothing from it.

Every function here carries a parity pin in ``tests/test_oracle_pins.py``.
"""
from .hysparse_ref import (  # noqa: F401
    BlockTable,
    block_table,
    block_score,
    topk_blocks,
    sparse_gather,
    swa,
    attend_subset,
    merge_partials,
    block_score_bwd,
    sparse_gather_bwd,
    swa_bwd,
    block_prob,
    gated_combine,
)
