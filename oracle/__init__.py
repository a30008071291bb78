"""CPU oracle for the k-pool DSA indexer selection (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product package never imports it
and has no CPU fallback.
"""
from .kpool_oracle import (  # noqa: F401
    bf16_to_f32,
    f32_to_bf16_rne,
    f64_to_bf16_rne,
    count_pools,
    pool_keys,
    pool_keys_gated,
    row_positions,
    visible_pools,
    row_scores,
    select_row,
    select_row_full_sort,
    expand_row,
    select,
)
