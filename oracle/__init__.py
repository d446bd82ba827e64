"""Reference oracle for Re-ttention-style sparse attention reshape.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
the test-suite, the smoke check and the CPU-baseline leg of the benchmark do.
It shares no code with the HIP path.
"""
from . import hilbert  # noqa: F401
from .rettention import (  # noqa: F401
    BLOCK,
    block_ranges,
    pool_blocks,
    pooled_scores,
    select_from_scores,
    select_blocks,
    dense_attention,
    calibrate,
    sparse_reshape,
    calibrate_rows,
    sparse_reshape_rows,
    sparse_reshape_r2,
    sparse_reshape_rows_r2,
    closed_form_fp64,
    kept_flops,
)
