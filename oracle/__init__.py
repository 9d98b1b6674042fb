"""CPU float64 oracle for mask-aware attention driven by the column-wise sparse mask.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this package.  The HIP library never calls it, and it shares no code with the HIP
library: it is the plain definition, written out for checking.
"""

from .flashmask_oracle import (  # noqa: F401
    dense_mask,
    unmasked_count,
    mask_storage_bytes,
    fwd_rows,
    bwd_rows,
    attention_fwd,
    attention_bwd,
    block_minmax,
    classify,
    prune_chunks,
    localize,
    localize_chunks_check,
)
