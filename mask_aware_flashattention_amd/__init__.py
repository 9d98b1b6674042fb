"""Mask-aware fused attention for MI355X (gfx950) driven by FlashMask's column-wise sparse mask.

The computation lives in ``libflashmask.so`` (hand-written HIP kernels behind a C ABI declared
in ``include/flashmask.h``); this package is its thin torch binding.
"""

from ._lib import FlashMaskError, load as load_library  # noqa: F401
from .api import (  # noqa: F401
    block_order,
    bwd,
    bwd_ex,
    bwd_workspace_bytes,
    classify,
    fwd,
    fwd_ex,
    fwd_noalloc,
    fwd_workspace_bytes,
    localize,
    prune_chunks,
    tile_sizes,
)
