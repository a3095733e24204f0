"""Exact tiled scaled-dot-product attention for MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``include/attn.h`` (``libattn.so``, built in-tree by
``python -m exact_tiled_attention_attn_amd.build``).  This package is the
thin Python binding: ``fwd`` / ``bwd`` / ``debug_tile_map`` marshal torch
device tensors into the ABI and allocate outputs and workspace with torch;
``attention`` / ``self_attention`` register the backward with torch.autograd
(saved state: Q, K, V, O and L).
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MASK_MODES,
    AttnError,
    AttnProblem,
    bwd,
    bwd_noalloc,
    count_tiles,
    debug_tile_map,
    dropout_mask,
    fwd,
    load_library,
    make_problem,
    timing_enable,
    timing_read,
    workspace_size,
)
from .autograd import attention, self_attention  # noqa: F401

__all__ = ["fwd", "bwd", "attention", "self_attention", "debug_tile_map", "workspace_size",
           "load_library", "AttnError"]
