"""Block-sparse masked attention (forward and backward) for AMD MI355X (gfx950).

The computation lives in the HIP library ``lib/libbmattn.so`` (C ABI in
include/bmattn.h); ``bmattn`` is its ctypes binding.  Build it with
``python -m block_sparse_masked_amd.build``.
"""

from . import bmattn  # noqa: F401

# The library is loaded on first use: every entry point raises ImportError
# when it is not built (or lacks a symbol), and nothing else runs in its
# place.  Loading it here would keep `python -m block_sparse_masked_amd.build`
# from running over a missing or stale library.
from .bmattn import (  # noqa: F401
    BlockMask,
    BmattnError,
    MaskDesc,
    build_block_mask,
    debug_dense_mask,
    forward,
    forward_workspace_size,
    paged_gather,
    validate,
    transpose_block_mask,
    build_backward_cols,
    backward,
    backward_workspace_size,
    duplicated_answer_ids,
    relabel,
)
