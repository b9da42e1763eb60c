"""Seeded synthetic inputs for the masked-attention forward.

Shapes, sequence lengths, per-token id layouts, page tables and random
values only: nothing here computes a mask, a score or a softmax. Both the
CPU oracle tests and the HIP path tests draw their inputs from this package.
"""

from .workloads import (  # noqa: F401
    USER_ROLE,
    THINK_ROLE,
    ANSWER_ROLE,
    LOSS_ROLE,
    HISTORY_ROLE,
    KINDS,
    TERMS,
    Layout,
    causal_single,
    full_single,
    packed_documents,
    shared_prefix,
    strip_thinking,
    strip_thinking_duplicated,
    shared_prefix_groups,
    prefix_lm,
    paged_decode,
    config,
    CONFIG_NAMES,
    random_layout,
    make_dense_qkv,
    make_paged_kv,
    derive_seed,
)
