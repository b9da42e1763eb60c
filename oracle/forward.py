"""Oracle forward over a whole layout (test infrastructure only).

Loops over sequences and heads and applies ``attention.three_pass`` to the
dense mask of each sequence.  Inputs may be torch tensors (any device, bf16
or fp32: they are widened exactly to float64 on the host) or numpy arrays.

Outputs: O ``[total_q, H, Dv]`` float64 and LSE ``[H, total_q]`` float64.
"""

from __future__ import annotations

import numpy as np

from .attention import three_pass, default_scale
from .masks import visible_for_layout
from .paged import paged_gather


def to_f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def head_slice(x, h: int):
    """Head ``h`` of a ``[..., H, D]`` tensor, widened to float64."""
    if x is None:
        return None
    return to_f64(x[..., h, :])


def sequence_kv(layout, s: int, kh: np.ndarray, vh: np.ndarray, block_table=None):
    """K and V ``[Lk, D]`` of sequence ``s`` for one head.

    ``kh``/``vh`` are ``[total_k, D]`` for contiguous layouts, or page pools
    ``[num_pages, page_size, D]`` for paged layouts (gathered through row ``s``
    of ``block_table``).
    """
    if layout.paged:
        bt = np.asarray(block_table[s].cpu() if hasattr(block_table, "cpu") else block_table[s])
        ctx = layout.seqlens_k[s]
        return (paged_gather(kh, bt, ctx, layout.page_size),
                paged_gather(vh, bt, ctx, layout.page_size))
    cu = layout.cu_k
    return kh[cu[s]:cu[s + 1]], vh[cu[s]:cu[s + 1]]


def sequence_head(layout, s: int, qh, kh, vh, block_table=None, scale=None, rows=None):
    """O and LSE of sequence ``s`` for one head; ``rows`` selects query rows."""
    scale = default_scale(layout.head_dim) if not scale else scale
    K, V = sequence_kv(layout, s, kh, vh, block_table)
    cu = layout.cu_q
    qs = qh[cu[s]:cu[s + 1]]
    vis = visible_for_layout(layout, s)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        qs = qs[rows]
        vis = vis[rows]
    return three_pass(qs, K, V, vis, scale)


def forward(layout, q, k=None, v=None, *, k_pool=None, v_pool=None, block_table=None,
            scale=None, heads=None):
    """O ``[total_q, H, Dv]`` and LSE ``[H, total_q]`` for every sequence."""
    H = layout.num_heads
    heads = range(H) if heads is None else heads
    Dv = layout.head_dim
    O = np.zeros((layout.total_q, H, Dv), np.float64)
    lse = np.full((H, layout.total_q), -np.inf, np.float64)
    cu = layout.cu_q
    for h in heads:
        qh = head_slice(q, h)
        if layout.paged:
            kh, vh = head_slice(k_pool, h), head_slice(v_pool, h)
        else:
            kh, vh = head_slice(k, h), head_slice(v, h)
        for s in range(layout.n_seqs):
            o, l = sequence_head(layout, s, qh, kh, vh, block_table, scale)
            O[cu[s]:cu[s + 1], h] = o
            lse[h, cu[s]:cu[s + 1]] = l
    return O, lse
