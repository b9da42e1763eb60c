"""Dense visibility masks for one sequence (oracle; test infrastructure only).

A mask is a boolean array ``vis[Lq, Lk]``: ``vis[i, j]`` is True when query
row ``i`` may attend key ``j`` of the same sequence.  Query row ``i`` sits at
absolute position ``(Lk - Lq) + i`` of the sequence, so with ``Lq == Lk`` the
rows are the keys themselves and with one query it is the last position (the
decode case).  This alignment is a reading: the pages only show ``Lq == Lk``.

Sources:
* causal -- Triton from First Principles, Ch. 9 "Mask and Structure Kernels",
  section 9.1 and Worked Example 9.1.1: a key is visible when its column index
  is at most the row index, the diagonal included (Worked Example 9.1.2 shows
  the strict comparison as the bug that drops the diagonal).  The same
  condition is applied per tile in Ch. 21, section 21.2.
* shared_prefix and strip_thinking -- xorl issue "Block-mask attention:
  express shared-prefix and strip-thinking multi-turn training that
  cu_seqlens cannot", section "Mask specifications": both predicates are the
  causal condition AND a condition on per-token ids.
* full -- no mask: Ch. 21, section 21.1's kernel before causal masking.
"""

from __future__ import annotations

import numpy as np


def query_positions(Lq: int, Lk: int) -> np.ndarray:
    """Absolute position of each query row inside its sequence of Lk keys."""
    return np.arange(Lq, dtype=np.int64) + (Lk - Lq)


def visible(kind: str, Lq: int, Lk: int, *, seg_q=None, seg_k=None, role_k=None,
            turn_q=None, turn_k=None, think_role: int = 1) -> np.ndarray:
    """Dense boolean mask ``[Lq, Lk]`` for one sequence.

    ``seg_q``/``turn_q`` are per query row, ``seg_k``/``role_k``/``turn_k``
    per key; each kind reads only the ids it needs.
    """
    qi = query_positions(Lq, Lk)[:, None]
    kj = np.arange(Lk, dtype=np.int64)[None, :]
    if kind == "full":
        return np.ones((Lq, Lk), dtype=bool)
    causal = kj <= qi  # diagonal kept
    if kind == "causal":
        return causal
    if kind == "shared_prefix":
        sq = np.asarray(seg_q, dtype=np.int64)[:, None]
        sk = np.asarray(seg_k, dtype=np.int64)[None, :]
        return causal & ((sk == 0) | (sk == sq))
    if kind == "strip_thinking":
        tq = np.asarray(turn_q, dtype=np.int64)[:, None]
        tk = np.asarray(turn_k, dtype=np.int64)[None, :]
        rk = np.asarray(role_k, dtype=np.int64)[None, :]
        hidden = (rk == think_role) & (tk < tq)
        return causal & ~hidden
    raise ValueError(f"unknown mask kind {kind!r}")


def visible_for_layout(layout, s: int) -> np.ndarray:
    """Dense mask of sequence ``s`` of a ``synth.Layout``."""
    ids = layout.ids_for_seq(s)
    return visible(layout.kind, layout.seqlens_q[s], layout.seqlens_k[s],
                   seg_q=ids.get("seg_q"), seg_k=ids.get("seg_k"), role_k=ids.get("role_k"),
                   turn_q=ids.get("turn_q"), turn_k=ids.get("turn_k"),
                   think_role=layout.think_role)
