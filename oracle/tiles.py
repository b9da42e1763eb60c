"""Tile classes and kv-tile lists from a dense mask (oracle; test infrastructure only).

The tile grid of a sequence starts at its first query row and first key.  For
block sizes (BM, BN) the tile (a, b) covers query rows ``a*BM .. a*BM+BM-1``
and keys ``b*BN .. b*BN+BN-1``; pairs outside the sequence count as not
visible.  A tile is

* EMPTY   (0) when none of its BM*BN pairs is visible,
* FULL    (2) when all BM*BN pairs are visible (so it lies inside the
            sequence and needs neither a mask nor a bounds check),
* PARTIAL (1) otherwise.

Sources: Triton from First Principles, Ch. 21, section 21.2, the tiled causal
diagram (blocks that are all valid, the diagonal block checked per pair, and
blocks skipped without a load); Ch. 9, section 9.2 (a whole tile skipped on one
scalar flag).  Counting out-of-range pairs as not visible -- so an edge tile is
never FULL -- is this project's reading; the diagram instead keeps a bounds
check inside its all-valid blocks.

The lists give, for each query-tile row, the FULL and the PARTIAL kv-tile
indices in ascending order.
"""

from __future__ import annotations

import numpy as np

EMPTY, PARTIAL, FULL = 0, 1, 2


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def classify(vis: np.ndarray, BM: int, BN: int, n_qt: int | None = None,
             n_kt: int | None = None) -> np.ndarray:
    """Class of every tile of one sequence: uint8 ``[n_qt, n_kt]``."""
    Lq, Lk = vis.shape
    n_qt = cdiv(Lq, BM) if n_qt is None else n_qt
    n_kt = cdiv(Lk, BN) if n_kt is None else n_kt
    if n_qt * BM < Lq or n_kt * BN < Lk:
        raise ValueError("tile grid smaller than the sequence")
    padded = np.zeros((n_qt * BM, n_kt * BN), dtype=bool)
    padded[:Lq, :Lk] = vis
    counts = padded.reshape(n_qt, BM, n_kt, BN).sum(axis=(1, 3))
    cls = np.full((n_qt, n_kt), PARTIAL, dtype=np.uint8)
    cls[counts == 0] = EMPTY
    cls[counts == BM * BN] = FULL
    return cls


def lists(cls: np.ndarray):
    """Ascending FULL and PARTIAL kv-tile indices of each query-tile row."""
    full = [np.nonzero(row == FULL)[0].astype(np.int32) for row in cls]
    part = [np.nonzero(row == PARTIAL)[0].astype(np.int32) for row in cls]
    return full, part


def block_sparsity(cls: np.ndarray) -> float:
    """Fraction of tiles that are EMPTY."""
    return float((cls == EMPTY).sum()) / float(cls.size)


def layout_tiles(layout, BM: int, BN: int):
    """Classes and lists of every sequence of a layout, on the shared row grid.

    Rows are numbered ``s * n_qt + a`` with ``n_qt = cdiv(max Lq, BM)`` and
    every row holds ``n_kt = cdiv(max Lk, BN)`` kv tiles, the shape the HIP
    builder writes.  Returns (cls [rows, n_kt] uint8, full_cnt, part_cnt,
    full_idx [rows, n_kt], part_idx [rows, n_kt]) with unused list slots -1.
    """
    from .masks import visible_for_layout

    n_qt = max(cdiv(layout.max_q, BM), 1)
    n_kt = max(cdiv(layout.max_k, BN), 1)
    rows = layout.n_seqs * n_qt
    cls = np.zeros((rows, n_kt), np.uint8)
    for s in range(layout.n_seqs):
        vis = visible_for_layout(layout, s)
        cls[s * n_qt:(s + 1) * n_qt] = classify(vis, BM, BN, n_qt, n_kt)
    full, part = lists(cls)
    full_cnt = np.array([len(x) for x in full], np.int32)
    part_cnt = np.array([len(x) for x in part], np.int32)
    full_idx = np.full((rows, n_kt), -1, np.int32)
    part_idx = np.full((rows, n_kt), -1, np.int32)
    for r in range(rows):
        full_idx[r, :full_cnt[r]] = full[r]
        part_idx[r, :part_cnt[r]] = part[r]
    return cls, full_cnt, part_cnt, full_idx, part_idx


def layout_tile_columns(layout, BM: int, BN: int):
    """The same classes read by kv-tile column: for column ``s * n_kt + b``
    the ascending FULL and PARTIAL query-tile indices a of tiles (a, b) of
    sequence s -- the orientation a pass that owns one kv tile and visits the
    query tiles that see it needs (the xorl issue's transposed block-sparse
    metadata for the backward, section "Verified FA4 gaps").  Returns
    (full_cnt, part_cnt [cols], full_idx, part_idx [cols, n_qt]) with unused
    slots -1."""
    cls = layout_tiles(layout, BM, BN)[0]
    n_kt = cls.shape[1]
    n_qt = cls.shape[0] // max(layout.n_seqs, 1)
    cols = layout.n_seqs * n_kt
    full_cnt = np.zeros(cols, np.int32)
    part_cnt = np.zeros(cols, np.int32)
    full_idx = np.full((cols, n_qt), -1, np.int32)
    part_idx = np.full((cols, n_qt), -1, np.int32)
    for s in range(layout.n_seqs):
        block = cls[s * n_qt:(s + 1) * n_qt]  # [n_qt, n_kt] of sequence s
        for b in range(n_kt):
            c = s * n_kt + b
            f = np.nonzero(block[:, b] == FULL)[0]
            p = np.nonzero(block[:, b] == PARTIAL)[0]
            full_cnt[c], part_cnt[c] = len(f), len(p)
            full_idx[c, :len(f)] = f
            part_idx[c, :len(p)] = p
    return full_cnt, part_cnt, full_idx, part_idx
