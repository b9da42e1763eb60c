"""Gather of a paged KV history (oracle; test infrastructure only).

A page pool holds ``[num_pages, page_size, ...]`` token rows.  Logical
position ``j`` of a sequence lives in physical page ``block_table[j //
page_size]`` at slot ``j % page_size``, i.e. at flat pool row
``block_table[j // page_size] * page_size + j % page_size`` (the slot mapping).

Source: nanoserve Day 21 "the Triton programming model, modeled on the CPU":
the gather is split into programs that each own one tile of positions; the
last tile is ragged, so a lane past the history is masked, its offset is made
safe before indexing, and it never writes ("What I learned", items 1 and 2,
and the figure caption).  The tile size changes nothing in the result.
"""

from __future__ import annotations

import numpy as np


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def slot_mapping(block_table_row, ctx: int, page_size: int) -> np.ndarray:
    """Flat pool row of each logical position 0 .. ctx-1."""
    bt = np.asarray(block_table_row, dtype=np.int64)
    j = np.arange(ctx, dtype=np.int64)
    return bt[j // page_size] * page_size + (j % page_size)


def paged_gather(pool, block_table_row, ctx: int, page_size: int, tile: int | None = None):
    """Contiguous ``[ctx, ...]`` copy of one sequence's paged history.

    Runs as ``cdiv(ctx, tile)`` programs; program ``p`` owns positions
    ``p*tile .. p*tile+tile-1``.  Returns the same dtype as ``pool``.
    """
    pool = np.asarray(pool)
    n_pages = pool.shape[0]
    assert pool.shape[1] == page_size
    flat = pool.reshape((n_pages * page_size,) + pool.shape[2:])
    bt = np.asarray(block_table_row, dtype=np.int64)
    out = np.zeros((ctx,) + pool.shape[2:], dtype=pool.dtype)
    tile = ctx if tile is None else int(tile)
    if ctx == 0:
        return out
    for prog in range(cdiv(ctx, tile)):
        pos = prog * tile + np.arange(tile, dtype=np.int64)
        live = pos < ctx
        safe = np.where(live, pos, 0)  # a masked lane's offset is neutralised first
        rows = bt[safe // page_size] * page_size + safe % page_size
        vals = flat[rows]
        out[pos[live]] = vals[live]  # masked lanes never write
    return out


def programs(ctx: int, tile: int):
    """Positions owned by each program and which of them are live."""
    out = []
    for prog in range(cdiv(ctx, tile)):
        pos = prog * tile + np.arange(tile)
        out.append((pos, pos < ctx))
    return out
