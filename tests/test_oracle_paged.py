"""Pins of oracle.paged and the paged oracle forward (CPU)."""

import math

import numpy as np
import torch

import _golden
import synth
from oracle import attention, masks, paged
from oracle import forward as oforward


def _scatter_history(hist, page_size, rng, extra_pages=3):
    """Write a contiguous history into a pool page by page, in a shuffled page
    order; returns (pool, block_table_row).  The inverse of a gather."""
    ctx = hist.shape[0]
    n = math.ceil(ctx / page_size)
    n_pages = n + extra_pages
    order = rng.permutation(n_pages)[:n]
    pool = np.full((n_pages, page_size) + hist.shape[1:], -7.0, hist.dtype)
    for p in range(n):
        chunk = hist[p * page_size:(p + 1) * page_size]
        pool[order[p], :chunk.shape[0]] = chunk
    return pool, order


def test_gather_byte_equal_for_every_tile_size():
    # nanoserve Day 21: a 13-token history, tile sizes 1, 2, 3, 4, 8, 13, 20.
    g = _golden.load("paged_gather.txt")
    rng = np.random.default_rng(0)
    ctx = int(g["history_tokens"])
    hist = rng.standard_normal((ctx, 2, 8)).astype(np.float32)
    for page_size in (1, 2, 4, 5, 16):
        pool, bt = _scatter_history(hist, page_size, rng)
        for tile in g["tile_sizes"].astype(int):
            out = paged.paged_gather(pool, bt, ctx, page_size, tile=int(tile))
            assert out.tobytes() == hist.tobytes(), (page_size, tile)


def test_gather_equals_slot_mapping_index():
    rng = np.random.default_rng(1)
    hist = rng.standard_normal((29, 3)).astype(np.float32)
    pool, bt = _scatter_history(hist, 4, rng)
    flat = pool.reshape(-1, 3)
    assert flat[paged.slot_mapping(bt, 29, 4)].tobytes() == hist.tobytes()


def test_program_grid_of_figure_example():
    # Figure caption: 10 tokens in tiles of 4 -> 3 programs; program 2 owns
    # positions 8, 9 (live) and 10, 11 (masked).
    g = _golden.load("paged_gather.txt")
    progs = paged.programs(int(g["example_tokens"]), int(g["example_tile"]))
    assert len(progs) == int(g["example_programs"])
    pos, live = progs[2]
    assert list(pos[live]) == list(g["program2_live"].astype(int))
    assert list(pos[~live]) == list(g["program2_masked"].astype(int))


def test_ragged_rows_through_pages():
    # Ch. 9, Worked Example 9.3.1: rows of real length 4, 2, 3 padded with 999.
    # Seen as three paged sequences (one 4-slot page each, contexts 4, 2, 3)
    # and attended by a zero query (equal scores), the output is the mean of
    # the live values; times the length it is the printed row sum.  A gather
    # that read past the context would pull in the 999 padding.
    g = _golden.load("ragged_rows.txt")
    lens = g["lengths"].astype(int).tolist()
    pool = g["padded"].reshape(3, 4, 1, 1)  # [pages, page_size, H, D]
    lay = synth.Layout("ragged", "causal", "f32", 1, 1, [1, 1, 1], lens, paged=True, page_size=4)
    bt = np.array([[0], [1], [2]], np.int32)
    q = np.zeros((3, 1, 1))
    O, _ = oforward.forward(lay, q, k_pool=np.zeros_like(pool), v_pool=pool, block_table=bt)
    assert np.allclose(O[:, 0, 0] * np.array(lens), g["row_sums"], rtol=0, atol=1e-12)


def test_paged_forward_equals_contiguous_forward():
    lay = synth.paged_decode(seed=2, n_seqs=3, lo=5, hi=40, page_size=4, H=2, D=8, dtype="f32")
    q, kp, vp, bt = synth.make_paged_kv(lay, seed=2, extra_pages=2)
    O, lse = oforward.forward(lay, q, k_pool=kp, v_pool=vp, block_table=bt)
    # Contiguous copies built with torch indexing (the slot mapping).
    for s in range(lay.n_seqs):
        ctx = lay.seqlens_k[s]
        slots = torch.from_numpy(paged.slot_mapping(bt[s].numpy(), ctx, 4))
        for h in range(2):
            K = kp[:, :, h].reshape(-1, 8)[slots]
            V = vp[:, :, h].reshape(-1, 8)[slots]
            o, l = attention.three_pass(q[s:s + 1, h], K, V, masks.visible("causal", 1, ctx),
                                        1 / math.sqrt(8))
            assert np.array_equal(O[s:s + 1, h], o)
            assert np.array_equal(lse[h, s:s + 1], l)
