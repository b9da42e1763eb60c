"""Pins of oracle.tiles: the printed tile diagram, a closed form and invariants (CPU)."""

import numpy as np

import _golden
import synth
from oracle import masks, tiles


def test_tile_classes_match_printed_diagram():
    # Ch. 21, section 21.2 diagram: query rows 8-11 at BLOCK 4.
    g = _golden.load("causal_tile_diagram.txt")
    B, L, a = int(g["block"]), int(g["seq_len"]), int(g["query_block"])
    cls = tiles.classify(masks.visible("causal", L, L), B, B)
    assert np.array_equal(cls[a], g["classes"][0].astype(np.uint8))


def _causal_class_closed_form(L, BM, BN, a, b):
    """Tile class of a causal self-attention sequence, from geometry alone."""
    q0, q1 = a * BM, min((a + 1) * BM, L)
    k0, k1 = b * BN, min((b + 1) * BN, L)
    if q0 >= L or k0 >= L or k0 > q1 - 1:
        return tiles.EMPTY
    inside = (a + 1) * BM <= L and (b + 1) * BN <= L
    if inside and (b + 1) * BN - 1 <= q0:
        return tiles.FULL
    return tiles.PARTIAL


def test_causal_classes_match_closed_form():
    for L in (1, 5, 16, 37, 64, 100):
        vis = masks.visible("causal", L, L)
        for BM in (1, 2, 3, 4, 8, 13, 16):
            for BN in (1, 2, 3, 4, 8, 13, 16):
                n_qt, n_kt = tiles.cdiv(L, BM) + 1, tiles.cdiv(L, BN) + 1  # extra empty row/col
                cls = tiles.classify(vis, BM, BN, n_qt, n_kt)
                expect = np.array([[_causal_class_closed_form(L, BM, BN, a, b)
                                    for b in range(n_kt)] for a in range(n_qt)], np.uint8)
                assert np.array_equal(cls, expect), (L, BM, BN)


def test_causal_block_sparsity_near_page_figure():
    # xorl issue, "Measured": causal is quoted as 48% sparse next to 128x128
    # blocks; at S=4096 the empty fraction is 48.4%.
    cls = tiles.classify(masks.visible("causal", 4096, 4096), 128, 128)
    assert abs(tiles.block_sparsity(cls) - 0.484375) < 1e-12
    assert round(tiles.block_sparsity(cls) * 100) == 48


def _expand(cls, vis, BM, BN):
    """Dense mask rebuilt from classes: FULL -> all, EMPTY -> none, PARTIAL -> predicate."""
    Lq, Lk = vis.shape
    out = np.zeros_like(vis)
    for a in range(cls.shape[0]):
        for b in range(cls.shape[1]):
            rs = slice(a * BM, min((a + 1) * BM, Lq))
            cs = slice(b * BN, min((b + 1) * BN, Lk))
            if cls[a, b] == tiles.FULL:
                out[rs, cs] = True
            elif cls[a, b] == tiles.PARTIAL:
                out[rs, cs] = vis[rs, cs]
    return out


def test_expansion_reproduces_dense_mask_random_layouts():
    rng = np.random.default_rng(5)
    for kind in synth.KINDS:
        for decode_q in (None, 1, 3):
            lay = synth.random_layout(rng, kind, n_seqs=2, max_len=45, decode_q=decode_q)
            for s in range(lay.n_seqs):
                vis = masks.visible_for_layout(lay, s)
                for BM in (1, 2, 3, 4, 8, 13, 16, 64):
                    for BN in (1, 2, 3, 4, 8, 13, 16, 64):
                        cls = tiles.classify(vis, BM, BN)
                        assert np.array_equal(_expand(cls, vis, BM, BN), vis)
                        # FULL tiles hold BM*BN visible pairs, EMPTY none, PARTIAL
                        # some but not all.
                        Lq, Lk = vis.shape
                        pad = np.zeros((cls.shape[0] * BM, cls.shape[1] * BN), bool)
                        pad[:Lq, :Lk] = vis
                        cnt = pad.reshape(cls.shape[0], BM, cls.shape[1], BN).sum(axis=(1, 3))
                        assert (cnt[cls == tiles.FULL] == BM * BN).all()
                        assert (cnt[cls == tiles.EMPTY] == 0).all()
                        p = cnt[cls == tiles.PARTIAL]
                        assert ((p > 0) & (p < BM * BN)).all()


def test_edge_tiles_never_full():
    vis = masks.visible("full", 10, 10)
    cls = tiles.classify(vis, 4, 4)
    assert cls[2, 0] == tiles.PARTIAL and cls[0, 2] == tiles.PARTIAL
    assert cls[0, 0] == tiles.FULL


def test_lists_ascending_and_layout_grid():
    lay = synth.packed_documents(seed=0, n_docs=3, lo=5, hi=40, H=1, D=8)
    BM, BN = 8, 4
    cls, fc, pc, fi, pi = tiles.layout_tiles(lay, BM, BN)
    n_qt = tiles.cdiv(lay.max_q, BM)
    assert cls.shape == (lay.n_seqs * n_qt, tiles.cdiv(lay.max_k, BN))
    for r in range(cls.shape[0]):
        f = fi[r, :fc[r]]
        p = pi[r, :pc[r]]
        assert (np.diff(f) > 0).all() and (np.diff(p) > 0).all()
        assert (fi[r, fc[r]:] == -1).all() and (pi[r, pc[r]:] == -1).all()
        assert set(f) == set(np.nonzero(cls[r] == tiles.FULL)[0])
        assert set(p) == set(np.nonzero(cls[r] == tiles.PARTIAL)[0])
    # Rows past a short sequence's last query tile are all EMPTY.
    for s, L in enumerate(lay.seqlens_q):
        used = tiles.cdiv(L, BM)
        assert (cls[s * n_qt + used:(s + 1) * n_qt] == tiles.EMPTY).all()


def test_config_tile_counts():
    # Shared-prefix (4096 + 16 x 1024) at 128x128, counted by hand: the prefix
    # is a 32-tile causal triangle (32*31/2 = 496 full, 32 diagonal partial);
    # each suffix's 8 query tiles see all 32 prefix tiles (256 full) and its
    # own 8-tile triangle (28 full, 8 partial).  Full 496 + 16*284 = 5040,
    # partial 32 + 16*8 = 160, empty 25600 - 5200 = 20400.
    lay = synth.shared_prefix()
    T = lay.total_q
    vis = masks.visible_for_layout(lay, 0)
    cls = tiles.classify(vis, 128, 128)
    assert cls.shape == (T // 128, T // 128)
    assert (cls == tiles.PARTIAL).sum() == 160
    assert (cls == tiles.FULL).sum() == 5040
    assert abs(tiles.block_sparsity(cls) - 20400 / 25600) < 1e-12
