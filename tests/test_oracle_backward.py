"""Pins of oracle.backward and the transposed tile lists (CPU): central finite
differences of the oracle's own forward, float64 autograd of a plain torch
attention, closed forms, and structural invariants."""

import numpy as np
import pytest
import torch

import synth
from oracle import attention, backward, masks, tiles


def _case(rng, Lq, Lk, D, density=0.6, empty_row=False):
    q, k, v, do = (rng.standard_normal(s) for s in ((Lq, D), (Lk, D), (Lk, D), (Lq, D)))
    vis = rng.random((Lq, Lk)) < density
    vis[np.arange(Lq), rng.integers(0, Lk, Lq)] = True  # every row sees a key
    if empty_row:
        vis[0] = False
    return q, k, v, do, vis


def _loss(q, k, v, vis, scale, do):
    o, _ = attention.three_pass(q, k, v, vis, scale)
    return float((o * do).sum())


def test_backward_matches_central_differences():
    # d/dx of sum(O * dO), by central differences of the forward alone.
    rng = np.random.default_rng(0)
    for Lq, Lk, D, er in ((5, 5, 3, False), (4, 7, 2, True), (6, 3, 4, False)):
        q, k, v, do, vis = _case(rng, Lq, Lk, D, empty_row=er)
        scale = 0.7
        dq, dk, dv = backward.sequence_backward(q, k, v, vis, scale, do)
        eps = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args = {"q": q, "k": k, "v": v}
                args[name] = xp
                fp = _loss(args["q"], args["k"], args["v"], vis, scale, do)
                args[name] = xm
                fm = _loss(args["q"], args["k"], args["v"], vis, scale, do)
                fd[idx] = (fp - fm) / (2 * eps)
            np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_matches_torch_autograd_float64():
    rng = np.random.default_rng(1)
    for Lq, Lk, D in ((9, 9, 8), (3, 12, 5), (16, 16, 16)):
        q, k, v, do, vis = _case(rng, Lq, Lk, D, density=0.4)
        scale = 1.0 / np.sqrt(D)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = (tq @ tk.T * scale).masked_fill(~torch.tensor(vis), float("-inf"))
        o = torch.softmax(s, dim=1) @ tv
        o.backward(torch.tensor(do))
        dq, dk, dv = backward.sequence_backward(q, k, v, vis, scale, do)
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_one_visible_key_per_row():
    # P is one-hot: dV gathers dO onto the visible keys, the saturated
    # softmax passes no gradient to the scores, so dQ = dK = 0.
    rng = np.random.default_rng(2)
    Lq, Lk, D = 6, 4, 3
    q, k, v, do = (rng.standard_normal(s) for s in ((Lq, D), (Lk, D), (Lk, D), (Lq, D)))
    pick = rng.integers(0, Lk, Lq)
    vis = np.zeros((Lq, Lk), bool)
    vis[np.arange(Lq), pick] = True
    dq, dk, dv = backward.sequence_backward(q, k, v, vis, 0.5, do)
    expect_dv = np.zeros((Lk, D))
    for i, j in enumerate(pick):
        expect_dv[j] += do[i]
    np.testing.assert_allclose(dv, expect_dv, rtol=0, atol=1e-15)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15


def test_backward_hidden_keys_and_empty_rows_get_nothing():
    rng = np.random.default_rng(3)
    q, k, v, do, vis = _case(rng, 7, 9, 4, empty_row=True)
    vis[:, 2] = False  # key 2 is never visible
    dq, dk, dv = backward.sequence_backward(q, k, v, vis, 0.3, do)
    assert not dk[2].any() and not dv[2].any()
    assert not dq[0].any()  # row 0 sees nothing


def test_backward_layout_is_per_sequence():
    # Packed sequences do not interact: the layout backward equals the
    # per-sequence backward of each piece, and the causal layout's dK of the
    # last key is scale * dS[:, -1]^T Q from the last row alone.
    rng = np.random.default_rng(4)
    lay = synth.random_layout(rng, "shared_prefix", n_seqs=3, max_len=12, H=2, D=4)
    q, k, v = synth.make_dense_qkv(lay, seed=1)
    do = synth.make_dense_qkv(lay, seed=2)[0]
    dQ, dK, dV = backward.backward(lay, q, k, v, do)
    cq, ck = lay.cu_q, lay.cu_k
    f = lambda x, h: x[..., h, :].double().numpy()
    for h in range(2):
        for s in range(lay.n_seqs):
            vis = masks.visible_for_layout(lay, s)
            dq, dk, dv = backward.sequence_backward(
                f(q, h)[cq[s]:cq[s + 1]], f(k, h)[ck[s]:ck[s + 1]], f(v, h)[ck[s]:ck[s + 1]], vis,
                attention.default_scale(lay.head_dim), f(do, h)[cq[s]:cq[s + 1]])
            assert np.array_equal(dQ[cq[s]:cq[s + 1], h], dq)
            assert np.array_equal(dK[ck[s]:ck[s + 1], h], dk)
            assert np.array_equal(dV[ck[s]:ck[s + 1], h], dv)


def test_tile_columns_transpose_the_printed_diagram():
    # Ch. 21, section 21.2's causal diagram (blocks of 4, 16 tokens): read by
    # key block, block b is full for query blocks after it, partial on the
    # diagonal, empty before.
    lay = synth.causal_single(16, 1, 8)
    fc, pc, fi, pi = tiles.layout_tile_columns(lay, 4, 4)
    for b in range(4):
        assert list(fi[b, :fc[b]]) == list(range(b + 1, 4))
        assert list(pi[b, :pc[b]]) == [b]
    assert (fi[3] == -1).all()


@pytest.mark.parametrize("kind", synth.KINDS)
def test_tile_columns_reexpand_to_the_classes(kind):
    rng = np.random.default_rng(5)
    for BM, BN in ((1, 1), (4, 3), (16, 8), (64, 128)):
        lay = synth.random_layout(rng, kind, n_seqs=3, max_len=70)
        cls = tiles.layout_tiles(lay, BM, BN)[0]
        fc, pc, fi, pi = tiles.layout_tile_columns(lay, BM, BN)
        n_kt = cls.shape[1]
        n_qt = cls.shape[0] // lay.n_seqs
        back = np.zeros_like(cls)
        for c in range(lay.n_seqs * n_kt):
            s, b = divmod(c, n_kt)
            assert np.all(np.diff(fi[c, :fc[c]]) > 0) and np.all(np.diff(pi[c, :pc[c]]) > 0)
            back[s * n_qt + fi[c, :fc[c]], b] = tiles.FULL
            back[s * n_qt + pi[c, :pc[c]], b] = tiles.PARTIAL
        assert np.array_equal(back, cls)
