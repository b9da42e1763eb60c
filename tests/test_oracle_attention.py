"""Pins of oracle.attention: printed values, brute force, closed forms,
library special cases and the invariants of the masked workloads (CPU)."""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import _golden
import synth
from oracle import attention, masks, tiles
from oracle import forward as oforward


def test_noncausal_vs_causal_printed_difference():
    # Ch. 21, Worked Example 21.2.2 with the chapter's inputs.
    g = _golden.load("noncausal_vs_causal.txt")
    torch.manual_seed(int(g["seed"]))
    M, N, D = int(g["M"]), int(g["N"]), int(g["D"])
    q = torch.randn(M, D)
    k = torch.randn(N, D)
    v = torch.randn(N, D)
    scale = 1.0 / math.sqrt(D)
    o_full, _ = attention.three_pass(q, k, v, masks.visible("full", M, N), scale)
    o_causal, _ = attention.three_pass(q, k, v, masks.visible("causal", M, N), scale)
    diff = np.abs(o_full - o_causal).max()
    # The page computed in float32; the oracle in float64 on the same inputs.
    assert abs(diff - g["max_abs_diff_fp32"]) < 1e-6


def test_noncausal_matches_library_softmax():
    # Ch. 21, Worked Example 21.1.1's shapes (M=17, N=23, D=8, seed 0); the
    # naive oracle is torch.softmax(q @ k.T * scale) @ v, run here in float64.
    torch.manual_seed(0)
    q, k, v = torch.randn(17, 8), torch.randn(23, 8), torch.randn(23, 8)
    scale = 1.0 / math.sqrt(8)
    o, lse = attention.three_pass(q, k, v, masks.visible("full", 17, 23), scale)
    q64, k64, v64 = q.double(), k.double(), v.double()
    ref = torch.softmax(q64 @ k64.T * scale, dim=-1) @ v64
    assert np.abs(o - ref.numpy()).max() < 1e-13
    ref_lse = torch.logsumexp(q64 @ k64.T * scale, dim=-1)
    assert np.abs(lse - ref_lse.numpy()).max() < 1e-13


def test_causal_matches_library_masked_softmax():
    # Ch. 21, section 21.2's naive causal oracle: masked_fill(~tril, -inf).
    torch.manual_seed(1)
    M = 20
    q, k, v = (torch.randn(M, 8, dtype=torch.float64) for _ in range(3))
    scale = 1.0 / math.sqrt(8)
    tril = torch.tril(torch.ones(M, M, dtype=torch.bool))
    ref = torch.softmax((q @ k.T * scale).masked_fill(~tril, float("-inf")), dim=-1) @ v
    o, _ = attention.three_pass(q, k, v, masks.visible("causal", M, M), scale)
    assert np.abs(o - ref.numpy()).max() < 1e-13


def _brute(q, k, v, vis, scale):
    """Pair-by-pair with exactly rounded sums (math.fsum)."""
    Lq, Lk = vis.shape
    O = np.zeros((Lq, v.shape[1]))
    lse = np.full(Lq, -np.inf)
    for i in range(Lq):
        js = [j for j in range(Lk) if vis[i, j]]
        if not js:
            continue
        s = {j: math.fsum(float(q[i, d]) * float(k[j, d]) for d in range(q.shape[1])) * scale
             for j in js}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in js}
        tot = math.fsum(w.values())
        for d in range(v.shape[1]):
            O[i, d] = math.fsum(w[j] / tot * float(v[j, d]) for j in js)
        lse[i] = m + math.log(tot)
    return O, lse


@pytest.mark.parametrize("kind", synth.KINDS)
def test_three_pass_matches_brute_force(kind):
    rng = np.random.default_rng(21)
    for decode_q in (None, 2):
        lay = synth.random_layout(rng, kind, n_seqs=2, max_len=12, D=5, decode_q=decode_q)
        for s in range(lay.n_seqs):
            vis = masks.visible_for_layout(lay, s)
            Lq, Lk = vis.shape
            q, k, v = rng.standard_normal((Lq, 5)), rng.standard_normal((Lk, 5)), \
                rng.standard_normal((Lk, 4))
            o, lse = attention.three_pass(q, k, v, vis, 0.37)
            ob, lb = _brute(q, k, v, vis, 0.37)
            assert np.abs(o - ob).max() < 1e-13
            fin = np.isfinite(lb)
            assert np.array_equal(fin, np.isfinite(lse))
            assert np.abs(lse[fin] - lb[fin]).max(initial=0) < 1e-13


def test_single_visible_key_closed_form():
    # One visible key: the output is that key's value row and LSE its score.
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal((1, 6)), rng.standard_normal((4, 6)), rng.standard_normal((4, 3))
    for j in range(4):
        vis = np.zeros((1, 4), bool)
        vis[0, j] = True
        o, lse = attention.three_pass(q, k, v, vis, 0.5)
        assert np.abs(o[0] - v[j]).max() < 1e-15
        assert abs(lse[0] - 0.5 * float(q[0] @ k[j])) < 1e-14


def test_equal_scores_closed_form():
    # Equal scores: the output is the mean of the visible values and
    # LSE = s + ln(n).
    rng = np.random.default_rng(4)
    Lk = 7
    q = np.zeros((3, 4))
    k = rng.standard_normal((Lk, 4))
    v = rng.standard_normal((Lk, 2))
    vis = masks.visible("causal", 3, Lk)
    o, lse = attention.three_pass(q, k, v, vis, 1.0)
    for i in range(3):
        n = int(vis[i].sum())
        assert np.abs(o[i] - v[:n].mean(axis=0)).max() < 1e-15
        assert abs(lse[i] - math.log(n)) < 1e-15


def test_lse_matches_library_logsumexp():
    rng = np.random.default_rng(8)
    lay = synth.random_layout(rng, "shared_prefix", n_seqs=1, max_len=30, D=6)
    vis = masks.visible_for_layout(lay, 0)
    L = vis.shape[0]
    q, k, v = rng.standard_normal((L, 6)), rng.standard_normal((L, 6)), rng.standard_normal((L, 6))
    _, lse = attention.three_pass(q, k, v, vis, 0.3)
    s = np.where(vis, q @ k.T * 0.3, -np.inf)
    assert np.abs(lse - logsumexp(s, axis=1)).max() < 1e-13


def test_fully_hidden_row_reading():
    q, k, v = np.ones((2, 2)), np.ones((3, 2)), np.ones((3, 2))
    vis = np.array([[True, False, False], [False, False, False]])
    o, lse = attention.three_pass(q, k, v, vis, 1.0)
    assert np.array_equal(o[1], [0.0, 0.0]) and np.isneginf(lse[1])
    o2, lse2 = attention.online_tiled(q, k, v, vis, 1.0, 1, 1)
    assert np.array_equal(o2[1], [0.0, 0.0]) and np.isneginf(lse2[1])


@pytest.mark.parametrize("kind", synth.KINDS)
def test_online_tiled_independent_of_block_size(kind):
    # The tiled online softmax (Ch. 21, section 21.1's recurrence) equals the
    # three-pass result for every block size, with empty tiles skipped.
    rng = np.random.default_rng(13)
    lay = synth.random_layout(rng, kind, n_seqs=1, max_len=48, min_len=20, D=6)
    vis = masks.visible_for_layout(lay, 0)
    L = vis.shape[0]
    q, k, v = (rng.standard_normal((L, 6)) * 2 for _ in range(3))
    o3, l3 = attention.three_pass(q, k, v, vis, 0.4)
    for BM in (1, 2, 3, 4, 8, 13, 16, 64):
        for BN in (1, 2, 3, 4, 8, 13, 16, 64):
            o, l = attention.online_tiled(q, k, v, vis, 0.4, BM, BN)
            assert np.abs(o - o3).max() < 1e-12, (BM, BN)
            assert np.abs(l - l3).max() < 1e-12, (BM, BN)


def test_online_tiled_page_example_shapes():
    # Ch. 21, Worked Example 21.1.1's non-block-aligned shapes at BLOCK 4.
    torch.manual_seed(0)
    q, k, v = torch.randn(17, 8), torch.randn(23, 8), torch.randn(23, 8)
    vis = masks.visible("full", 17, 23)
    o3, _ = attention.three_pass(q, k, v, vis, 1 / math.sqrt(8))
    o, _ = attention.online_tiled(q, k, v, vis, 1 / math.sqrt(8), 4, 4)
    assert np.abs(o - o3).max() < 1e-13


def test_shared_prefix_suffix_equals_prefix_plus_suffix_alone():
    # Each suffix's output equals causal attention over [prefix, that suffix]
    # run as its own sequence.
    P, n, S, D = 9, 3, 6, 5
    lay = synth.shared_prefix(prefix=P, n_suffix=n, suffix=S, H=1, D=D)
    rng = np.random.default_rng(17)
    T = lay.total_q
    q, k, v = (rng.standard_normal((T, D)) for _ in range(3))
    o, lse = attention.three_pass(q, k, v, masks.visible_for_layout(lay, 0), 0.45)
    pre = np.arange(P)
    for i in range(1, n + 1):
        suf = P + (i - 1) * S + np.arange(S)
        idx = np.concatenate([pre, suf])
        o_alone, l_alone = attention.three_pass(q[idx], k[idx], v[idx],
                                                masks.visible("causal", P + S, P + S), 0.45)
        assert np.abs(o[suf] - o_alone[P:]).max() < 1e-13
        assert np.abs(lse[suf] - l_alone[P:]).max() < 1e-13
    # The prefix itself is plain causal attention.
    o_p, _ = attention.three_pass(q[:P], k[:P], v[:P], masks.visible("causal", P, P), 0.45)
    assert np.abs(o[:P] - o_p).max() < 1e-13


def test_strip_thinking_last_turn_equals_deleted_think_spans():
    # The last turn's output equals causal attention over the conversation
    # with the think spans of every earlier turn deleted.
    lay = synth.strip_thinking(n_turns=4, user=3, think=5, answer=4, H=1, D=6)
    rng = np.random.default_rng(19)
    T = lay.total_q
    q, k, v = (rng.standard_normal((T, 6)) for _ in range(3))
    o, lse = attention.three_pass(q, k, v, masks.visible_for_layout(lay, 0), 0.41)
    role, turn = lay.role_k, lay.turn_k
    last = turn.max()
    keep = np.nonzero(~((role == synth.THINK_ROLE) & (turn < last)))[0]
    L = len(keep)
    o_del, l_del = attention.three_pass(q[keep], k[keep], v[keep], masks.visible("causal", L, L),
                                        0.41)
    rows_last = np.nonzero(turn == last)[0]
    pos_in_keep = np.searchsorted(keep, rows_last)
    assert np.abs(o[rows_last] - o_del[pos_in_keep]).max() < 1e-13
    assert np.abs(lse[rows_last] - l_del[pos_in_keep]).max() < 1e-13


def test_packed_documents_equal_documents_alone():
    lay = synth.packed_documents(seed=3, n_docs=3, lo=4, hi=20, H=2, D=8, dtype="f32")
    q, k, v = synth.make_dense_qkv(lay, seed=3)
    O, lse = oforward.forward(lay, q, k, v)
    cu = lay.cu_q
    for s in range(lay.n_seqs):
        L = lay.seqlens_q[s]
        for h in range(2):
            o1, l1 = attention.three_pass(q[cu[s]:cu[s + 1], h], k[cu[s]:cu[s + 1], h],
                                          v[cu[s]:cu[s + 1], h], masks.visible("causal", L, L),
                                          1 / math.sqrt(8))
            assert np.array_equal(O[cu[s]:cu[s + 1], h], o1)
            assert np.array_equal(lse[h, cu[s]:cu[s + 1]], l1)


def test_forward_uses_exact_bf16_inputs():
    # bf16 inputs are widened exactly: the oracle sees the rounded values.
    lay = synth.causal_single(L=8, H=1, D=4, dtype="bf16")
    q, k, v = synth.make_dense_qkv(lay, seed=0)
    O, _ = oforward.forward(lay, q, k, v)
    o, _ = attention.three_pass(q[:, 0].float().numpy(), k[:, 0].float().numpy(),
                                v[:, 0].float().numpy(), masks.visible("causal", 8, 8), 0.5)
    assert np.array_equal(O[:, 0], o)


def test_tiles_skip_changes_nothing():
    # Skipping empty tiles is a speed-up, not a change of result: the online
    # variant with and without the skip agree exactly.
    rng = np.random.default_rng(23)
    lay = synth.random_layout(rng, "strip_thinking", n_seqs=1, max_len=40, min_len=30, D=4)
    vis = masks.visible_for_layout(lay, 0)
    L = vis.shape[0]
    q, k, v = (rng.standard_normal((L, 4)) for _ in range(3))
    a, la = attention.online_tiled(q, k, v, vis, 0.5, 4, 4, skip_empty=True)
    b, lb = attention.online_tiled(q, k, v, vis, 0.5, 4, 4, skip_empty=False)
    assert np.abs(a - b).max() < 1e-13 and np.abs(la - lb).max() < 1e-13
    cls = tiles.classify(vis, 4, 4)
    assert (cls == tiles.EMPTY).any()
