"""Pins of oracle.masks against the pages and independent constructions (CPU)."""

import numpy as np
import pytest

import _golden
import synth
from oracle import masks


def test_causal_mask_matches_printed_4x4():
    # Ch. 9, Worked Example 9.1.1: the causal mask applied to 1..16.
    g = _golden.load("causal_mask_4x4.txt")
    vis = masks.visible("causal", 4, 4)
    assert np.array_equal(np.where(vis, g["input"], 0.0), g["causal"])
    # Worked Example 9.1.2: the strict comparison is the printed bug; the
    # oracle's mask must not reproduce it.
    assert not np.array_equal(np.where(vis, g["input"], 0.0), g["strict"])
    strict = np.arange(4)[None, :] < np.arange(4)[:, None]
    assert np.array_equal(np.where(strict, g["input"], 0.0), g["strict"])


def test_causal_equals_lower_triangle_library():
    for L in (1, 2, 7, 33):
        assert np.array_equal(masks.visible("causal", L, L), np.tril(np.ones((L, L), bool)))


def test_decode_query_sees_whole_context():
    # One query at the end of its context sees every key (the decode reading).
    for Lk in (1, 5, 17):
        vis = masks.visible("causal", 1, Lk)
        assert vis.shape == (1, Lk) and vis.all()
    # Several trailing queries: the bottom-right part of the full triangle.
    Lq, Lk = 3, 9
    assert np.array_equal(masks.visible("causal", Lq, Lk),
                          np.tril(np.ones((Lk, Lk), bool))[Lk - Lq:])


def _shared_prefix_by_sets(seg):
    """Visible sets built from the segment layout, not from the predicate:
    prefix tokens see the prefix up to themselves; a token of suffix i sees the
    whole prefix part that precedes it plus its own suffix up to itself."""
    T = len(seg)
    vis = np.zeros((T, T), bool)
    for qpos in range(T):
        if seg[qpos] == 0:
            allowed = [j for j in range(qpos + 1) if seg[j] == 0]
        else:
            allowed = [j for j in range(qpos + 1) if seg[j] == 0] + \
                      [j for j in range(qpos + 1) if seg[j] == seg[qpos]]
        vis[qpos, sorted(set(allowed))] = True
    return vis


def test_shared_prefix_matches_set_construction():
    lay = synth.shared_prefix(prefix=5, n_suffix=3, suffix=4, H=1, D=8)
    seg = lay.seg_k
    vis = masks.visible("shared_prefix", len(seg), len(seg), seg_q=seg, seg_k=seg)
    assert np.array_equal(vis, _shared_prefix_by_sets(seg))
    # Suffix 2 never sees suffix 1.
    s1 = np.nonzero(seg == 1)[0]
    s2 = np.nonzero(seg == 2)[0]
    assert not vis[np.ix_(s2, s1)].any()


def test_shared_prefix_reductions():
    rng = np.random.default_rng(3)
    for L in (1, 6, 20):
        zero = np.zeros(L, np.int32)
        assert np.array_equal(masks.visible("shared_prefix", L, L, seg_q=zero, seg_k=zero),
                              masks.visible("causal", L, L))
        ids = rng.integers(0, 4, size=L).astype(np.int32)
        sp = masks.visible("shared_prefix", L, L, seg_q=ids, seg_k=ids)
        assert not (sp & ~masks.visible("causal", L, L)).any()
        assert np.array_equal(np.diag(sp), np.ones(L, bool))  # diagonal always kept


def test_shared_prefix_position_reading_equivalent():
    # The causal test on the packed index equals the one on position_ids that
    # restart at len(P) for every suffix (the page's position convention).
    P, n, S = 6, 3, 5
    lay = synth.shared_prefix(prefix=P, n_suffix=n, suffix=S, H=1, D=8)
    seg = lay.seg_k
    pos = np.concatenate([np.arange(P)] + [P + np.arange(S) for _ in range(n)])
    T = len(seg)
    by_pos = np.zeros((T, T), bool)
    for i in range(T):
        for j in range(T):
            by_pos[i, j] = (pos[i] >= pos[j]) and (seg[j] == 0 or seg[j] == seg[i])
    assert np.array_equal(masks.visible("shared_prefix", T, T, seg_q=seg, seg_k=seg), by_pos)


def _strip_thinking_by_spans(role, turn, think):
    """A query at position p of turn t sees positions <= p minus the think
    spans of every earlier turn (built from span lists)."""
    T = len(role)
    spans = {}
    for j in range(T):
        if role[j] == think:
            spans.setdefault(int(turn[j]), []).append(j)
    vis = np.zeros((T, T), bool)
    for p in range(T):
        hidden = set()
        for t, js in spans.items():
            if t < turn[p]:
                hidden.update(js)
        for j in range(p + 1):
            if j not in hidden:
                vis[p, j] = True
    return vis


def test_strip_thinking_matches_span_construction():
    lay = synth.strip_thinking(n_turns=3, user=2, think=3, answer=2, H=1, D=8)
    role, turn = lay.role_k, lay.turn_k
    T = len(role)
    vis = masks.visible("strip_thinking", T, T, role_k=role, turn_q=turn, turn_k=turn,
                        think_role=synth.THINK_ROLE)
    assert np.array_equal(vis, _strip_thinking_by_spans(role, turn, synth.THINK_ROLE))
    # The query's own-turn thinking stays visible: answer of turn 1 sees think of turn 1.
    a1 = np.nonzero((role == 2) & (turn == 1))[0]
    k1 = np.nonzero((role == synth.THINK_ROLE) & (turn == 1))[0]
    assert vis[np.ix_(a1, k1)].all()
    k0 = np.nonzero((role == synth.THINK_ROLE) & (turn == 0))[0]
    assert not vis[np.ix_(a1, k0)].any()


def test_strip_thinking_random_layouts_match_spans():
    rng = np.random.default_rng(11)
    for _ in range(5):
        lay = synth.random_layout(rng, "strip_thinking", n_seqs=1, max_len=30)
        T = lay.seqlens_k[0]
        vis = masks.visible("strip_thinking", T, T, role_k=lay.role_k, turn_q=lay.turn_q,
                            turn_k=lay.turn_k)
        assert np.array_equal(vis, _strip_thinking_by_spans(lay.role_k, lay.turn_k, 1))


def test_strip_thinking_without_think_is_causal():
    L = 12
    role = np.array([0, 2] * 6, np.int32)
    turn = np.repeat(np.arange(6), 2).astype(np.int32)
    assert np.array_equal(masks.visible("strip_thinking", L, L, role_k=role, turn_q=turn,
                                        turn_k=turn),
                          masks.visible("causal", L, L))


def test_packed_documents_block_diagonal():
    # Each document is its own sequence: concatenating the per-sequence masks
    # on the packed axis gives the block-diagonal causal mask of the batch.
    lens = [3, 1, 4]
    T = sum(lens)
    big = np.zeros((T, T), bool)
    o = 0
    for L in lens:
        big[o:o + L, o:o + L] = masks.visible("causal", L, L)
        o += L
    doc = np.repeat(np.arange(len(lens)), lens)
    expect = (np.arange(T)[None, :] <= np.arange(T)[:, None]) & (doc[:, None] == doc[None, :])
    assert np.array_equal(big, expect)


def test_full_mask():
    assert masks.visible("full", 3, 5).all()
    with pytest.raises(ValueError):
        masks.visible("bogus", 2, 2)


def _dup_visible(role, turn):
    T = len(role)
    return masks.visible("strip_thinking_duplicated", T, T, role_q=role, role_k=role, turn_q=turn,
                         turn_k=turn, think_role=synth.THINK_ROLE, loss_role=synth.LOSS_ROLE,
                         history_role=synth.HISTORY_ROLE)


def test_duplicated_answers_match_hand_worked_12x12():
    # xorl issue, "The exactness question", option (b), worked by hand.
    g = _golden.load("strip_thinking_duplicated_12x12.txt")
    role, turn = g["role"].astype(np.int32), g["turn"].astype(np.int32)
    assert np.array_equal(_dup_visible(role, turn), g["visible"].astype(bool))
    lay = synth.strip_thinking_duplicated(n_turns=2, user=1, think=1, answer=2, H=1, D=8)
    assert np.array_equal(lay.role_k, role) and np.array_equal(lay.turn_k, turn)
    assert np.array_equal(masks.visible_for_layout(lay, 0), g["visible"].astype(bool))


def test_duplicated_answers_without_answers_is_strip_thinking():
    # With no answer tokens there is nothing to duplicate: option (b) is the
    # plain strip-thinking mask of the same sequence.
    rng = np.random.default_rng(3)
    for _ in range(4):
        n = int(rng.integers(1, 30))
        role = rng.choice([synth.USER_ROLE, synth.THINK_ROLE], size=n).astype(np.int32)
        turn = np.sort(rng.integers(0, 4, size=n)).astype(np.int32)
        plain = masks.visible("strip_thinking", n, n, role_k=role, turn_q=turn, turn_k=turn,
                              think_role=synth.THINK_ROLE)
        assert np.array_equal(_dup_visible(role, turn), plain)


def _conversation(rng, n_turns, cap):
    """Span lengths (user, think, answer) of each turn, answers non-empty."""
    return [(int(rng.integers(1, cap)), int(rng.integers(0, cap)), int(rng.integers(1, cap)))
            for _ in range(n_turns)]


def _toy_network(x, vis, weights):
    """Residual single-head attention layers, no positions: a token's state
    depends only on the states of the keys it sees."""
    from oracle import attention
    for wq, wk, wv in weights:
        o, _ = attention.three_pass(x @ wq, x @ wk, x @ wv, vis, 0.5)
        x = x + o
    return x


def test_duplicated_answers_reproduce_inference_contexts():
    # The point of option (b): with every answer duplicated, one packed pass
    # gives each token the hidden states it has at inference, at every
    # depth.  Inference of turn t runs plain causal attention over the
    # conversation as replayed then: earlier turns without their thinking,
    # then the current turn as generated.  The history copy of turn t must
    # equal the answer of turn t replayed the same way.  Mask only (option
    # (a), one copy per answer) matches at depth 1 and fails at depth 2.
    rng = np.random.default_rng(17)
    d, depth = 8, 2
    diverged = 0
    for trial in range(3):
        conv = _conversation(rng, n_turns=int(rng.integers(2, 5)), cap=4)
        n_tok = sum(u + th + a for u, th, a in conv)
        emb = rng.standard_normal((n_tok, d))
        weights = [tuple(rng.standard_normal((d, d)) * 0.7 for _ in range(3)) for _ in range(depth)]
        ids = []  # per turn: token ids of the user, think and answer spans
        nxt = 0
        for u, th, a in conv:
            ids.append([list(range(nxt, nxt + u)), list(range(nxt + u, nxt + u + th)),
                        list(range(nxt + u + th, nxt + u + th + a))])
            nxt += u + th + a
        # the duplicated sequence and, per position, which copy it holds
        seq, role, turn = [], [], []
        for t, (us, ths, ans) in enumerate(ids):
            for r, span in ((synth.USER_ROLE, us), (synth.THINK_ROLE, ths), (synth.LOSS_ROLE, ans),
                            (synth.HISTORY_ROLE, ans)):
                seq += span
                role += [r] * len(span)
                turn += [t] * len(span)
        role, turn = np.array(role, np.int32), np.array(turn, np.int32)
        packed = _toy_network(emb[seq], _dup_visible(role, turn), weights)

        def run_causal(tokens):
            return _toy_network(emb[tokens], masks.visible("causal", len(tokens), len(tokens)),
                                weights)

        for t, (us, ths, ans) in enumerate(ids):
            replayed = [x for s in range(t) for x in ids[s][0] + ids[s][2]]
            gen = run_causal(replayed + us + ths + ans)
            n = len(replayed)
            for r, span in ((synth.USER_ROLE, us), (synth.THINK_ROLE, ths), (synth.LOSS_ROLE, ans)):
                at = np.nonzero((role == r) & (turn == t))[0]
                where = [n + (us + ths + ans).index(x) for x in span]
                np.testing.assert_allclose(packed[at], gen[where], rtol=0, atol=1e-12)
            hist = run_causal(replayed + us + ans)
            at = np.nonzero((role == synth.HISTORY_ROLE) & (turn == t))[0]
            np.testing.assert_allclose(packed[at], hist[n + len(us):], rtol=0, atol=1e-12)

        # option (a): one copy per answer, strip-thinking mask
        seq_a = [x for us, ths, ans in ids for x in us + ths + ans]
        role_a = np.array([r for us, ths, ans in ids for r, span in
                           ((synth.USER_ROLE, us), (synth.THINK_ROLE, ths), (synth.ANSWER_ROLE, ans))
                           for _ in span], np.int32)
        turn_a = np.array([t for t, (us, ths, ans) in enumerate(ids) for _ in us + ths + ans],
                          np.int32)
        T = len(seq_a)
        vis_a = masks.visible("strip_thinking", T, T, role_k=role_a, turn_q=turn_a, turn_k=turn_a)
        last = len(ids) - 1
        us, ths, ans = ids[last]
        replayed = [x for s in range(last) for x in ids[s][0] + ids[s][2]]
        gen = run_causal(replayed + us + ths + ans)
        at = np.nonzero(turn_a == last)[0]
        one_layer = lambda toks, vis: _toy_network(emb[toks], vis, weights[:1])
        np.testing.assert_allclose(
            one_layer(seq_a, vis_a)[at],
            one_layer(replayed + us + ths + ans,
                      masks.visible("causal", len(gen), len(gen)))[len(replayed):],
            rtol=0, atol=1e-12)
        if any(th > 0 for _, th, _ in conv[:last]):
            assert np.abs(_toy_network(emb[seq_a], vis_a, weights)[at] - gen[len(replayed):]).max() > 1e-6
            diverged += 1
    assert diverged >= 1


def _composed(terms, T, **ids):
    ids = {k: np.asarray(v).astype(np.int32) for k, v in ids.items()}
    return masks.visible("composed", T, T, terms=terms, seg_q=ids.get("seg"), seg_k=ids.get("seg"),
                         role_k=ids.get("role"), turn_q=ids.get("turn"), turn_k=ids.get("turn"),
                         doc_q=ids.get("doc"), doc_k=ids.get("doc"), think_role=synth.THINK_ROLE)


def test_composed_document_strip_thinking_hand_worked():
    g = _golden.load("composed_document_strip_10x10.txt")
    vis = _composed(("causal", "document", "strip_thinking"), 10, role=g["role"], turn=g["turn"],
                    doc=g["doc"])
    assert np.array_equal(vis, g["visible"].astype(bool))
    # the order of the terms does not matter
    vis2 = _composed(("strip_thinking", "causal", "document"), 10, role=g["role"], turn=g["turn"],
                     doc=g["doc"])
    assert np.array_equal(vis2, vis)


def test_shared_prefix_groups_hand_worked():
    g = _golden.load("shared_prefix_groups_9x9.txt")
    lay = synth.shared_prefix_groups(n_groups=2, prefix=2, n_suffix=2, suffix=1, pad=1, H=1, D=8)
    assert np.array_equal(lay.seg_k, g["seg"]) and np.array_equal(lay.doc_k, g["doc"])
    assert np.array_equal(masks.visible_for_layout(lay, 0), g["visible"].astype(bool))


def test_composed_single_terms_are_the_plain_kinds():
    rng = np.random.default_rng(12)
    for _ in range(5):
        T = int(rng.integers(1, 40))
        seg = np.sort(rng.integers(0, 3, T))
        role = rng.integers(0, 3, T)
        turn = np.sort(rng.integers(0, 4, T))
        kw = dict(seg=seg, role=role, turn=turn)
        assert np.array_equal(_composed(("causal",), T, **kw), masks.visible("causal", T, T))
        assert np.array_equal(_composed(("causal", "shared_prefix"), T, **kw),
                              masks.visible("shared_prefix", T, T, seg_q=seg, seg_k=seg))
        assert np.array_equal(_composed(("causal", "strip_thinking"), T, **kw),
                              masks.visible("strip_thinking", T, T, role_k=role, turn_q=turn,
                                            turn_k=turn))
        assert np.array_equal(_composed(("document",), T, doc=np.zeros(T)),
                              masks.visible("full", T, T))


def test_composed_document_term_equals_separate_sequences():
    # Document ids inside one sequence give the block-diagonal of the
    # documents' own masks; padding rows and columns are empty.
    rng = np.random.default_rng(13)
    for terms, kind in ((("causal", "document"), "causal"),
                        (("causal", "document", "shared_prefix"), "shared_prefix"),
                        (("causal", "document", "strip_thinking"), "strip_thinking")):
        lens = rng.integers(1, 12, size=4)
        pad = rng.random(4) < 0.3
        doc = np.concatenate([np.full(n, -1 if p else d) for d, (n, p) in enumerate(zip(lens, pad))])
        T = int(lens.sum())
        seg = np.concatenate([np.sort(rng.integers(0, 3, n)) for n in lens])
        role = rng.integers(0, 3, T)
        turn = np.concatenate([np.sort(rng.integers(0, 3, n)) for n in lens])
        expect = np.zeros((T, T), bool)
        o = 0
        for n, p in zip(lens, pad):
            if not p:
                sl = slice(o, o + n)
                expect[sl, sl] = masks.visible(kind, n, n, seg_q=seg[sl], seg_k=seg[sl],
                                               role_k=role[sl], turn_q=turn[sl], turn_k=turn[sl])
            o += n
        got = _composed(terms, T, seg=seg, role=role, turn=turn, doc=doc)
        assert np.array_equal(got, expect), terms


def test_composed_or_prefix_lm_hand_worked():
    g = _golden.load("composed_prefix_lm_7x7.txt")
    vis = _composed((("causal",), ("document",)), 7, doc=g["doc"])
    assert np.array_equal(vis, g["visible"].astype(bool))


def test_composed_or_groups_hand_worked():
    g = _golden.load("composed_or_groups_8x8.txt")
    groups = (("causal", "strip_thinking"), ("document", "shared_prefix"))
    ids = dict(role=g["role"], turn=g["turn"], seg=g["seg"], doc=g["doc"])
    vis = _composed(groups, 8, **ids)
    assert np.array_equal(vis, g["visible"].astype(bool))
    # neither the order of the groups nor the order inside a group matters
    assert np.array_equal(_composed((("shared_prefix", "document"), ("strip_thinking", "causal")), 8,
                                    **ids), vis)


def test_composed_or_prefix_lm_closed_form():
    # causal OR (both inside the prefix document) is the lower triangle with
    # the prefix square filled in, for any prefix length (0 .. T).
    for T in (1, 5, 33):
        for P in sorted({0, 1, T // 2, T}):
            doc = np.where(np.arange(T) < P, 0, -1)
            expect = np.tril(np.ones((T, T), bool))
            expect[:P, :P] = True
            assert np.array_equal(_composed((("causal",), ("document",)), T, doc=doc), expect), (T, P)


def test_composed_one_group_is_the_and_and_groups_are_idempotent():
    rng = np.random.default_rng(21)
    for _ in range(6):
        T = int(rng.integers(1, 30))
        ids = dict(seg=np.sort(rng.integers(0, 3, T)), role=rng.integers(0, 3, T),
                   turn=np.sort(rng.integers(0, 4, T)), doc=np.sort(rng.integers(-1, 3, T)))
        a = tuple(t for t in masks.TERMS if rng.random() < 0.5) or ("causal",)
        b = tuple(t for t in masks.TERMS if rng.random() < 0.5) or ("document",)
        va = _composed(a, T, **ids)
        assert np.array_equal(_composed((a,), T, **ids), va)
        assert np.array_equal(_composed((a, a), T, **ids), va)
        vab = _composed((a, b), T, **ids)
        assert np.array_equal(_composed((b, a), T, **ids), vab)
        assert (vab >= va).all() and (vab >= _composed(b, T, **ids)).all()


def test_composed_rejects_malformed_groups():
    for bad in ((), ((),), (("causal",), ()), (("causal",), "document"), (("sliding",),)):
        with pytest.raises(ValueError):
            _composed(bad, 3, doc=np.zeros(3))


def test_composed_rejects_unknown_terms():
    with pytest.raises(ValueError):
        _composed(("causal", "sliding_window"), 3)
