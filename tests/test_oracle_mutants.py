"""Planted mistakes in the oracle must fail at least one pin (CPU).

Each mutant replaces one oracle function with a plausibly wrong version (a
strict comparison, a dropped scale, a wrong index, a missing rescale ...)
and runs pins from the other test modules, which must raise.
"""

import numpy as np
import pytest

import test_oracle_attention as ta
import test_oracle_masks as tm
import test_oracle_paged as tp
import test_oracle_tiles as tt
from oracle import attention, masks, paged, tiles


def _fails(*pins):
    failed = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    return failed


def test_mutant_strict_causal(monkeypatch):
    orig = masks.visible

    def strict(kind, Lq, Lk, **kw):
        vis = orig(kind, Lq, Lk, **kw)
        if kind != "full":
            qi = masks.query_positions(Lq, Lk)[:, None]
            vis = vis & (np.arange(Lk)[None, :] != qi)
        return vis

    monkeypatch.setattr(masks, "visible", strict)
    assert _fails(tm.test_causal_mask_matches_printed_4x4, tm.test_causal_equals_lower_triangle_library,
                  tt.test_tile_classes_match_printed_diagram) >= 1


def test_mutant_shared_prefix_wrong_side(monkeypatch):
    orig = masks.visible

    def wrong(kind, Lq, Lk, **kw):
        if kind == "shared_prefix":  # tests the query's segment for 0 instead of the key's
            sq = np.asarray(kw["seg_q"])[:, None]
            sk = np.asarray(kw["seg_k"])[None, :]
            return orig("causal", Lq, Lk) & ((sq == 0) | (sk == sq))
        return orig(kind, Lq, Lk, **kw)

    monkeypatch.setattr(masks, "visible", wrong)
    assert _fails(tm.test_shared_prefix_matches_set_construction,
                  ta.test_shared_prefix_suffix_equals_prefix_plus_suffix_alone) >= 1


def test_mutant_strip_thinking_le(monkeypatch):
    orig = masks.visible

    def wrong(kind, Lq, Lk, **kw):
        if kind == "strip_thinking":  # hides the query's own-turn thinking too
            tq = np.asarray(kw["turn_q"])[:, None]
            tk = np.asarray(kw["turn_k"])[None, :]
            rk = np.asarray(kw["role_k"])[None, :]
            return orig("causal", Lq, Lk) & ~((rk == 1) & (tk <= tq))
        return orig(kind, Lq, Lk, **kw)

    monkeypatch.setattr(masks, "visible", wrong)
    assert _fails(tm.test_strip_thinking_matches_span_construction,
                  ta.test_strip_thinking_last_turn_equals_deleted_think_spans) >= 1


def test_mutant_dropped_scale(monkeypatch):
    orig = attention.three_pass
    monkeypatch.setattr(attention, "three_pass",
                        lambda q, k, v, vis, scale, **kw: orig(q, k, v, vis, 1.0, **kw))
    assert _fails(ta.test_noncausal_vs_causal_printed_difference,
                  ta.test_noncausal_matches_library_softmax) >= 1


def test_mutant_transposed_value_weighting(monkeypatch):
    orig = attention.three_pass

    def wrong(q, k, v, vis, scale, **kw):  # weights the keys instead of the values
        return orig(q, k, k[:, :np.asarray(v).shape[1]] if hasattr(k, "shape") else k, vis, scale)

    monkeypatch.setattr(attention, "three_pass", wrong)
    assert _fails(ta.test_noncausal_matches_library_softmax, ta.test_single_visible_key_closed_form) >= 1


def test_mutant_online_without_acc_rescale(monkeypatch):
    def wrong(q, k, v, vis, scale, BM, BN, skip_empty=True):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        Lq, Lk = vis.shape
        O = np.zeros((Lq, v.shape[1]))
        lse = np.full(Lq, -np.inf)
        for r0 in range(0, Lq, BM):
            r1 = min(Lq, r0 + BM)
            m = np.full(r1 - r0, -np.inf)
            l = np.zeros(r1 - r0)
            acc = np.zeros((r1 - r0, v.shape[1]))
            for c0 in range(0, Lk, BN):
                c1 = min(Lk, c0 + BN)
                s = np.where(vis[r0:r1, c0:c1], q[r0:r1] @ k[c0:c1].T * scale, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                mu = np.where(np.isneginf(m_new), 0, m_new)
                alpha = np.exp(m - mu)
                p = np.exp(s - mu[:, None])
                l = alpha * l + p.sum(1)
                acc = acc + p @ v[c0:c1]  # the rescale of acc is missing
                m = m_new
            O[r0:r1] = acc / np.where(l > 0, l, 1)[:, None]
            lse[r0:r1] = m + np.log(np.where(l > 0, l, 1))
        return O, lse

    monkeypatch.setattr(attention, "online_tiled", wrong)
    with pytest.raises(AssertionError):
        ta.test_online_tiled_independent_of_block_size("causal")


def test_mutant_edge_tiles_full(monkeypatch):
    def wrong(vis, BM, BN, n_qt=None, n_kt=None):  # forgets that padding is not visible
        Lq, Lk = vis.shape
        n_qt = tiles.cdiv(Lq, BM) if n_qt is None else n_qt
        n_kt = tiles.cdiv(Lk, BN) if n_kt is None else n_kt
        cls = np.zeros((n_qt, n_kt), np.uint8)
        for a in range(n_qt):
            for b in range(n_kt):
                blk = vis[a * BM:(a + 1) * BM, b * BN:(b + 1) * BN]
                if blk.size == 0 or not blk.any():
                    cls[a, b] = tiles.EMPTY
                elif blk.all():
                    cls[a, b] = tiles.FULL
                else:
                    cls[a, b] = tiles.PARTIAL
        return cls

    monkeypatch.setattr(tiles, "classify", wrong)
    assert _fails(tt.test_causal_classes_match_closed_form, tt.test_edge_tiles_never_full) >= 1


def test_mutant_gather_page_slot_swapped(monkeypatch):
    def wrong(pool, bt, ctx, page_size, tile=None):
        pool = np.asarray(pool)
        flat = pool.reshape((-1,) + pool.shape[2:])
        j = np.arange(ctx)
        bt = np.asarray(bt, np.int64)
        rows = bt[j % len(bt)] * page_size + j // page_size  # page and slot swapped
        rows = np.clip(rows, 0, flat.shape[0] - 1)
        return flat[rows]

    monkeypatch.setattr(paged, "paged_gather", wrong)
    assert _fails(tp.test_gather_byte_equal_for_every_tile_size) >= 1


def test_mutant_gather_reads_past_context(monkeypatch):
    orig = paged.paged_gather

    def wrong(pool, bt, ctx, page_size, tile=None):  # gathers whole pages
        n = -(-ctx // page_size)
        return orig(pool, bt, n * page_size, page_size, tile)

    monkeypatch.setattr(paged, "paged_gather", wrong)
    import oracle.forward as of
    monkeypatch.setattr(of, "paged_gather", wrong)
    assert _fails(tp.test_ragged_rows_through_pages, tp.test_gather_byte_equal_for_every_tile_size) >= 1


def _dup_mutant(monkeypatch, fn):
    monkeypatch.setattr(masks, "_duplicated_answer_context", fn)
    return _fails(tm.test_duplicated_answers_match_hand_worked_12x12,
                  tm.test_duplicated_answers_reproduce_inference_contexts)


def _dup_parts(role_q, role_k, turn_q, turn_k, think, loss, history):
    rq = np.asarray(role_q)[:, None]
    tq = np.asarray(turn_q)[:, None]
    rk = np.asarray(role_k)[None, :]
    tk = np.asarray(turn_k)[None, :]
    return rq, tq, rk, tk


def test_mutant_history_copy_sees_own_thinking(monkeypatch):
    def wrong(role_q, role_k, turn_q, turn_k, think, loss, history):
        rq, tq, rk, tk = _dup_parts(role_q, role_k, turn_q, turn_k, think, loss, history)
        away = (rk == think) | (rk == loss)
        return ((tk < tq) & ~away) | ((tk == tq) & (rq == history) & (rk != loss)) | \
               ((tk == tq) & (rq != history) & (rk != history))
    assert _dup_mutant(monkeypatch, wrong) >= 1


def test_mutant_later_turns_see_loss_copy(monkeypatch):
    def wrong(role_q, role_k, turn_q, turn_k, think, loss, history):
        rq, tq, rk, tk = _dup_parts(role_q, role_k, turn_q, turn_k, think, loss, history)
        away = (rk == think) | (rk == history)  # the copies swapped for history
        return ((tk < tq) & ~away) | ((tk == tq) & (rq == history) & (rk != think) & (rk != loss)) | \
               ((tk == tq) & (rq != history) & (rk != history))
    assert _dup_mutant(monkeypatch, wrong) >= 1


def test_mutant_history_copy_misses_own_user_text(monkeypatch):
    def wrong(role_q, role_k, turn_q, turn_k, think, loss, history):
        rq, tq, rk, tk = _dup_parts(role_q, role_k, turn_q, turn_k, think, loss, history)
        away = (rk == think) | (rk == loss)
        return ((tk < tq) & ~away) | ((tk == tq) & (rq == history) & (rk == history)) | \
               ((tk == tq) & (rq != history) & (rk != history))
    assert _dup_mutant(monkeypatch, wrong) >= 1


def test_mutant_loss_copy_misses_own_thinking(monkeypatch):
    def wrong(role_q, role_k, turn_q, turn_k, think, loss, history):
        rq, tq, rk, tk = _dup_parts(role_q, role_k, turn_q, turn_k, think, loss, history)
        away = (rk == think) | (rk == loss)
        return ((tk < tq) & ~away) | ((tk == tq) & (rq == history) & ~away) | \
               ((tk == tq) & (rq != history) & (rk != history) & ~((rq == loss) & (rk == think)))
    assert _dup_mutant(monkeypatch, wrong) >= 1


import test_oracle_backward as tb
from oracle import backward as obackward


def _bwd_mutant(monkeypatch, fn):
    monkeypatch.setattr(obackward, "sequence_backward", fn)
    return _fails(tb.test_backward_matches_central_differences,
                  tb.test_backward_matches_torch_autograd_float64)


def test_mutant_backward_without_softmax_correction(monkeypatch):
    def wrong(q, k, v, vis, scale, do):  # dS = P * dP, the row term dropped
        p = obackward.probabilities(q, k, vis, scale)
        ds = p * (do @ np.asarray(v).T)
        return scale * ds @ k, scale * ds.T @ q, p.T @ do
    assert _bwd_mutant(monkeypatch, wrong) >= 1


def test_mutant_backward_missing_scale_on_dk(monkeypatch):
    def wrong(q, k, v, vis, scale, do):
        p = obackward.probabilities(q, k, vis, scale)
        dp = do @ np.asarray(v).T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        return scale * ds @ k, ds.T @ q, p.T @ do
    assert _bwd_mutant(monkeypatch, wrong) >= 1


def test_mutant_backward_unnormalised_probabilities(monkeypatch):
    def wrong(q, k, v, vis, scale, do):  # exp(S) without dividing by the row sum
        s = np.where(vis, (np.asarray(q) @ np.asarray(k).T) * scale, -np.inf)
        p = np.exp(s - np.where(vis.any(1), s.max(1, initial=-np.inf), 0)[:, None])
        dp = do @ np.asarray(v).T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        return scale * ds @ k, scale * ds.T @ q, p.T @ do
    assert _bwd_mutant(monkeypatch, wrong) >= 1


def test_mutant_tile_columns_off_by_one(monkeypatch):
    orig = tiles.layout_tile_columns

    def wrong(layout, BM, BN):
        fc, pc, fi, pi = orig(layout, BM, BN)
        fi = np.where(fi >= 0, fi + 1, fi)  # query-tile index shifted
        return fc, pc, fi, pi

    monkeypatch.setattr(tiles, "layout_tile_columns", wrong)
    assert _fails(tb.test_tile_columns_transpose_the_printed_diagram,
                  lambda: tb.test_tile_columns_reexpand_to_the_classes("causal")) >= 1


def test_mutant_composed_padding_visible(monkeypatch):
    orig = masks._composed

    def wrong(Lq, Lk, terms, causal, **kw):  # negative document ids not treated as padding
        kw = dict(kw)
        if kw.get("doc_q") is not None:
            kw["doc_q"] = np.abs(np.asarray(kw["doc_q"])) + 7
            kw["doc_k"] = np.abs(np.asarray(kw["doc_k"])) + 7
        return orig(Lq, Lk, terms, causal, **kw)

    monkeypatch.setattr(masks, "_composed", wrong)
    assert _fails(tm.test_composed_document_strip_thinking_hand_worked,
                  tm.test_shared_prefix_groups_hand_worked,
                  tm.test_composed_document_term_equals_separate_sequences) >= 1


def test_mutant_composed_or_instead_of_and(monkeypatch):
    orig = masks._composed

    def wrong(Lq, Lk, terms, causal, **kw):  # terms ORed after the causal one
        rest = [t for t in terms if t != "causal"]
        vis = np.zeros((Lq, Lk), bool)
        for t in rest:
            vis |= orig(Lq, Lk, (t,), causal, **kw)
        if not rest:
            vis[:] = True
        return vis & (causal if "causal" in terms else True)

    monkeypatch.setattr(masks, "_composed", wrong)
    assert _fails(tm.test_composed_document_strip_thinking_hand_worked,
                  tm.test_shared_prefix_groups_hand_worked) >= 1


def test_mutant_composed_groups_anded(monkeypatch):
    def wrong(Lq, Lk, terms, causal, **kw):  # groups combined by AND instead of OR
        vis = np.ones((Lq, Lk), bool)
        for group in masks.term_groups(terms):
            vis &= masks._and_group(Lq, Lk, group, causal, **kw)
        return vis

    monkeypatch.setattr(masks, "_composed", wrong)
    assert _fails(tm.test_composed_or_prefix_lm_hand_worked, tm.test_composed_or_groups_hand_worked,
                  tm.test_composed_or_prefix_lm_closed_form) == 3


def test_mutant_composed_or_and_swapped(monkeypatch):
    def wrong(Lq, Lk, terms, causal, **kw):  # OR inside each group, AND across groups
        vis = np.ones((Lq, Lk), bool)
        for group in masks.term_groups(terms):
            any_term = np.zeros((Lq, Lk), bool)
            for t in group:
                any_term |= masks._and_group(Lq, Lk, (t,), causal, **kw)
            vis &= any_term
        return vis

    monkeypatch.setattr(masks, "_composed", wrong)
    assert _fails(tm.test_composed_or_prefix_lm_hand_worked, tm.test_composed_or_groups_hand_worked,
                  tm.test_composed_or_prefix_lm_closed_form) >= 2
