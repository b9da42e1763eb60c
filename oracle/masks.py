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
* strip_thinking_duplicated -- the same issue, section "The exactness
  question", option (b): every answer span appears twice, a loss copy that
  sees its own turn's thinking and a history copy that sees the context
  inference has once the thinking is stripped; later turns see the history
  copy only.
* full -- no mask: Ch. 21, section 21.1's kernel before causal masking.
* composed -- the xorl issue, section "Proposed work", item 3 (composable
  builders: causal, document, shared-prefix and strip-thinking pieces) and
  section "Current state in this tree" (causal + document + padding in one
  mask): the AND of the chosen terms.  The document term keeps pairs of one
  document; a negative document id marks padding, which no query sees.
  Reading: the pieces compose by AND inside a group and by OR across groups
  (an OR of ANDs), so that e.g. a prefix-LM mask is "causal" OR "both in the
  prefix document".  ``terms`` is either one group (a tuple of term names)
  or a tuple of such groups.
"""

from __future__ import annotations

import numpy as np


def query_positions(Lq: int, Lk: int) -> np.ndarray:
    """Absolute position of each query row inside its sequence of Lk keys."""
    return np.arange(Lq, dtype=np.int64) + (Lk - Lq)


TERMS = ("causal", "document", "shared_prefix", "strip_thinking")


def visible(kind: str, Lq: int, Lk: int, *, seg_q=None, seg_k=None, role_q=None, role_k=None,
            turn_q=None, turn_k=None, think_role: int = 1, loss_role: int = 2,
            history_role: int = 3, doc_q=None, doc_k=None, terms=()) -> np.ndarray:
    """Dense boolean mask ``[Lq, Lk]`` for one sequence.

    ``seg_q``/``role_q``/``turn_q`` are per query row, ``seg_k``/``role_k``/
    ``turn_k`` per key; each kind reads only the ids it needs.
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
    if kind == "composed":
        return _composed(Lq, Lk, terms, causal, seg_q=seg_q, seg_k=seg_k, role_k=role_k,
                         turn_q=turn_q, turn_k=turn_k, doc_q=doc_q, doc_k=doc_k,
                         think_role=think_role)
    if kind == "strip_thinking_duplicated":
        return causal & _duplicated_answer_context(role_q, role_k, turn_q, turn_k,
                                                   think_role, loss_role, history_role)
    raise ValueError(f"unknown mask kind {kind!r}")


def term_groups(terms) -> tuple:
    """The AND-groups of a composed mask: one group (a tuple of term names)
    becomes a 1-tuple of groups; a tuple of groups is kept.  Every group is
    non-empty and names only TERMS."""
    terms = tuple(terms)
    if not terms:
        raise ValueError("a composed mask needs at least one term")
    groups = (terms,) if all(isinstance(t, str) for t in terms) else tuple(tuple(g) for g in terms)
    for g in groups:
        if not g or not all(isinstance(t, str) for t in g):
            raise ValueError(f"malformed term group {g!r}")
    return groups


def _composed(Lq, Lk, terms, causal, **ids):
    """OR over the AND-groups of ``terms`` (see term_groups)."""
    vis = np.zeros((Lq, Lk), dtype=bool)
    for group in term_groups(terms):
        vis |= _and_group(Lq, Lk, group, causal, **ids)
    return vis


def _and_group(Lq, Lk, terms, causal, *, seg_q, seg_k, role_k, turn_q, turn_k, doc_q, doc_k,
               think_role):
    """AND of the chosen terms (any subset of TERMS, in any order)."""
    unknown = set(terms) - set(TERMS)
    if unknown:
        raise ValueError(f"unknown mask terms {sorted(unknown)}")
    vis = np.ones((Lq, Lk), dtype=bool)
    if "causal" in terms:
        vis &= causal
    if "document" in terms:
        dq = np.asarray(doc_q, dtype=np.int64)[:, None]
        dk = np.asarray(doc_k, dtype=np.int64)[None, :]
        vis &= (dk == dq) & (dk >= 0)
    if "shared_prefix" in terms:
        sq = np.asarray(seg_q, dtype=np.int64)[:, None]
        sk = np.asarray(seg_k, dtype=np.int64)[None, :]
        vis &= (sk == 0) | (sk == sq)
    if "strip_thinking" in terms:
        tq = np.asarray(turn_q, dtype=np.int64)[:, None]
        tk = np.asarray(turn_k, dtype=np.int64)[None, :]
        rk = np.asarray(role_k, dtype=np.int64)[None, :]
        vis &= ~((rk == think_role) & (tk < tq))
    return vis


def _duplicated_answer_context(role_q, role_k, turn_q, turn_k, think_role, loss_role,
                               history_role) -> np.ndarray:
    """Which keys lie in each query's context when answers are duplicated
    (causality aside).

    xorl issue, "The exactness question", option (b).  A finished turn
    enters later turns the way inference replays it: its thinking is gone
    and its answer is the history copy, so a key of an earlier turn is in
    the context unless it is thinking or a loss copy.  Inside the query's
    own turn the two answer copies see different things: the history copy
    sees the turn stripped of its thinking (and of the loss copy, which
    inference never holds beside it); every other token of the turn (user
    text, thinking, the loss copy) sees the turn as generated, i.e. without
    the history copy.  Keys of later turns are never in the context.
    """
    rq = np.asarray(role_q, dtype=np.int64)[:, None]
    tq = np.asarray(turn_q, dtype=np.int64)[:, None]
    rk = np.asarray(role_k, dtype=np.int64)[None, :]
    tk = np.asarray(turn_k, dtype=np.int64)[None, :]
    stripped_away = (rk == think_role) | (rk == loss_role)
    query_is_history = rq == history_role
    earlier = tk < tq
    same_turn = tk == tq
    from_history = earlier & ~stripped_away
    own_turn_replayed = same_turn & query_is_history & ~stripped_away
    own_turn_generated = same_turn & ~query_is_history & (rk != history_role)
    return from_history | own_turn_replayed | own_turn_generated


def visible_for_layout(layout, s: int) -> np.ndarray:
    """Dense mask of sequence ``s`` of a ``synth.Layout``."""
    ids = layout.ids_for_seq(s)
    return visible(layout.kind, layout.seqlens_q[s], layout.seqlens_k[s],
                   seg_q=ids.get("seg_q"), seg_k=ids.get("seg_k"), role_q=ids.get("role_q"),
                   role_k=ids.get("role_k"), turn_q=ids.get("turn_q"), turn_k=ids.get("turn_k"),
                   think_role=layout.think_role, loss_role=layout.loss_role,
                   history_role=layout.history_role, doc_q=ids.get("doc_q"),
                   doc_k=ids.get("doc_k"), terms=layout.terms)
