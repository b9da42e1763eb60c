"""Workload layouts and seeded tensors.

Token layout (shared by every consumer): queries of all sequences are packed
along one token axis, ``q[total_q, H, D]``; keys and values likewise,
``k[total_k, H, D]``, with head_dim contiguous. Sequence ``s`` owns query rows
``cu_q[s] .. cu_q[s+1]-1`` and key rows ``cu_k[s] .. cu_k[s+1]-1`` (or, when
paged, logical key positions ``0 .. seqlens_k[s]-1`` reached through a block
table into a page pool ``[num_pages, page_size, H, D]``).

Per-token ids describe structure only:
  * ``seg``  -- segment id (0 = shared prefix, i >= 1 = the i-th suffix),
  * ``role`` -- 0 user, 1 think, 2 answer; with duplicated answers 2 is the
    answer's loss copy and 3 its history copy,
  * ``turn`` -- conversation turn index,
  * ``doc``  -- document index inside a packed sequence (negative: padding).

Random values are float32 standard normals drawn from a torch generator on the
requested device and rounded to the workload dtype (bf16 by round to nearest
even).  The structure (lengths, page permutation) comes from numpy's
``default_rng`` and does not depend on the device.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

USER_ROLE = 0
THINK_ROLE = 1
ANSWER_ROLE = LOSS_ROLE = 2
HISTORY_ROLE = 3
KINDS = ("full", "causal", "shared_prefix", "strip_thinking", "strip_thinking_duplicated", "composed")
TERMS = ("causal", "document", "shared_prefix", "strip_thinking")


def derive_seed(seed: int, *tags: int) -> int:
    """A 63-bit seed for one tensor, derived from the workload seed and tags."""
    ss = np.random.SeedSequence([int(seed)] + [int(t) for t in tags])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


@dataclass
class Layout:
    """Structure of one workload (no tensor values)."""

    name: str
    kind: str
    dtype: str  # "f32" or "bf16"
    num_heads: int
    head_dim: int
    seqlens_q: list
    seqlens_k: list
    # Per-token ids.  q-side arrays are indexed by packed query row, k-side
    # arrays by packed key row (cu_k[s] + j).  For self-attention layouts the
    # q and k arrays are the same object.
    seg_q: Optional[np.ndarray] = None
    seg_k: Optional[np.ndarray] = None
    role_q: Optional[np.ndarray] = None
    role_k: Optional[np.ndarray] = None
    turn_q: Optional[np.ndarray] = None
    turn_k: Optional[np.ndarray] = None
    doc_q: Optional[np.ndarray] = None
    doc_k: Optional[np.ndarray] = None
    terms: tuple = ()  # composed kind: one group of ANDed terms, or a tuple of groups (ORed)
    think_role: int = THINK_ROLE
    loss_role: int = LOSS_ROLE
    history_role: int = HISTORY_ROLE
    paged: bool = False
    page_size: int = 16
    notes: dict = field(default_factory=dict)

    def __post_init__(self):
        assert self.kind in KINDS, self.kind
        assert self.dtype in ("f32", "bf16"), self.dtype
        self.seqlens_q = [int(x) for x in self.seqlens_q]
        self.seqlens_k = [int(x) for x in self.seqlens_k]
        assert len(self.seqlens_q) == len(self.seqlens_k)

    @property
    def n_seqs(self) -> int:
        return len(self.seqlens_q)

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens_q)]).astype(np.int32)

    @property
    def cu_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens_k)]).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(sum(self.seqlens_q))

    @property
    def total_k(self) -> int:
        return int(sum(self.seqlens_k))

    @property
    def max_q(self) -> int:
        return max(self.seqlens_q) if self.seqlens_q else 0

    @property
    def max_k(self) -> int:
        return max(self.seqlens_k) if self.seqlens_k else 0

    def pages_per_seq(self) -> list:
        ps = self.page_size
        return [(c + ps - 1) // ps for c in self.seqlens_k]

    def ids_for_seq(self, s: int) -> dict:
        """The id slices that belong to sequence ``s`` (q-side and k-side)."""
        cq, ck = self.cu_q, self.cu_k
        out = {}
        for name in ("seg_q", "role_q", "turn_q", "doc_q"):
            a = getattr(self, name)
            if a is not None:
                out[name] = a[cq[s]:cq[s + 1]]
        for name in ("seg_k", "role_k", "turn_k", "doc_k"):
            a = getattr(self, name)
            if a is not None:
                out[name] = a[ck[s]:ck[s + 1]]
        return out


# --------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------

def causal_single(L: int = 256, H: int = 2, D: int = 64, dtype: str = "f32") -> Layout:
    """One causal sequence (batch 1, no packing)."""
    return Layout("causal_single", "causal", dtype, H, D, [L], [L])


def full_single(Lq: int, Lk: int, H: int = 1, D: int = 8, dtype: str = "f32") -> Layout:
    """One sequence with every key visible to every query (no mask)."""
    return Layout("full_single", "full", dtype, H, D, [Lq], [Lk])


def packed_documents(seed: int = 0, n_docs: int = 8, lo: int = 64, hi: int = 2048,
                     H: int = 16, D: int = 128, dtype: str = "bf16") -> Layout:
    """Packed causal documents; each document is its own sequence.

    Lengths are integers drawn uniformly from [lo, hi] inclusive.
    """
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, size=n_docs, endpoint=True).astype(int).tolist()
    return Layout("packed_documents", "causal", dtype, H, D, lens, lens,
                  notes={"lengths": lens})


def shared_prefix(prefix: int = 4096, n_suffix: int = 16, suffix: int = 1024,
                  H: int = 32, D: int = 128, dtype: str = "bf16") -> Layout:
    """[P, S_1, ..., S_n] packed in one sequence; segment 0 is the prefix."""
    seg = np.concatenate([np.zeros(prefix, np.int32)] +
                         [np.full(suffix, i, np.int32) for i in range(1, n_suffix + 1)])
    T = int(seg.size)
    return Layout("shared_prefix", "shared_prefix", dtype, H, D, [T], [T],
                  seg_q=seg, seg_k=seg,
                  notes={"prefix": prefix, "n_suffix": n_suffix, "suffix": suffix})


def strip_thinking(n_turns: int = 8, user: int = 256, think: int = 1536, answer: int = 512,
                   H: int = 32, D: int = 128, dtype: str = "bf16") -> Layout:
    """n_turns of (user, think, answer) spans packed in one sequence."""
    roles, turns = [], []
    for t in range(n_turns):
        for r, n in ((0, user), (THINK_ROLE, think), (2, answer)):
            roles.append(np.full(n, r, np.int32))
            turns.append(np.full(n, t, np.int32))
    role = np.concatenate(roles)
    turn = np.concatenate(turns)
    T = int(role.size)
    return Layout("strip_thinking", "strip_thinking", dtype, H, D, [T], [T],
                  role_k=role, turn_q=turn, turn_k=turn,
                  notes={"n_turns": n_turns, "user": user, "think": think, "answer": answer})


def strip_thinking_duplicated(n_turns: int = 8, user: int = 256, think: int = 1536,
                              answer: int = 512, H: int = 32, D: int = 128,
                              dtype: str = "bf16") -> Layout:
    """n_turns of (user, think, answer loss copy, answer history copy) spans
    packed in one sequence: the strip-thinking conversation with every
    answer span written twice, the history copy right after the loss copy."""
    roles, turns = [], []
    for t in range(n_turns):
        for r, n in ((USER_ROLE, user), (THINK_ROLE, think), (LOSS_ROLE, answer),
                     (HISTORY_ROLE, answer)):
            roles.append(np.full(n, r, np.int32))
            turns.append(np.full(n, t, np.int32))
    role = np.concatenate(roles)
    turn = np.concatenate(turns)
    T = int(role.size)
    return Layout("strip_thinking_duplicated", "strip_thinking_duplicated", dtype, H, D, [T], [T],
                  role_q=role, role_k=role, turn_q=turn, turn_k=turn,
                  notes={"n_turns": n_turns, "user": user, "think": think, "answer": answer})


def shared_prefix_groups(n_groups: int = 4, prefix: int = 1024, n_suffix: int = 8,
                         suffix: int = 384, pad: int = 256, H: int = 32, D: int = 128,
                         dtype: str = "bf16") -> Layout:
    """Several shared-prefix groups and trailing padding packed in ONE
    sequence, told apart by document ids (composed: causal AND document AND
    shared-prefix).  Group g is [P_g, S_g1, ..., S_gn] with document id g and
    segment ids restarting per group (0 for P_g); padding has document -1."""
    segs, docs = [], []
    for g in range(n_groups):
        seg = np.concatenate([np.zeros(prefix, np.int32)] +
                             [np.full(suffix, i, np.int32) for i in range(1, n_suffix + 1)])
        segs.append(seg)
        docs.append(np.full(seg.size, g, np.int32))
    segs.append(np.zeros(pad, np.int32))
    docs.append(np.full(pad, -1, np.int32))
    seg = np.concatenate(segs)
    doc = np.concatenate(docs)
    T = int(seg.size)
    return Layout("shared_prefix_groups", "composed", dtype, H, D, [T], [T], seg_q=seg, seg_k=seg,
                  doc_q=doc, doc_k=doc, terms=("causal", "document", "shared_prefix"),
                  notes={"n_groups": n_groups, "prefix": prefix, "n_suffix": n_suffix,
                         "suffix": suffix, "pad": pad})


def prefix_lm(prefixes=(1024,), lengths=(4096,), H: int = 8, D: int = 128,
              dtype: str = "bf16") -> Layout:
    """Prefix-LM sequences: the first prefixes[s] tokens of sequence s see
    each other both ways, the rest is causal -- the composed mask (causal)
    OR (document), with the prefix in document 0 and the rest in -1."""
    lens = [int(n) for n in lengths]
    doc = np.concatenate([np.where(np.arange(n) < p, 0, -1) for p, n in zip(prefixes, lens)]
                         ).astype(np.int32) if lens else np.zeros(0, np.int32)
    return Layout("prefix_lm", "composed", dtype, H, D, lens, lens, doc_q=doc, doc_k=doc,
                  terms=(("causal",), ("document",)), notes={"prefixes": [int(p) for p in prefixes]})


def paged_decode(seed: int = 0, n_seqs: int = 64, lo: int = 512, hi: int = 32768,
                 page_size: int = 16, H: int = 32, D: int = 128, dtype: str = "bf16") -> Layout:
    """One new query per sequence over a paged context of ragged length."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi, size=n_seqs, endpoint=True).astype(int).tolist()
    return Layout("paged_decode", "causal", dtype, H, D, [1] * n_seqs, ctx,
                  paged=True, page_size=page_size, notes={"ctx": ctx})


CONFIG_NAMES = ("causal_f32", "packed_documents", "shared_prefix", "strip_thinking", "paged_decode",
                "strip_thinking_duplicated", "shared_prefix_groups")


def config(name: str, seed: int = 0) -> Layout:
    """The named workloads at their full sizes."""
    if name == "causal_f32":
        return causal_single(256, 2, 64, "f32")
    if name == "packed_documents":
        return packed_documents(seed)
    if name == "shared_prefix":
        return shared_prefix()
    if name == "strip_thinking":
        return strip_thinking()
    if name == "paged_decode":
        return paged_decode(seed)
    if name == "strip_thinking_duplicated":
        return strip_thinking_duplicated()
    if name == "shared_prefix_groups":
        return shared_prefix_groups()
    if name == "prefix_lm":
        return prefix_lm((2048,), (8192,), H=16, D=128)
    raise KeyError(name)


def random_layout(rng: np.random.Generator, kind: str, n_seqs: int = 3, max_len: int = 40,
                  H: int = 2, D: int = 8, dtype: str = "f32", decode_q: Optional[int] = None,
                  paged: bool = False, page_size: int = 4, n_segments: int = 3,
                  n_turns: int = 3, min_len: int = 1) -> Layout:
    """A small random layout for property tests.

    Self-attention (Lq == Lk) unless ``decode_q`` is given, in which case each
    sequence has min(decode_q, Lk) queries at the end of its context.  Ids are
    random but structured: segment ids are runs with 0 first; roles cycle
    through user/think/answer spans of random length inside each turn.
    """
    lens_k = rng.integers(min_len, max_len, size=n_seqs, endpoint=True).astype(int).tolist()
    if decode_q is None:
        lens_q = list(lens_k)
    else:
        lens_q = [min(decode_q, lk) for lk in lens_k]
    seg_k = role_k = turn_k = seg_q = turn_q = role_q = doc_k = doc_q = None
    terms = ()
    if kind == "shared_prefix":
        parts = []
        for L in lens_k:
            cuts = np.sort(rng.integers(0, L + 1, size=n_segments - 1))
            bounds = np.concatenate([[0], cuts, [L]])
            ids = np.zeros(L, np.int32)
            for i in range(n_segments):
                ids[bounds[i]:bounds[i + 1]] = i
            parts.append(ids)
        seg_k = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
    elif kind == "strip_thinking":
        rparts, tparts = [], []
        for L in lens_k:
            role = np.zeros(L, np.int32)
            turn = np.zeros(L, np.int32)
            pos = 0
            t = 0
            while pos < L:
                for r in (0, THINK_ROLE, 2):
                    n = int(rng.integers(1, max(2, L // (n_turns * 2) + 2)))
                    role[pos:pos + n] = r
                    turn[pos:pos + n] = t
                    pos += n
                    if pos >= L:
                        break
                t += 1
            rparts.append(role)
            tparts.append(turn)
        role_k = np.concatenate(rparts).astype(np.int32) if rparts else np.zeros(0, np.int32)
        turn_k = np.concatenate(tparts).astype(np.int32) if tparts else np.zeros(0, np.int32)
    elif kind == "strip_thinking_duplicated":
        # turns of user, think, loss-copy and history-copy spans; the two
        # answer copies have one length; the sequence may end inside a turn
        rparts, tparts = [], []
        for L in lens_k:
            role = np.zeros(L, np.int32)
            turn = np.zeros(L, np.int32)
            pos = 0
            t = 0
            cap = max(2, L // (n_turns * 3) + 2)
            while pos < L:
                nu, nt, na = (int(x) for x in rng.integers(1, cap, size=3))
                for r, n in ((USER_ROLE, nu), (THINK_ROLE, nt), (LOSS_ROLE, na), (HISTORY_ROLE, na)):
                    role[pos:pos + n] = r
                    turn[pos:pos + n] = t
                    pos += n
                    if pos >= L:
                        break
                t += 1
            rparts.append(role)
            tparts.append(turn)
        role_k = np.concatenate(rparts).astype(np.int32) if rparts else np.zeros(0, np.int32)
        turn_k = np.concatenate(tparts).astype(np.int32) if tparts else np.zeros(0, np.int32)
    elif kind == "composed":
        # a random non-empty subset of the terms, with every id array drawn:
        # documents as runs (some padding, id -1), segments as runs with 0
        # first inside each document, roles and turns as in strip_thinking
        # one AND-group, or (half the time) an OR of two or three groups
        n_groups = 1 if rng.random() < 0.5 else int(rng.integers(2, 4))
        groups = []
        for _ in range(n_groups):
            g = ()
            while not g:
                g = tuple(t for t in TERMS if rng.random() < 0.6)
            groups.append(g)
        terms = groups[0] if n_groups == 1 else tuple(groups)
        sp, rp, tp, dp = [], [], [], []
        for L in lens_k:
            doc = np.zeros(L, np.int32)
            seg = np.zeros(L, np.int32)
            role = np.zeros(L, np.int32)
            turn = np.zeros(L, np.int32)
            pos, d = 0, 0
            while pos < L:
                e = min(L, pos + int(rng.integers(1, max(2, L // 2 + 1))))
                doc[pos:e] = -1 if rng.random() < 0.15 else d
                cuts = np.sort(rng.integers(pos, e + 1, size=n_segments - 1))
                bounds = np.concatenate([[pos], cuts, [e]])
                for i in range(n_segments):
                    seg[bounds[i]:bounds[i + 1]] = i
                d += 1
                pos = e
            p2, t = 0, 0
            while p2 < L:
                for r in (0, THINK_ROLE, 2):
                    n = int(rng.integers(1, max(2, L // (n_turns * 2) + 2)))
                    role[p2:p2 + n] = r
                    turn[p2:p2 + n] = t
                    p2 += n
                    if p2 >= L:
                        break
                t += 1
            sp.append(seg)
            rp.append(role)
            tp.append(turn)
            dp.append(doc)
        cat = lambda parts: np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
        seg_k, role_k, turn_k, doc_k = cat(sp), cat(rp), cat(tp), cat(dp)
    # q-side ids: the last lens_q[s] key positions of each sequence.
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(int)

    def q_side(arr):
        if arr is None:
            return None
        if decode_q is None:
            return arr
        return np.concatenate([arr[cu_k[s + 1] - lens_q[s]:cu_k[s + 1]] for s in range(n_seqs)]
                              ).astype(np.int32)

    seg_q = q_side(seg_k)
    turn_q = q_side(turn_k)
    doc_q = q_side(doc_k)
    if kind == "strip_thinking_duplicated":
        role_q = q_side(role_k)
    return Layout(f"random_{kind}", kind, dtype, H, D, lens_q, lens_k,
                  seg_q=seg_q, seg_k=seg_k, role_q=role_q, role_k=role_k, turn_q=turn_q,
                  turn_k=turn_k, doc_q=doc_q, doc_k=doc_k, terms=terms,
                  paged=paged, page_size=page_size)


# --------------------------------------------------------------------------
# Tensor values.
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype(name: str):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _normal(shape, seed: int, tag: int, device, dtype_name: str):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(seed, tag))
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.to(_dtype(dtype_name))


def make_dense_qkv(layout: Layout, seed: int = 0, device="cpu"):
    """q [total_q, H, D], k and v [total_k, H, D], contiguous, layout dtype."""
    H, D = layout.num_heads, layout.head_dim
    q = _normal((layout.total_q, H, D), seed, 1, device, layout.dtype)
    k = _normal((layout.total_k, H, D), seed, 2, device, layout.dtype)
    v = _normal((layout.total_k, H, D), seed, 3, device, layout.dtype)
    return q, k, v


def make_paged_kv(layout: Layout, seed: int = 0, device="cpu", extra_pages: int = 0,
                  table_pad: int = 0):
    """q, k_pool, v_pool, block_table for a paged layout.

    Every sequence's pages are distinct physical pages chosen by a seeded
    permutation of the pool, so logically adjacent pages are scattered.
    ``block_table[s, p]`` is the physical page of logical page ``p``; unused
    entries hold -1.  ``extra_pages`` adds pool pages that no sequence uses.
    """
    torch = _torch()
    H, D, ps = layout.num_heads, layout.head_dim, layout.page_size
    npg = layout.pages_per_seq()
    n_pages = int(sum(npg)) + int(extra_pages)
    rng = np.random.default_rng(derive_seed(seed, 7))
    perm = rng.permutation(n_pages).astype(np.int32)
    width = max(npg) + int(table_pad) if npg else 1
    table = np.full((layout.n_seqs, max(width, 1)), -1, np.int32)
    pos = 0
    for s, n in enumerate(npg):
        table[s, :n] = perm[pos:pos + n]
        pos += n
    q = _normal((layout.total_q, H, D), seed, 1, device, layout.dtype)
    k_pool = _normal((n_pages, ps, H, D), seed, 2, device, layout.dtype)
    v_pool = _normal((n_pages, ps, H, D), seed, 3, device, layout.dtype)
    bt = torch.from_numpy(table).to(device)
    return q, k_pool, v_pool, bt
