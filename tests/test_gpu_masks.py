"""GPU vs oracle, bit-exact: tile classes, kv-tile lists, the row schedule,
the dense-mask export and the paged gather."""

import numpy as np
import pytest
import torch

import synth
from block_sparse_masked_amd import bmattn as bm
from oracle import paged as opaged

import _hip
from _hip import DEV, say

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (2, 3), (4, 4), (13, 8), (16, 64), (64, 16), (128, 64), (1, 64), (37, 29),
          (128, 128), (256, 64)]
KIND_SEED = {"full": 1, "causal": 2, "shared_prefix": 3, "strip_thinking": 4,
             "strip_thinking_duplicated": 5, "composed": 6}


@pytest.mark.parametrize("decode_q", [None, 1, 3])
@pytest.mark.parametrize("kind", synth.KINDS)
def test_tiles_bit_exact_random_layouts(kind, decode_q):
    rng = np.random.default_rng(100 * KIND_SEED[kind] + (decode_q or 0))
    for trial in range(3):
        lay = synth.random_layout(rng, kind, n_seqs=3, max_len=90, decode_q=decode_q)
        desc = _hip.desc_for(lay)
        for BM, BN in SHAPES:
            say(f"tiles kind={kind} decode_q={decode_q} trial={trial} lens={lay.seqlens_k} BM={BM} BN={BN}")
            t = _hip.check_tiles(lay, desc, BM, BN)
            _hip.check_dense(lay, desc, t)


def test_tiles_empty_and_tiny_sequences():
    lay = synth.Layout("edge", "causal", "f32", 1, 8, [0, 1, 5, 0], [0, 1, 5, 0])
    desc = _hip.desc_for(lay)
    for BM, BN in [(1, 1), (4, 4), (128, 64)]:
        say(f"tiles empty sequences BM={BM} BN={BN}")
        t = _hip.check_tiles(lay, desc, BM, BN)
        _hip.check_dense(lay, desc, t)


@pytest.mark.parametrize("name", ["causal_f32", "packed_documents", "shared_prefix",
                                  "strip_thinking", "strip_thinking_duplicated",
                                  "shared_prefix_groups", "prefix_lm"])
def test_tiles_bit_exact_named_workloads(name):
    lay = synth.config(name)
    desc = _hip.desc_for(lay)
    say(f"tiles {name} at 128x64")
    t = _hip.check_tiles(lay, desc, 128, 64)
    say(f"dense export {name}")
    _hip.check_dense(lay, desc, t)


def test_tiles_bit_exact_paged_decode():
    lay = synth.config("paged_decode")
    desc = _hip.desc_for(lay)
    say("tiles paged_decode at 1x64")
    t = _hip.check_tiles(lay, desc, 1, 64)
    # every listed tile but a sequence's ragged last one is FULL
    fc = t.full_cnt.cpu().numpy()
    pc = t.part_cnt.cpu().numpy()
    ctx = np.array(lay.seqlens_k)
    assert np.array_equal(fc, ctx // 64)
    assert np.array_equal(pc, (ctx % 64 != 0).astype(np.int32))


def test_validate_flags():
    lay = synth.paged_decode(seed=1, n_seqs=4, lo=5, hi=60, page_size=4, H=1, D=8, dtype="f32")
    desc = _hip.desc_for(lay)
    q, kp, vp, bt = synth.make_paged_kv(lay, seed=1, device="cpu")
    btd = bt.to(DEV)
    say("validate: good description")
    assert bm.validate(desc, btd, 4, kp.shape[0]) == 0
    bad = btd.clone()
    bad[0, 0] = kp.shape[0]
    say("validate: bad block table entry")
    assert bm.validate(desc, bad, 4, kp.shape[0]) == 8
    cu = torch.tensor(lay.cu_k, dtype=torch.int32)
    cu[2] = cu[1] - 1  # a decreasing offset
    d2 = bm.MaskDesc.create("causal", lay.cu_q, cu, desc.max_seqlen_q, desc.max_seqlen_k, device=DEV)
    say("validate: decreasing cu_seqlens_k")
    assert bm.validate(d2) & 2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("page_size", [1, 3, 4, 16])
def test_paged_gather_byte_equal(dtype, page_size):
    rng = np.random.default_rng(page_size)
    for trial in range(2):
        ctx = rng.integers(1, 200, size=4).tolist() + [13]
        lay = synth.Layout("gather", "causal", dtype, 3, 64 if dtype == "f32" else 128,
                           [1] * len(ctx), ctx, paged=True, page_size=page_size)
        q, kp, vp, bt = synth.make_paged_kv(lay, seed=trial, device="cpu", extra_pages=5,
                                            table_pad=2)
        desc = _hip.desc_for(lay)
        say(f"gather dtype={dtype} page={page_size} ctx={ctx}")
        got = bm.paged_gather(kp.to(DEV), bt.to(DEV), desc).cpu()
        raw = kp.view(torch.int16) if dtype == "bf16" else kp.view(torch.int32)
        gotr = got.view(torch.int16) if dtype == "bf16" else got.view(torch.int32)
        cu = lay.cu_k
        for s in range(lay.n_seqs):
            for tile in (1, 13, None):
                want = opaged.paged_gather(raw.numpy(), bt[s].numpy(), ctx[s], page_size, tile=tile)
                assert want.tobytes() == gotr[cu[s]:cu[s + 1]].numpy().tobytes(), (s, tile)


def test_paged_gather_byte_equal_decode_contexts():
    # The paged-decode workload's contexts and page table at 2 heads.
    lay = synth.paged_decode(seed=0, H=2)
    q, kp, vp, bt = synth.make_paged_kv(lay, seed=0, device="cpu")
    desc = _hip.desc_for(lay)
    say(f"gather paged_decode contexts, total {lay.total_k} tokens")
    got = bm.paged_gather(kp.to(DEV), bt.to(DEV), desc).cpu().view(torch.int16).numpy()
    raw = kp.view(torch.int16).numpy()
    cu = lay.cu_k
    for s in range(lay.n_seqs):
        want = opaged.paged_gather(raw, bt[s].numpy(), lay.seqlens_k[s], 16)
        assert want.tobytes() == got[cu[s]:cu[s + 1]].tobytes(), s


def _dup_flags(lay):
    src = bm.MaskDesc.create("strip_thinking", lay.cu_q, lay.cu_k, max(lay.max_q, 1),
                             max(lay.max_k, 1), device=DEV, role_k=lay.role_k, turn_q=lay.turn_q,
                             turn_k=lay.turn_k)
    role_q = torch.as_tensor(lay.role_q, dtype=torch.int32, device=DEV)
    _, flags = bm.duplicated_answer_ids(src, role_q, check=True)
    return int(flags.item())


def test_duplicated_answer_layout_flags():
    # The device check of the layout conditions under which the relabelled
    # ids are exact: 0 on well-formed layouts, one bit per broken condition.
    rng = np.random.default_rng(21)
    for dq in (None, 2):
        lay = synth.random_layout(rng, "strip_thinking_duplicated", n_seqs=20, max_len=300,
                                  decode_q=dq)
        say(f"duplicated flags: well-formed decode_q={dq}")
        assert _dup_flags(lay) == 0
    lay = synth.strip_thinking_duplicated(n_turns=3, user=2, think=3, answer=2, H=1, D=8)

    def broken(**ids):
        base = dict(role_q=lay.role_q.copy(), role_k=lay.role_k.copy(), turn_q=lay.turn_q.copy(),
                    turn_k=lay.turn_k.copy())
        for name, fn in ids.items():
            base[name] = fn(base[name])
        return synth.Layout("b", "strip_thinking_duplicated", "f32", 1, 8, lay.seqlens_q,
                            lay.seqlens_k, **base)

    def dec_turn(t):
        t = t.copy()
        t[-1] = 0
        return t

    def hist_first(r):
        r = r.copy()
        h = np.nonzero(r == synth.HISTORY_ROLE)[0]
        r[h[0]], r[h[0] - 1] = r[h[0] - 1], r[h[0]]  # history copy before a loss-copy token
        return r

    def q_other(r):
        r = r.copy()
        r[0] = synth.THINK_ROLE
        return r

    def max_turn(t):
        t = t.copy()
        t[-1] = np.iinfo(np.int32).max
        return t

    say("duplicated flags: broken layouts")
    assert _dup_flags(broken(turn_k=dec_turn, turn_q=dec_turn)) == 1
    assert _dup_flags(broken(role_k=hist_first, role_q=hist_first)) == 2
    assert _dup_flags(broken(role_q=q_other)) == 4
    assert _dup_flags(broken(turn_q=max_turn, turn_k=max_turn)) == 8


def test_duplicated_answer_ids_in_place():
    rng = np.random.default_rng(8)
    lay = synth.random_layout(rng, "strip_thinking_duplicated", n_seqs=3, max_len=200)
    d1 = _hip.desc_for(lay)
    src = bm.MaskDesc.create("strip_thinking", lay.cu_q, lay.cu_k, lay.max_q, lay.max_k, device=DEV,
                             role_k=lay.role_k, turn_q=lay.turn_q, turn_k=lay.turn_k)
    role_q = torch.as_tensor(lay.role_q, dtype=torch.int32, device=DEV)
    rk, tq = src.role_k.clone(), src.turn_q.clone()
    say("duplicated ids in place")
    dst = bm.MaskDesc(src.kind, src.n_seqs, src.max_seqlen_q, src.max_seqlen_k, src.total_q,
                      src.total_k, src.cu_seqlens_q, src.cu_seqlens_k, None, None, src.role_k,
                      src.turn_q, src.turn_k, src.think_role)
    bm.duplicated_answer_ids(src, role_q, out=dst)
    torch.cuda.synchronize()
    assert torch.equal(dst.role_k, d1.role_k) and torch.equal(dst.turn_q, d1.turn_q)
    assert not torch.equal(rk, dst.role_k) and not torch.equal(tq, dst.turn_q)
    # rerunning into a description's own arrays reproduces them
    before = (d1.role_k.clone(), d1.turn_q.clone())
    d1.role_k.fill_(-5)
    d1.turn_q.fill_(-5)
    bm.relabel(d1)
    torch.cuda.synchronize()
    assert torch.equal(d1.role_k, before[0]) and torch.equal(d1.turn_q, before[1])


@pytest.mark.parametrize("terms", [("causal",), ("document",), ("causal", "document"),
                                   ("causal", "shared_prefix"), ("causal", "strip_thinking"),
                                   ("document", "shared_prefix", "strip_thinking"),
                                   ("causal", "document", "shared_prefix", "strip_thinking")])
def test_composed_every_term_set(terms):
    # Each term set on random layouts (with padding and several documents).
    rng = np.random.default_rng(sum(bm.TERM_CODES[t] for t in terms) * 31 + len(terms))
    for trial in range(2):
        lay = synth.random_layout(rng, "composed", n_seqs=3, max_len=200)
        lay.terms = terms
        desc = _hip.desc_for(lay)
        for BM, BN in ((128, 64), (64, 128), (16, 16), (1, 64)):
            say(f"composed terms={terms} trial={trial} lens={lay.seqlens_k} {BM}x{BN}")
            t = _hip.check_tiles(lay, desc, BM, BN)
            _hip.check_dense(lay, desc, t)


OR_GROUPS = [
    (("causal",), ("document",)),  # prefix-LM
    (("causal", "strip_thinking"), ("document", "shared_prefix")),
    (("document",), ("shared_prefix",), ("causal",)),
    (("causal", "shared_prefix"), ("causal", "strip_thinking")),
    (("strip_thinking",), ("document", "causal"), ("shared_prefix", "causal"), ("causal",)),
]


@pytest.mark.parametrize("gi", range(len(OR_GROUPS)))
def test_composed_or_groups(gi):
    # OR of AND-groups on random layouts: tile classes, lists and the dense
    # mask bit for bit against the oracle (the classifier enumerates them).
    groups = OR_GROUPS[gi]
    rng = np.random.default_rng(500 + gi)
    for trial in range(2):
        lay = synth.random_layout(rng, "composed", n_seqs=3, max_len=260)
        lay.terms = groups
        desc = _hip.desc_for(lay)
        for BM, BN in ((128, 64), (64, 128), (16, 16), (1, 64)):
            say(f"composed OR groups={groups} trial={trial} lens={lay.seqlens_k} {BM}x{BN}")
            t = _hip.check_tiles(lay, desc, BM, BN)
            _hip.check_dense(lay, desc, t)


def test_prefix_lm_tiles():
    # Prefix-LM sequences of several prefix lengths (0, inside a tile, on a
    # tile edge, the whole sequence): tiles at the forward's and the
    # backward's shapes and the decode shape.
    lay = synth.prefix_lm(prefixes=(0, 77, 128, 300, 1000), lengths=(300, 900, 640, 300, 1000), H=1)
    desc = _hip.desc_for(lay)
    for BM, BN in ((128, 64), (64, 128), (1, 64)):
        say(f"prefix-LM tiles {BM}x{BN}")
        _hip.check_tiles(lay, desc, BM, BN)


def test_composed_single_terms_match_plain_kinds_bit_exact():
    # {causal, shared_prefix} over the same ids builds the same block mask as
    # the SHARED_PREFIX kind; likewise strip-thinking and causal.
    rng = np.random.default_rng(77)
    for kind, terms in (("causal", ("causal",)), ("shared_prefix", ("causal", "shared_prefix")),
                        ("strip_thinking", ("causal", "strip_thinking"))):
        lay = synth.random_layout(rng, kind, n_seqs=3, max_len=400)
        plain = _hip.desc_for(lay)
        comp = bm.MaskDesc.create("composed", lay.cu_q, lay.cu_k, lay.max_q, lay.max_k, device=DEV,
                                  seg_q=lay.seg_q, seg_k=lay.seg_k, role_k=lay.role_k,
                                  turn_q=lay.turn_q, turn_k=lay.turn_k, terms=terms)
        say(f"composed {terms} vs plain {kind}")
        a = bm.build_block_mask(plain, 128, 64)
        b = bm.build_block_mask(comp, 128, 64)
        torch.cuda.synchronize()
        for f in ("tile_class", "full_cnt", "part_cnt", "full_idx", "part_idx", "row_order"):
            assert torch.equal(getattr(a, f), getattr(b, f)), (kind, f)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind", ["causal", "full"])
@pytest.mark.parametrize("BM,BN", [(128, 64), (1, 64)])
@pytest.mark.parametrize("layout", ["many_rows", "many_tiles", "many_kv_tiles"])
def test_tiles_general_classifier_causal_and_full(kind, BM, BN, layout):
    # CAUSAL and FULL masks of more than 1024 tile rows (1100 short
    # sequences) or more than 65 536 tiles (one sequence of 33 000 tokens)
    # take the general classifier, not the one-workgroup path of small masks.
    # Rows of more than 4095 kv tiles (contexts of 262 144 keys and more) are
    # ranked by comparing every pair of rows, not from count histograms.
    if layout == "many_rows":
        rng = np.random.default_rng(11 + BM + len(kind))
        lens = lens_k = [int(x) for x in rng.integers(1, 300, size=1100)]
    elif layout == "many_tiles":
        lens = lens_k = [33000]
    else:
        lens = [5, 1, 130, 3, 64, 200, 7, 2, 33]
        lens_k = [270000, 262145, 100000, 262143, 262200, 300000, 1000, 270001, 262144]
    lay = synth.Layout(layout, kind, "bf16", 1, 128, lens, lens_k)
    n_qt, n_kt = -(-max(lens) // BM), -(-max(lens_k) // BN)
    rows = len(lens) * n_qt
    assert rows > 1024 or rows * n_kt > 65536
    desc = _hip.desc_for(lay)
    say(f"general classifier kind={kind} {layout} BM={BM} BN={BN} rows={rows} tiles={rows * n_kt}")
    _hip.check_tiles(lay, desc, BM, BN)
