"""GPU forward vs the float64 oracle (O and LSE within tolerance), on small
layouts that span several tiles with ragged tails, on every named workload
at full size (every row of every head), and the
invariants of the forward: run-to-run bit-reproducibility, packing
invariance, paged == contiguous, and untouched unreachable K/V."""

import math

import numpy as np
import pytest
import torch

import synth
from block_sparse_masked_amd import bmattn as bm
from oracle import forward as oforward

import _hip
from _hip import DEV, say

pytestmark = pytest.mark.gpu


def test_causal_f32_config():
    lay = synth.config("causal_f32")
    say("forward causal_f32 (1x2x256x64)")
    o, lse, q, k, v, desc, t = _hip.run_dense(lay, seed=0)
    O, L = _hip.oracle_dense(lay, q, k, v)
    _hip.check_close(o, lse, O, L, "f32", "causal_f32")


def test_page_example_noncausal_and_causal():
    # Triton from First Principles, Ch. 21, section 21.2's script inputs: the
    # library's FULL and CAUSAL forwards differ by the printed 1.7221667...
    torch.manual_seed(0)
    q, k, v = torch.randn(20, 8), torch.randn(20, 8), torch.randn(20, 8)
    pad = lambda x: torch.nn.functional.pad(x, (0, 56)).reshape(20, 1, 64)
    outs = {}
    for kind in ("full", "causal"):
        lay = synth.Layout("page", kind, "f32", 1, 64, [20], [20])
        desc = _hip.desc_for(lay)
        t = bm.build_block_mask(desc, 128, 64)
        # zero-padded head_dim 64 keeps q.k; the scale stays 1/sqrt(8)
        o, _ = bm.forward(pad(q).to(DEV), pad(k).to(DEV), pad(v).to(DEV), desc, t,
                          scale=1 / math.sqrt(8))
        outs[kind] = o.cpu()[:, 0, :8]
    diff = (outs["full"] - outs["causal"]).abs().max().item()
    assert abs(diff - 1.7221667766571045) < 1e-5


CASES = []
for kind in synth.KINDS:
    for dtype, D in (("f32", 64), ("bf16", 128), ("bf16", 64), ("f32", 128)):
        CASES.append((kind, dtype, D))


@pytest.mark.parametrize("kind,dtype,D", CASES)
def test_prefill_random_layouts(kind, dtype, D):
    rng = np.random.default_rng(7 + len(kind) + D)
    for trial in range(2):
        lay = synth.random_layout(rng, kind, n_seqs=3, max_len=330, min_len=1, H=2, D=D,
                                  dtype=dtype)
        say(f"prefill kind={kind} dtype={dtype} D={D} lens={lay.seqlens_q}")
        o, lse, q, k, v, desc, t = _hip.run_dense(lay, seed=trial)
        O, L = _hip.oracle_dense(lay, q, k, v)
        _hip.check_close(o, lse, O, L, dtype, f"{kind}/{dtype}/D{D}")


@pytest.mark.parametrize("kind", synth.KINDS)
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_prefill_paged(kind, dtype, D):
    rng = np.random.default_rng(31 + D)
    lay = synth.random_layout(rng, kind, n_seqs=3, max_len=300, min_len=60, H=2, D=D, dtype=dtype,
                              paged=True, page_size=16)
    q, kp, vp, bt = synth.make_paged_kv(lay, seed=4, device="cpu", extra_pages=3)
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, 128, 64)
    say(f"prefill paged kind={kind} dtype={dtype} lens={lay.seqlens_q}")
    o, lse = bm.forward(q.to(DEV), kp.to(DEV), vp.to(DEV), desc, t, block_table=bt.to(DEV))
    O, L = oforward.forward(lay, q, k_pool=kp, v_pool=vp, block_table=bt)
    _hip.check_close(o, lse, O, L, dtype, f"paged {kind}")


@pytest.mark.parametrize("kind", synth.KINDS)
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_decode_layouts(kind, paged, dtype, D):
    rng = np.random.default_rng(53 + D + paged)
    for nq in (1, 3):
        lay = synth.random_layout(rng, kind, n_seqs=4, max_len=900, min_len=1, H=5, D=D,
                                  dtype=dtype, decode_q=nq, paged=paged, page_size=16)
        desc = _hip.desc_for(lay)
        t = bm.build_block_mask(desc, 1, 64)
        say(f"decode kind={kind} paged={paged} dtype={dtype} D={D} q={nq} ctx={lay.seqlens_k}")
        if paged:
            q, kp, vp, bt = synth.make_paged_kv(lay, seed=nq, device="cpu", extra_pages=2)
            o, lse = bm.forward(q.to(DEV), kp.to(DEV), vp.to(DEV), desc, t, block_table=bt.to(DEV))
            O, L = oforward.forward(lay, q, k_pool=kp, v_pool=vp, block_table=bt)
        else:
            q, k, v = synth.make_dense_qkv(lay, seed=nq, device="cpu")
            o, lse = bm.forward(q.to(DEV), k.to(DEV), v.to(DEV), desc, t)
            O, L = oforward.forward(lay, q, k, v)
        _hip.check_close(o, lse, O, L, dtype, f"decode {kind}")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_prefix_lm_prefill_decode_and_paged(dtype, D):
    # The OR composition (causal) OR (document): prefix-LM sequences with the
    # prefix inside a tile, on a tile edge and the whole sequence; prefill on
    # contiguous and paged K/V, then decode of the last 3 positions.
    lay = synth.prefix_lm(prefixes=(77, 128, 300), lengths=(500, 640, 300), H=2, D=D, dtype=dtype)
    say(f"prefix-LM prefill {dtype} D={D}")
    o, lse, q, k, v, desc, t = _hip.run_dense(lay, seed=3)
    O, L = _hip.oracle_dense(lay, q, k, v)
    _hip.check_close(o, lse, O, L, dtype, "prefix-LM prefill")
    pl = synth.Layout("prefix_lm", "composed", dtype, 2, D, lay.seqlens_q, lay.seqlens_k, doc_q=lay.doc_q,
                      doc_k=lay.doc_k, terms=lay.terms, paged=True, page_size=16)
    qp, kp, vp, bt = synth.make_paged_kv(pl, seed=4, device="cpu", extra_pages=2)
    say(f"prefix-LM paged {dtype} D={D}")
    op, lp = bm.forward(qp.to(DEV), kp.to(DEV), vp.to(DEV), _hip.desc_for(pl), bm.build_block_mask(
        _hip.desc_for(pl), 128, 64), block_table=bt.to(DEV))
    Op, Lp = oforward.forward(pl, qp, k_pool=kp, v_pool=vp, block_table=bt)
    _hip.check_close(op, lp, Op, Lp, dtype, "prefix-LM paged")
    # decode: the last 3 queries of each sequence against its whole context
    cu = np.concatenate([[0], np.cumsum(lay.seqlens_k)])
    dq = np.concatenate([lay.doc_k[cu[s + 1] - 3:cu[s + 1]] for s in range(lay.n_seqs)]).astype(np.int32)
    dl = synth.Layout("prefix_lm_decode", "composed", dtype, 2, D, [3] * lay.n_seqs, lay.seqlens_k,
                      doc_q=dq, doc_k=lay.doc_k, terms=lay.terms)
    qd, kd, vd = synth.make_dense_qkv(dl, seed=5, device="cpu")
    ddesc = _hip.desc_for(dl)
    say(f"prefix-LM decode {dtype} D={D}")
    od, ld = bm.forward(qd.to(DEV), kd.to(DEV), vd.to(DEV), ddesc, bm.build_block_mask(ddesc, 1, 64))
    Od, Ld = oforward.forward(dl, qd, kd, vd)
    _hip.check_close(od, ld, Od, Ld, dtype, "prefix-LM decode")


@pytest.mark.parametrize("paged", [False, True])
def test_decode_longest_context(paged):
    # One query over 262 147 keys (4097 kv tiles of 64, 513 splits, a ragged
    # last page) beside a short sequence, every head.
    lay = synth.Layout("long_decode", "causal", "bf16", 2, 128, [1, 1], [262147, 5000], paged=paged,
                       page_size=16)
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, 1, 64)
    say(f"decode longest context paged={paged}")
    if paged:
        q, kp, vp, bt = synth.make_paged_kv(lay, seed=6, device="cpu", extra_pages=1)
        o, lse = bm.forward(q.to(DEV), kp.to(DEV), vp.to(DEV), desc, t, block_table=bt.to(DEV))
        O, L = oforward.forward(lay, q, k_pool=kp, v_pool=vp, block_table=bt)
    else:
        q, k, v = synth.make_dense_qkv(lay, seed=6, device="cpu")
        o, lse = bm.forward(q.to(DEV), k.to(DEV), v.to(DEV), desc, t)
        O, L = oforward.forward(lay, q, k, v)
    _hip.check_close(o, lse, O, L, "bf16", f"decode 262147 paged={paged}")


def test_prefill_longest_causal_row_sampled():
    # A causal sequence of 65 536 tokens: rows of up to 1024 kv tiles.  The
    # oracle takes each sampled row as the last query of its own prefix (the
    # decode form of the causal mask), so no 65 536^2 mask is built.
    from oracle import attention as oattention
    from oracle import masks as omasks

    L = 65536
    lay = synth.causal_single(L=L, H=1, D=128, dtype="bf16")
    say("prefill 65536-token causal row")
    o, lse, q, k, v, desc, t = _hip.run_dense(lay, seed=8)
    rows = sorted({0, 1, 63, 64, 127, 128, 4095, 30000, L - 2, L - 1} |
                  set(np.random.default_rng(8).integers(0, L, 16).tolist()))
    qh, kh, vh = (oforward.head_slice(x, 0) for x in (q, k, v))
    O = np.zeros((len(rows), 1, 128))
    Lse = np.zeros((1, len(rows)))
    sc = oattention.default_scale(128)
    for n, i in enumerate(rows):
        vis = omasks.visible("causal", 1, i + 1)
        O[n, 0], Lse[0, n] = (x[0] for x in oattention.three_pass(qh[i:i + 1], kh[:i + 1], vh[:i + 1], vis, sc))
    idx = torch.tensor(rows)
    _hip.check_close(o[idx], lse[:, idx], O, Lse, "bf16", "65536 causal rows")


def test_empty_sequences_and_rows_without_keys():
    # Sequences of length 0 write nothing; with more queries than keys the
    # first rows see no key: O = 0 and LSE = -inf.
    lay = synth.Layout("edge", "causal", "f32", 1, 64, [0, 5, 3], [0, 5, 1])
    q, k, v = synth.make_dense_qkv(lay, seed=0)
    desc = _hip.desc_for(lay)
    for BM in (128, 1):
        t = bm.build_block_mask(desc, BM, 64)
        say(f"edge rows BM={BM}")
        o, lse = bm.forward(q.to(DEV), k.to(DEV), v.to(DEV), desc, t)
        O, L = oforward.forward(lay, q, k, v)
        _hip.check_close(o, lse, O, L, "f32", "edge")
        assert np.isneginf(lse.cpu().numpy()[0, 5:7]).all()


def test_packed_documents_full_size():
    lay = synth.config("packed_documents")
    say(f"forward packed_documents lens={lay.seqlens_q}")
    o, lse, q, k, v, desc, t = _hip.run_dense(lay, seed=0)
    O, L = _hip.oracle_dense(lay, q, k, v)
    mx, mean = _hip.check_close(o, lse, O, L, "bf16", "packed_documents")
    say(f"packed_documents max-abs {mx:.3e} mean-abs {mean:.3e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["shared_prefix", "strip_thinking", "strip_thinking_duplicated",
                                  "shared_prefix_groups", "prefix_lm"])
def test_single_sequence_workloads_every_row_and_head(name):
    # The whole output: every query row of every head against the float64
    # oracle, max-abs and mean-abs over all of O, LSE likewise.
    lay = synth.config(name)
    say(f"forward {name} full size ({lay.total_q} tokens x {lay.num_heads} heads)")
    o, lse, q, k, v, desc, t = _hip.run_dense(lay, seed=0)
    O, L = _hip.oracle_one_sequence(lay, q, k, v)
    mx, mean = _hip.check_close(o, lse, O, L, "bf16", name)
    say(f"{name} every row and head: max-abs {mx:.3e} mean-abs {mean:.3e}")


@pytest.mark.timeout(900)
def test_paged_decode_every_sequence_and_head():
    # Every sequence and head of the 64-sequence paged decode batch; one
    # sequence's pages at a time come to the host.
    lay = synth.config("paged_decode")
    say(f"forward paged_decode full size, {lay.total_k} context tokens")
    q, kp, vp, bt = synth.make_paged_kv(lay, seed=0, device=DEV)
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, 1, 64)
    o, lse = bm.forward(q, kp, vp, desc, t, block_table=bt)
    torch.cuda.synchronize()
    H, D = lay.num_heads, lay.head_dim
    O = np.zeros((lay.n_seqs, H, D), np.float64)
    L = np.zeros((H, lay.n_seqs), np.float64)
    for s, ctx in enumerate(lay.seqlens_k):
        n = -(-ctx // 16)
        pages = bt[s, :n].long()
        kh_all, vh_all = kp[pages].cpu(), vp[pages].cpu()  # [n, 16, H, D]
        sub = synth.Layout("one", "causal", "bf16", H, D, [1], [int(ctx)], paged=True, page_size=16)
        bt_sub = np.arange(n, dtype=np.int32)[None, :]
        for h in range(H):
            O[s, h], L[h, s] = (x[0] for x in oforward.sequence_head(
                sub, 0, oforward.to_f64(q[s:s + 1, h]), oforward.to_f64(kh_all[:, :, h]),
                oforward.to_f64(vh_all[:, :, h]), block_table=bt_sub))
    mx, mean = _hip.check_close(o, lse, O, L, "bf16", "paged_decode")
    say(f"paged_decode every sequence and head: max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_bit_reproducible_run_to_run():
    lay = synth.shared_prefix(prefix=1024, n_suffix=4, suffix=512, H=4)
    q, k, v = (x.to(DEV) for x in synth.make_dense_qkv(lay, seed=3, device="cpu"))
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, 128, 64)
    say("reproducibility x3")
    o1, l1 = bm.forward(q, k, v, desc, t)
    o2, l2 = bm.forward(q, k, v, desc, t)
    t2 = bm.build_block_mask(desc, 128, 64)
    o3, l3 = bm.forward(q, k, v, desc, t2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("BM", [128, 1])
def test_packing_invariance_bit_exact(BM):
    # Each packed document's output is bit-identical to the document run alone.
    lay = synth.packed_documents(seed=2, n_docs=4, lo=30, hi=700, H=4)
    if BM == 1:
        lay = synth.Layout("decode", "causal", "bf16", 4, 128, [1] * 4, lay.seqlens_k)
    q, k, v = synth.make_dense_qkv(lay, seed=2, device="cpu")
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, BM, 64)
    say(f"packing invariance BM={BM} lens={lay.seqlens_k}")
    o, l = bm.forward(q.to(DEV), k.to(DEV), v.to(DEV), desc, t)
    cq, ck = lay.cu_q, lay.cu_k
    for s in range(lay.n_seqs):
        one = synth.Layout("one", "causal", "bf16", 4, 128, [lay.seqlens_q[s]], [lay.seqlens_k[s]])
        d1 = _hip.desc_for(one)
        t1 = bm.build_block_mask(d1, BM, 64)
        o1, l1 = bm.forward(q[cq[s]:cq[s + 1]].to(DEV), k[ck[s]:ck[s + 1]].to(DEV),
                            v[ck[s]:ck[s + 1]].to(DEV), d1, t1)
        assert torch.equal(o[cq[s]:cq[s + 1]], o1), s
        assert torch.equal(l[:, cq[s]:cq[s + 1]], l1), s


@pytest.mark.parametrize("kind", ["causal", "strip_thinking"])
def test_paged_equals_contiguous_bit_exact(kind):
    rng = np.random.default_rng(77)
    lay = synth.random_layout(rng, kind, n_seqs=3, max_len=400, min_len=100, H=2, D=128,
                              dtype="bf16", paged=True, page_size=16)
    q, kp, vp, bt = synth.make_paged_kv(lay, seed=9, device="cpu", extra_pages=4)
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, 128, 64)
    say(f"paged == contiguous kind={kind}")
    op, lp = bm.forward(q.to(DEV), kp.to(DEV), vp.to(DEV), desc, t, block_table=bt.to(DEV))
    kc = bm.paged_gather(kp.to(DEV), bt.to(DEV), desc)
    vc = bm.paged_gather(vp.to(DEV), bt.to(DEV), desc)
    oc, lc = bm.forward(q.to(DEV), kc, vc, desc, t)
    torch.cuda.synchronize()
    assert torch.equal(op, oc) and torch.equal(lp, lc)


@pytest.mark.parametrize("BM", [128, 1])
def test_unreachable_kv_never_read(BM):
    # NaN in pool pages no sequence uses, in page slots past each context and
    # in rows past the packed K/V: the outputs are bit-identical to a clean run.
    lay = synth.paged_decode(seed=4, n_seqs=5, lo=40, hi=700, page_size=16, H=2, D=128)
    if BM == 128:
        lay = synth.Layout("prefill", "causal", "bf16", 2, 128, lay.seqlens_k, lay.seqlens_k,
                           paged=True, page_size=16)
    q, kp, vp, bt = synth.make_paged_kv(lay, seed=4, device="cpu", extra_pages=6)
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, BM, 64)
    say(f"NaN poisoning BM={BM}")
    clean = bm.forward(q.to(DEV), kp.to(DEV), vp.to(DEV), desc, t, block_table=bt.to(DEV))
    kpn, vpn = kp.clone(), vp.clone()
    used = set()
    for s, c in enumerate(lay.seqlens_k):
        n = -(-c // 16)
        used.update(bt[s, :n].tolist())
        last = int(bt[s, n - 1])
        tail = c - (n - 1) * 16
        kpn[last, tail:] = float("nan")
        vpn[last, tail:] = float("nan")
    for pg in range(kp.shape[0]):
        if pg not in used:
            kpn[pg] = float("nan")
            vpn[pg] = float("nan")
    dirty = bm.forward(q.to(DEV), kpn.to(DEV), vpn.to(DEV), desc, t, block_table=bt.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(clean[0], dirty[0]) and torch.equal(clean[1], dirty[1])
    # Contiguous K/V with NaN rows past the last key.
    kc = bm.paged_gather(kp.to(DEV), bt.to(DEV), desc)
    vc = bm.paged_gather(vp.to(DEV), bt.to(DEV), desc)
    T = kc.shape[0]
    kbig = torch.full((T + 200, 2, 128), float("nan"), dtype=kc.dtype, device=DEV)
    vbig = kbig.clone()
    kbig[:T] = kc
    vbig[:T] = vc
    a = bm.forward(q.to(DEV), kc, vc, desc, t)
    b = bm.forward(q.to(DEV), kbig[:T], vbig[:T], desc, t)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.isfinite(a[0].float()).all()


def test_strided_views_and_explicit_scale():
    # Q/K/V as head-strided views of one fused buffer; O into a strided view.
    lay = synth.causal_single(L=300, H=3, D=128, dtype="bf16")
    fused = synth.make_dense_qkv(synth.causal_single(L=300, H=9, D=128, dtype="bf16"), seed=1)[0]
    q, k, v = fused[:, 0:3], fused[:, 3:6], fused[:, 6:9]
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, 128, 64)
    out_buf = torch.zeros(300, 6, 128, dtype=torch.bfloat16, device=DEV)
    say("strided views")
    fd = fused.to(DEV)
    o, lse = bm.forward(fd[:, 0:3], fd[:, 3:6], fd[:, 6:9], desc, t, out=out_buf[:, 1:4], scale=0.05)
    torch.cuda.synchronize()
    O, L = oforward.forward(lay, q, k, v, scale=0.05)
    _hip.check_close(out_buf[:, 1:4], lse, O, L, "bf16", "strided")
    assert torch.count_nonzero(out_buf[:, 0]) == 0 and torch.count_nonzero(out_buf[:, 4:]) == 0


def test_binding_rejects_mismatched_tensors_before_launch():
    # An int64 block table, K/V with fewer heads than Q, and an output too
    # small for total_q raise BmattnError in the binding; nothing is launched,
    # so the preset output stays untouched.
    lay = synth.random_layout(np.random.default_rng(3), "causal", n_seqs=2, max_len=200, min_len=70,
                              H=2, D=128, dtype="bf16", paged=True, page_size=16)
    q, kp, vp, bt = synth.make_paged_kv(lay, seed=1, device=DEV)
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, 128, 64)
    out = torch.full_like(q, 7.0)
    say("binding checks: int64 block table")
    with pytest.raises(bm.BmattnError):
        bm.forward(q, kp, vp, desc, t, block_table=bt.long(), out=out)
    say("binding checks: fewer K/V heads")
    with pytest.raises(bm.BmattnError):
        bm.forward(q, kp[:, :, :1], vp[:, :, :1], desc, t, block_table=bt, out=out)
    say("binding checks: short output")
    with pytest.raises(bm.BmattnError):
        bm.forward(q, kp, vp, desc, t, block_table=bt, out=out[:10])
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
