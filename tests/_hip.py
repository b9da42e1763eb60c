"""Helpers for the GPU tests: layouts -> device descriptions, oracle
expectations in the HIP library's array shapes, and the tolerance check."""

import sys

import numpy as np
import torch

import synth
from block_sparse_masked_amd import bmattn as bm
from oracle import masks as omasks
from oracle import tiles as otiles
from oracle import forward as oforward

DEV = "cuda"

# Tolerances against the float64 oracle (max-abs, mean-abs).
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def desc_for(layout, device=DEV) -> bm.MaskDesc:
    return bm.MaskDesc.create(layout.kind, layout.cu_q, layout.cu_k, max(layout.max_q, 1),
                              max(layout.max_k, 1), device=device, seg_q=layout.seg_q,
                              seg_k=layout.seg_k, role_q=layout.role_q, role_k=layout.role_k,
                              turn_q=layout.turn_q, turn_k=layout.turn_k,
                              think_role=layout.think_role, loss_role=layout.loss_role,
                              history_role=layout.history_role, doc_q=layout.doc_q,
                              doc_k=layout.doc_k, terms=layout.terms)


def oracle_tiles(layout, BM, BN):
    """Oracle classes and lists in the library's layout, plus the schedule:
    rows by descending listed-tile count, ties by ascending row."""
    cls, fc, pc, fi, pi = otiles.layout_tiles(layout, BM, BN)
    work = fc + pc
    order = np.array(sorted(range(len(work)), key=lambda r: (-int(work[r]), r)), np.int32)
    return cls, fc, pc, fi, pi, order


def check_tiles(layout, desc, BM, BN):
    t = bm.build_block_mask(desc, BM, BN)
    torch.cuda.synchronize()
    cls, fc, pc, fi, pi, order = oracle_tiles(layout, BM, BN)
    rows, n_kt = cls.shape
    assert (t.n_qt * layout.n_seqs, t.n_kt) == (rows, n_kt)
    g = lambda x: x.cpu().numpy()
    assert np.array_equal(g(t.tile_class).reshape(rows, n_kt), cls), "tile classes"
    assert np.array_equal(g(t.full_cnt), fc), "full counts"
    assert np.array_equal(g(t.part_cnt), pc), "partial counts"
    assert np.array_equal(g(t.full_idx).reshape(rows, n_kt), fi), "full lists"
    assert np.array_equal(g(t.part_idx).reshape(rows, n_kt), pi), "partial lists"
    assert np.array_equal(g(t.row_order), order), "row schedule"
    return t


def check_dense(layout, desc, t):
    for s in range(layout.n_seqs):
        got = bm.debug_dense_mask(desc, t, s).cpu().numpy()
        Lq, Lk = layout.seqlens_q[s], layout.seqlens_k[s]
        want = np.zeros_like(got)
        want[:Lq, :Lk] = omasks.visible_for_layout(layout, s)
        assert np.array_equal(got, want), f"dense mask of sequence {s}"


def to_dev(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def check_close(o, lse, O_ref, LSE_ref, dtype, what=""):
    """O [T, H, D] (device) against the float64 oracle; LSE [H, T]."""
    mx_tol, mean_tol = TOL[dtype]
    o = o.detach().float().cpu().numpy().astype(np.float64)
    err = np.abs(o - O_ref)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert err.max() <= mx_tol, f"{what}: O max-abs {err.max():.3e} > {mx_tol}"
    assert err.mean() <= mean_tol, f"{what}: O mean-abs {err.mean():.3e} > {mean_tol}"
    if lse is not None:
        l = lse.detach().cpu().numpy().astype(np.float64)
        fin = np.isfinite(LSE_ref)
        assert np.array_equal(fin, np.isfinite(l)), f"{what}: LSE -inf pattern"
        if fin.any():
            le = np.abs(l[fin] - LSE_ref[fin])
            assert le.max() <= mx_tol, f"{what}: LSE max-abs {le.max():.3e}"
            assert le.mean() <= mean_tol, f"{what}: LSE mean-abs {le.mean():.3e}"
    return float(err.max()), float(err.mean())


def run_dense(layout, seed=0, BM=128, BN=64, scale=0.0):
    """Contiguous K/V forward through the library; returns (o, lse, q, k, v, desc, tiles)."""
    q, k, v = synth.make_dense_qkv(layout, seed=seed, device="cpu")
    qd, kd, vd = to_dev(q, k, v)
    desc = desc_for(layout)
    t = bm.build_block_mask(desc, BM, BN)
    o, lse = bm.forward(qd, kd, vd, desc, t, scale=scale)
    torch.cuda.synchronize()
    return o, lse, q, k, v, desc, t


def oracle_dense(layout, q, k, v, scale=None):
    return oforward.forward(layout, q, k, v, scale=scale)


def oracle_workers() -> int:
    """Host threads for the oracle: the cores this process may use, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_one_sequence(layout, q, k, v, heads=None, scale=None):
    """O [T, H, D] and LSE [H, T] (float64) of a one-sequence contiguous layout,
    every head (or ``heads``): the oracle's dense mask, built once, and its
    three passes per head, the heads spread over host threads with BLAS
    single-threaded in each (numpy releases the interpreter lock in BLAS and
    in its array loops)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import attention as oattention

    assert layout.n_seqs == 1 and not layout.paged
    H, T = layout.num_heads, layout.total_q
    heads = list(range(H)) if heads is None else list(heads)
    sc = oattention.default_scale(layout.head_dim) if not scale else scale
    vis = omasks.visible_for_layout(layout, 0)
    O = np.zeros((T, H, layout.head_dim), np.float64)
    L = np.full((H, T), -np.inf, np.float64)

    def one(h):
        O[:, h], L[h] = oattention.three_pass(oforward.head_slice(q, h), oforward.head_slice(k, h),
                                              oforward.head_slice(v, h), vis, sc)

    with threadpool_limits(1), ThreadPoolExecutor(oracle_workers()) as ex:
        list(ex.map(one, heads))
    return O, L


def oracle_backward_one_sequence(layout, q, k, v, do, heads, workers=2):
    """(dQ, dK, dV) [T, len(heads), D] float64 of a one-sequence contiguous
    layout for the listed heads: the oracle's dense mask, built once, and
    its per-sequence backward per head, ``workers`` heads at a time (each
    holds several T x T float64 matrices) with the BLAS threads shared out."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import attention as oattention
    from oracle import backward as obackward

    assert layout.n_seqs == 1 and not layout.paged
    heads = list(heads)
    sc = oattention.default_scale(layout.head_dim)
    vis = omasks.visible_for_layout(layout, 0)
    T, D = layout.total_q, layout.head_dim
    out = [np.zeros((T, len(heads), D), np.float64) for _ in range(3)]

    def one(i):
        h = heads[i]
        g = obackward.sequence_backward(*(oforward.head_slice(x, h) for x in (q, k, v)), vis, sc,
                                        oforward.head_slice(do, h))
        for a, b in zip(out, g):
            a[:, i] = b

    with threadpool_limits(max(1, oracle_workers() // workers)), ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(len(heads))))
    return out
