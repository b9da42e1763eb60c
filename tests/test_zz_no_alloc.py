"""GPU test of bmattn_forward_noalloc, the forward that allocates nothing:
its decode split workspace is the library's static device scratch.  Two
calls in a row (the second with a smaller input) give the same bits as
bmattn_forward with a caller workspace (same kernels, same splits), and the
prefill path (no workspace) does too.  Named to run last: it shares the
scratch with nothing else, and a failure here hides no other test."""

import numpy as np
import pytest
import torch

import synth
from block_sparse_masked_amd import bmattn as bm
from oracle import forward as oforward

import _hip
from _hip import DEV, say

pytestmark = pytest.mark.gpu


def _decode_case(seed, n_seqs, lo, hi, H):
    lay = synth.paged_decode(seed=seed, n_seqs=n_seqs, lo=lo, hi=hi, page_size=16, H=H, D=128)
    q, kp, vp, bt = synth.make_paged_kv(lay, seed=seed, device=DEV, extra_pages=3)
    desc = _hip.desc_for(lay)
    t = bm.build_block_mask(desc, 1, 64)
    return lay, q, kp, vp, bt, desc, t


def test_noalloc_decode_two_calls_match_forward():
    # Larger first, then smaller: the second call reuses (and overwrites part
    # of) what the first left in the scratch.
    for seed, n_seqs, lo, hi, H in ((1, 24, 3000, 20000, 8), (2, 5, 20, 2000, 4)):
        lay, q, kp, vp, bt, desc, t = _decode_case(seed, n_seqs, lo, hi, H)
        need = bm.forward_workspace_size(q, kp, vp, desc, t, block_table=bt)
        say(f"noalloc decode seed={seed} seqs={n_seqs} H={H} workspace {need} bytes")
        assert 0 < need <= bm.NOALLOC_MAX_WORKSPACE
        o1, l1 = bm.forward_noalloc(q, kp, vp, desc, t, block_table=bt)
        o2, l2 = bm.forward(q, kp, vp, desc, t, block_table=bt)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        if seed == 2:  # and against the oracle
            O, L = oforward.forward(lay, q.cpu(), k_pool=kp.cpu(), v_pool=vp.cpu(), block_table=bt.cpu())
            _hip.check_close(o1, l1, O, L, "bf16", "noalloc decode")


def test_noalloc_prefill_matches_forward():
    for L_ in (700, 300):
        lay = synth.shared_prefix(prefix=L_ // 2, n_suffix=2, suffix=L_ // 4, H=2)
        q, k, v = (x.to(DEV) for x in synth.make_dense_qkv(lay, seed=5, device="cpu"))
        desc = _hip.desc_for(lay)
        t = bm.build_block_mask(desc, 128, 64)
        say(f"noalloc prefill tokens={lay.total_q}")
        o1, l1 = bm.forward_noalloc(q, k, v, desc, t)
        o2, l2 = bm.forward(q, k, v, desc, t)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
