"""Calls on different streams share no state: two layouts' block-mask
builds, forwards and backwards launched concurrently on two streams give
the same bits as the same calls made one after the other."""

import numpy as np
import pytest
import torch

import synth
from _hip import DEV, desc_for, say
from block_sparse_masked_amd import bmattn as bm

pytestmark = pytest.mark.gpu


def _case(kind, seed):
    rng = np.random.default_rng(seed)
    lay = synth.random_layout(rng, kind, n_seqs=3, max_len=600, min_len=100, H=4, D=128, dtype="bf16")
    q, k, v = synth.make_dense_qkv(lay, seed=seed, device=DEV)
    do = synth.make_dense_qkv(lay, seed=seed + 1, device=DEV)[0]
    desc = desc_for(lay)
    return lay, q, k, v, do, desc


def _run(case):
    lay, q, k, v, do, desc = case
    rows = bm.build_block_mask(desc, *bm.BWD_ROWS)
    o, lse = bm.forward(q, k, v, desc, rows)
    _, cols = bm.build_backward_cols(desc)
    dq, dk, dv = bm.backward(q, k, v, o, lse, do, desc, rows, cols)
    return o, lse, dq, dk, dv


def test_two_streams_match_sequential():
    cases = [_case("shared_prefix", 41), _case("composed", 43)]
    seq = [_run(c) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    par = [None, None]
    for rep in range(3):
        for i, (c, s) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(s):
                par[i] = _run(c)
        torch.cuda.synchronize()
        for i in range(2):
            for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), par[i], seq[i]):
                assert torch.equal(a, b), f"rep {rep} case {i}: {name} differs from the sequential run"
    say(f"two streams x3: {[c[0].total_q for c in cases]} tokens, bit-identical")
