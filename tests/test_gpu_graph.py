"""HIP-graph capture of the hot path (block-mask build + forward), as the
benchmark replays it, and of the backward call with its block-mask builds:
every replay, with eager work between replays, must reproduce the eagerly
launched result bit for bit (the kernels are deterministic), and the eager
forward result must match the oracle."""

import numpy as np
import pytest
import torch

import synth
from _hip import DEV, check_close, desc_for, oracle_dense, say
from block_sparse_masked_amd import bmattn as bm


def _graph_case(lay, seed, BM, BN, paged):
    if paged:
        q, kp, vp, bt = synth.make_paged_kv(lay, seed=seed, device=DEV)
        k, v = kp, vp
    else:
        q, k, v = synth.make_dense_qkv(lay, seed=seed, device=DEV)
        bt = None
    desc = desc_for(lay)
    tiles = bm.build_block_mask(desc, BM, BN)
    out = torch.empty_like(q)
    lse = torch.empty((lay.num_heads, lay.total_q), dtype=torch.float32, device=DEV)
    nbytes = bm.forward_workspace_size(q, k, v, desc, tiles, block_table=bt)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV) if nbytes else None

    def step():
        bm.build_block_mask(desc, BM, BN, out=tiles)
        bm.forward(q, k, v, desc, tiles, block_table=bt, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l, ref_order = out.clone(), lse.clone(), tiles.row_order.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    return q, k, v, bt, desc, tiles, out, lse, ref_o, ref_l, ref_order, g


@pytest.mark.gpu
@pytest.mark.parametrize("name,paged", [("packed_documents", False), ("small_shared_prefix", False),
                                        ("small_decode", True)])
def test_graph_replay_matches_eager(name, paged):
    rng = np.random.default_rng(11)
    if name == "packed_documents":
        lay, BM = synth.config("packed_documents", seed=0), 128
    elif name == "small_shared_prefix":
        lay = synth.random_layout(rng, "shared_prefix", n_seqs=2, max_len=400, H=4, D=128, dtype="bf16")
        BM = 128
    else:
        lay = synth.random_layout(rng, "causal", n_seqs=5, max_len=900, H=4, D=128, dtype="bf16",
                                  decode_q=1, paged=True)
        BM = 1
    say(f"graph case {name}: seqs {lay.n_seqs} q {lay.total_q} k {lay.total_k}")
    (q, k, v, bt, desc, tiles, out, lse, ref_o, ref_l, ref_order, g) = _graph_case(lay, 3, BM, 64, paged)
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        tiles.row_order.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        # eager work between replays
        x = torch.randn(256, 256, device=DEV)
        (x @ x).sum().item()
        assert torch.equal(out, ref_o), f"replay {r}: O differs from the eager launch"
        assert torch.equal(lse, ref_l), f"replay {r}: LSE differs from the eager launch"
        assert torch.equal(tiles.row_order, ref_order), f"replay {r}: schedule differs"
    if not paged:
        exp_o, exp_l = oracle_dense(lay, q.cpu(), k.cpu(), v.cpu())
        check_close(ref_o, ref_l, exp_o, exp_l, lay.dtype, name)


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["causal", "shared_prefix", "composed"])
def test_backward_graph_replay_matches_eager(kind):
    """The backward call with both block-mask builds it needs (the 128 x 64
    rows and the 64 x 128 columns), captured as one graph: every replay,
    with eager work between replays, gives the eager gradients bit for bit
    (the backward has no atomics)."""
    rng = np.random.default_rng(23)
    lay = synth.random_layout(rng, kind, n_seqs=3, max_len=300, min_len=40, H=3, D=128, dtype="bf16")
    say(f"backward graph case {kind}: seqs {lay.n_seqs} q {lay.total_q}")
    q, k, v = synth.make_dense_qkv(lay, seed=5, device=DEV)
    do = synth.make_dense_qkv(lay, seed=6, device=DEV)[0]
    desc = desc_for(lay)
    rows = bm.build_block_mask(desc, *bm.BWD_ROWS)
    o, lse = bm.forward(q, k, v, desc, rows)
    ctiles, cols = bm.build_backward_cols(desc)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(bm.backward_workspace_size(q, desc), 16), dtype=torch.uint8, device=DEV)

    def step():
        bm.build_block_mask(desc, *bm.BWD_ROWS, out=rows)
        bm.build_backward_cols(desc, tiles=ctiles, out=cols)
        bm.backward(q, k, v, o, lse, do, desc, rows, cols, dq=dq, dk=dk, dv=dv, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for x in (dq, dk, dv):
            x.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        x = torch.randn(256, 256, device=DEV)
        (x @ x).sum().item()
        for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager launch"


@pytest.mark.gpu
def test_duplicated_answer_step_graph_replay_matches_eager():
    """The duplicated-answer step as the benchmark captures it (relabel the
    ids with the layout check, build the block mask, forward): every replay
    reproduces the eager O and LSE bit for bit and reports a valid layout."""
    rng = np.random.default_rng(29)
    lay = synth.random_layout(rng, "strip_thinking_duplicated", n_seqs=2, max_len=400, min_len=100,
                              H=2, D=128, dtype="bf16")
    say(f"duplicated graph case: seqs {lay.n_seqs} q {lay.total_q}")
    q, k, v = synth.make_dense_qkv(lay, seed=7, device=DEV)
    desc = desc_for(lay)
    tiles = bm.build_block_mask(desc, 128, 64)
    out = torch.empty_like(q)
    lse = torch.empty((lay.num_heads, lay.total_q), dtype=torch.float32, device=DEV)
    holder = {}

    def step():
        holder["flags"] = bm.relabel(desc, check=True)
        bm.build_block_mask(desc, 128, 64, out=tiles)
        bm.forward(q, k, v, desc, tiles, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    assert int(holder["flags"].item()) == 0, "the generated layout must meet the relabelling conditions"
    ref_o, ref_l = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    flags = holder["flags"]
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        flags.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        x = torch.randn(256, 256, device=DEV)
        (x @ x).sum().item()
        assert int(flags.item()) == 0, f"replay {r}: layout check"
        assert torch.equal(out, ref_o), f"replay {r}: O differs from the eager launch"
        assert torch.equal(lse, ref_l), f"replay {r}: LSE differs from the eager launch"
