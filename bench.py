"""Benchmark of the block-sparse masked attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: bmattn_build_block_mask (tile classes, kv-tile lists,
schedule) followed by bmattn_forward (O and LSE).  The metric counts only the
unmasked score elements: 4 * head_dim flops per visible (query, key) pair per
head (2*D for Q K^T, 2*D for P V).  Prints one JSON line.

The default workload is the largest single-GPU configuration, the shared
prefix: one sequence of a 4096-token prefix (segment 0) and 16 suffixes of
1024 tokens (segments 1..16), 32 heads, head_dim 128, bf16.  Other named
workloads: causal_f32, packed_documents (8 causal documents with lengths
uniform in [64, 2048], 16 heads), strip_thinking, paged_decode,
strip_thinking_duplicated (whose step starts with the relabelling of its ids,
bmattn_duplicated_answer_ids), shared_prefix_groups (a composed mask: four
shared-prefix groups and padding in one sequence).

roofline.achieved divides the algorithmic work of one forward by the forward
kernel's average duration: G forward calls captured in one HIP graph and
replayed between two HIP events on the stream the kernels run on, so the
average holds kernel time and the few microseconds between graph nodes, not
host launch work.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "masked-attention TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SOURCES = {"prefill": "block_sparse_masked_amd/csrc/forward_prefill_bf16.hip",
                  "decode": "block_sparse_masked_amd/csrc/forward_decode.hip",
                  "backward": "block_sparse_masked_amd/csrc/backward_bf16.hip"}


def visible_pairs(lay) -> int:
    """Visible (query, key) pairs per head, in closed form for each workload."""
    if lay.name == "shared_prefix":
        P, n, S = lay.notes["prefix"], lay.notes["n_suffix"], lay.notes["suffix"]
        return P * (P + 1) // 2 + n * (S * P + S * (S + 1) // 2)
    if lay.name == "strip_thinking":
        u, th, a, n = (lay.notes[k] for k in ("user", "think", "answer", "n_turns"))
        T = u + th + a
        tot = 0
        for t in range(n):
            b = t * T
            # a query at position p of turn t sees p + 1 keys minus t think spans
            tot += (T * (2 * b + T + 1)) // 2 - T * t * th
        return tot
    if lay.name == "shared_prefix_groups":
        g, P, n, S = (lay.notes[k] for k in ("n_groups", "prefix", "n_suffix", "suffix"))
        return g * (P * (P + 1) // 2 + n * (S * P + S * (S + 1) // 2))  # padding sees nothing
    if lay.name == "strip_thinking_duplicated":
        u, th, a, n = (lay.notes[k] for k in ("user", "think", "answer", "n_turns"))
        tot = 0
        for t in range(n):
            hist = t * (u + a)  # earlier turns: user text and history copies
            n1 = u + th + a     # user, think, loss copy: the turn as generated
            tot += n1 * hist + n1 * (n1 + 1) // 2
            # history copy: earlier turns, its own user text, itself causally
            tot += a * (hist + u) + a * (a + 1) // 2
        return tot
    if lay.name == "prefix_lm":
        # the prefix rows see the whole prefix, every later row keys 0 .. itself
        return sum(min(P, L) ** 2 + (L * (L + 1) - min(P, L) * (min(P, L) + 1)) // 2
                   for P, L in zip(lay.notes["prefixes"], lay.seqlens_q))
    if lay.kind == "full":
        return sum(q * k for q, k in zip(lay.seqlens_q, lay.seqlens_k))
    if lay.kind == "causal":
        import numpy as np
        tot = 0
        for lq, lk in zip(lay.seqlens_q, lay.seqlens_k):
            # query row i sits at position lk - lq + i and sees keys 0 .. that position
            i = np.arange(lq, dtype=np.int64)
            tot += int(np.clip(lk - lq + i + 1, 0, lk).sum())
        return tot
    raise ValueError(lay.name)


def src_hash(path: str) -> str:
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        recs = json.load(f)
    for r in recs:
        if r.get("kernel") == kernel and r.get("workload") == workload:
            if r.get("src_sha256") != src_hash(KERNEL_SOURCES[kernel]):
                return None
            return r.get("hbm_bytes_per_launch")
    return None


def cpu_baseline(lay, q, k, v, kp, vp, bt, flops_total: float, budget_s: float = 10.0):
    """The oracle as it stands, timed on the host cores on a bounded sample."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import forward as oforward

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    if lay.paged:
        # One context per pass, heads 0..3: the oracle gathers and attends.
        import torch
        seqs = list(range(lay.n_seqs))
        done_pairs, passes, t0 = 0, 0, time.perf_counter()
        for s in seqs:
            n = -(-lay.seqlens_k[s] // lay.page_size)
            pages = bt[s, :n].long()
            sub = type(lay)("one", "causal", lay.dtype, lay.num_heads, lay.head_dim, [1],
                            [lay.seqlens_k[s]], paged=True, page_size=lay.page_size)
            btab = np.arange(n, dtype=np.int32)[None, :]
            for h in range(4):
                oforward.sequence_head(sub, 0, oforward.to_f64(q[s:s + 1, h]),
                                       oforward.to_f64(kp[pages, :, h]), oforward.to_f64(vp[pages, :, h]),
                                       block_table=btab)
                done_pairs += lay.seqlens_k[s]
            passes += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        fl = 4.0 * lay.head_dim * done_pairs
        return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"{passes} of {lay.n_seqs} sequences x heads 0-3 (float64 numpy), {dt:.1f} s"}
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    passes, t0 = 0, time.perf_counter()
    if lay.name in ("shared_prefix", "strip_thinking", "strip_thinking_duplicated",
                    "shared_prefix_groups"):
        # One head per pass of the single long sequence.
        import dataclasses
        one_head = dataclasses.replace(lay, num_heads=1)
        for h in range(lay.num_heads):
            oforward.forward(one_head, qc[:, h:h + 1], kc[:, h:h + 1], vc[:, h:h + 1])
            passes += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        fl = flops_total * passes / lay.num_heads
        return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"{passes} of {lay.num_heads} heads (float64 numpy), {dt:.1f} s"}
    while True:
        oforward.forward(lay, qc, kc, vc)
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops_total * passes / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole workload x{passes} (float64 numpy), {dt:.1f} s"}


def cpu_baseline_backward(lay, q, k, v, do, flops_per_head: float, budget_s: float = 10.0):
    """The oracle backward on the host cores, one head per pass (bounded)."""
    from threadpoolctl import threadpool_info
    from oracle import backward as obackward

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    qc, kc, vc, dc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    passes, t0 = 0, time.perf_counter()
    for h in range(lay.num_heads):
        obackward.backward(lay, qc, kc, vc, dc, heads=[h])
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops_per_head * passes / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{passes} of {lay.num_heads} heads (float64 numpy), {dt:.1f} s"}


def bench_backward(args, lay, q, k, v, desc, tiles, torch, bm):
    """The backward of the workload: flops = 10 * head_dim per visible pair
    per head (S recomputed, dP, dV, dQ, dK: five products of 2 * head_dim,
    the usual count of 2.5 forwards), inputs and the forward's O / LSE
    resident in HBM."""
    import synth
    if lay.paged or lay.dtype != "bf16":
        print("[bench] the backward is compiled for bf16 with contiguous K/V", file=sys.stderr)
        sys.exit(2)
    H, D = lay.num_heads, lay.head_dim
    do = synth.make_dense_qkv(lay, seed=args.seed + 1000, device="cuda")[0]
    o, lse = bm.forward(q, k, v, desc, tiles)
    ctiles, cols = bm.build_backward_cols(desc)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(bm.backward_workspace_size(q, desc), 16), dtype=torch.uint8, device="cuda")

    def step():
        bm.build_backward_cols(desc, tiles=ctiles, out=cols)
        bm.backward(q, k, v, o, lse, do, desc, tiles, cols, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph_steps = 1
    if args.launch == "graph":
        graph_steps = max(d for d in range(1, 21) if args.steps % d == 0)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(graph_steps):
                step()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps // graph_steps):
            graph.replay()
    else:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The backward call alone (prep, dK/dV and dQ kernels), HIP events on its stream.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        bm.backward(q, k, v, o, lse, do, desc, tiles, cols, dq=dq, dk=dk, dv=dv, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    bwd_ms = [a.elapsed_time(b) for a, b in evs]
    bwd_call = sum(bwd_ms) / len(bwd_ms)
    bwd_avg = kernel_ms(torch, lambda: bm.backward(q, k, v, o, lse, do, desc, tiles, cols, dq=dq,
                                                   dk=dk, dv=dv, workspace=ws),
                        max(graph_steps, 10), args.steps)
    fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in fe:
        a.record()
        bm.forward(q, k, v, desc, tiles, out=o, lse=lse)
        b.record()
    torch.cuda.synchronize()
    fwd_avg = sum(a.elapsed_time(b) for a, b in fe) / len(fe)

    pairs = visible_pairs(lay)
    flops = 10.0 * D * H * pairs
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (bwd_avg * 1e-3) / 1e12
    res = {
        "metric": "masked-attention backward TFLOP/s (unmasked FLOPs, 10*D per visible pair) "
                  "+ % bf16 MFMA peak, 1 GPU",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": lay.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "pass": "backward", "seed": args.seed,
                   "num_heads": H, "head_dim": D, "total_q": lay.total_q, "total_k": lay.total_k,
                   "rows_tiles": list(bm.BWD_ROWS), "cols_tiles": list(bm.BWD_COLS),
                   "launch": args.launch, "graph_steps": graph_steps, "visible_pairs_per_head": pairs,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_from_profile("backward", args.workload)},
        "detail": {"backward_kernels_ms": bwd_avg, "backward_call_ms": bwd_call,
                   "backward_call_ms_min": min(bwd_ms),
                   "forward_call_ms": fwd_avg, "fwd_plus_bwd_ms": fwd_avg + bwd_avg},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle backward on the host cores", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_backward(lay, q, k, v, do, flops / H, args.cpu_budget)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def kernel_ms(torch, call, per_graph: int, steps: int) -> float:
    """Average duration of ``call`` (its kernels): G back-to-back calls
    captured as one HIP graph, replayed between HIP events recorded on the
    stream the graph runs on."""
    per_graph = max(1, per_graph)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(per_graph):
                call()
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    a.record(stream)
    for _ in range(reps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * per_graph)


def copy_calibration(mib: int, steps: int):
    """A plain streaming kernel of known size: dst = src * 1 over fp32."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / max(steps, 1)
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                      "ms_per_copy": dt * 1e3, "steps": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="shared_prefix")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="replay each step as a captured HIP graph (default) or launch it eagerly")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward instead: a step is the column-list build of the "
                         "backward's 64x128 block mask plus bmattn_backward (dQ, dK, dV)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the workload, run a plain fp32 copy of MIB MiB (read once, "
                         "written once) --steps times: the known-size kernel against which the "
                         "HBM byte counters are scaled")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    import synth
    from block_sparse_masked_amd import bmattn as bm

    dev = "cuda"
    lay = synth.config(args.workload, seed=args.seed)
    H, D = lay.num_heads, lay.head_dim
    print(f"[bench] workload {args.workload}: seqs {lay.n_seqs}, tokens q {lay.total_q} "
          f"k {lay.total_k}, H {H}, D {D}, {lay.dtype}", file=sys.stderr, flush=True)
    kp = vp = bt = None
    if lay.paged:
        q, kp, vp, bt = synth.make_paged_kv(lay, seed=args.seed, device=dev)
        k, v = kp, vp
    else:
        q, k, v = synth.make_dense_qkv(lay, seed=args.seed, device=dev)
    desc = bm.MaskDesc.create(lay.kind, lay.cu_q, lay.cu_k, lay.max_q, lay.max_k, device=dev,
                              seg_q=lay.seg_q, seg_k=lay.seg_k, role_q=lay.role_q,
                              role_k=lay.role_k, turn_q=lay.turn_q, turn_k=lay.turn_k,
                              think_role=lay.think_role, loss_role=lay.loss_role,
                              history_role=lay.history_role, doc_q=lay.doc_q, doc_k=lay.doc_k,
                              terms=lay.terms)
    relabel = desc.duplicated_from is not None
    if relabel:
        flags = bm.relabel(desc, check=True)
        if int(flags.item()) != 0:
            raise SystemExit(f"[bench] duplicated-answer layout check failed: {int(flags.item())}")
    BM, BN = (1, 64) if lay.max_q == 1 else (128, 64)
    tiles = bm.build_block_mask(desc, BM, BN)
    if args.backward:
        bench_backward(args, lay, q, k, v, desc, tiles, torch, bm)
        return
    out = torch.empty_like(q)
    lse = torch.empty((H, lay.total_q), dtype=torch.float32, device=dev)
    ws_bytes = bm.forward_workspace_size(q, k, v, desc, tiles, block_table=bt)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None

    def step(ev=None):
        if relabel:
            bm.relabel(desc)
        bm.build_block_mask(desc, BM, BN, out=tiles)
        if ev is not None:
            ev[0].record()
        bm.forward(q, k, v, desc, tiles, block_table=bt, out=out, lse=lse, workspace=ws)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    graph_steps = 1
    if args.launch == "graph":
        # G consecutive steps (mask build + forward each) captured as one HIP
        # graph on a side stream and replayed K / G times: the same kernels
        # with the same arguments, without per-launch host work, and one
        # graph launch per G steps.  G is the largest divisor of K up to 20,
        # so exactly K steps are timed.
        graph_steps = max(d for d in range(1, 21) if args.steps % d == 0)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(graph_steps):
                step()
        for _ in range(max(1, args.warmup // graph_steps)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps // graph_steps):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # Each forward call alone, timed with events on its launch stream.
        for i in range(args.steps):
            evs[i][0].record()
            bm.forward(q, k, v, desc, tiles, block_table=bt, out=out, lse=lse, workspace=ws)
            evs[i][1].record()
        torch.cuda.synchronize()
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    fwd_ms = [a.elapsed_time(b) for a, b in evs]
    fwd_call_ms = sum(fwd_ms) / len(fwd_ms)
    fwd_avg_ms = kernel_ms(torch, lambda: bm.forward(q, k, v, desc, tiles, block_table=bt, out=out,
                                                     lse=lse, workspace=ws),
                           max(graph_steps, 10), args.steps)

    # mask build alone (cacheable across steps; reported separately), launched
    # the same way as the steps
    def builds(n):
        for _ in range(n):
            if relabel:
                bm.relabel(desc)
            bm.build_block_mask(desc, BM, BN, out=tiles)
    if args.launch == "graph":
        bgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(bgraph):
            builds(graph_steps)
        bgraph.replay()
        torch.cuda.synchronize()
        tb = time.perf_counter()
        for _ in range(args.steps // graph_steps):
            bgraph.replay()
    else:
        torch.cuda.synchronize()
        tb = time.perf_counter()
        builds(args.steps)
    torch.cuda.synchronize()
    build_ms = (time.perf_counter() - tb) * 1e3 / args.steps

    pairs = visible_pairs(lay)
    flops = 4.0 * D * H * pairs
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    el = 2 if lay.dtype == "bf16" else 4
    if lay.paged:
        kernel = "decode"
        algo_bytes = 2.0 * H * D * el * lay.total_k + 2.0 * H * D * el * lay.total_q
        achieved = algo_bytes / (fwd_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profile(kernel, args.workload)}
    else:
        kernel = "prefill"
        achieved = flops / (fwd_avg_ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if lay.dtype == "bf16" else PEAK_F32_TFLOPS
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": traffic_from_profile(kernel, args.workload)}

    res = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": lay.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "seed": args.seed, "num_heads": H, "head_dim": D,
                   "seqlens_q": lay.seqlens_q if lay.n_seqs <= 16 else f"{lay.n_seqs} seqs",
                   "total_q": lay.total_q, "total_k": lay.total_k, "block_m": BM, "block_n": BN,
                   "launch": args.launch, "graph_steps": graph_steps,
                   "visible_pairs_per_head": pairs, "flops_per_step": flops},
        "roofline": roof,
        "detail": {"forward_kernel_ms": fwd_avg_ms, "forward_call_ms": fwd_call_ms,
                   "forward_call_ms_min": min(fwd_ms), "mask_build_ms": build_ms,
                   "pct_bf16_peak_step": 100.0 * value / PEAK_BF16_TFLOPS},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host cores", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(lay, q, k, v, kp, vp, bt, flops, args.cpu_budget)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
