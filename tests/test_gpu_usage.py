"""The usage example of the README, run as written: it must execute, and its
O for one (document, head) must match the float64 oracle."""

import os
import re

import numpy as np
import pytest
import torch

from oracle import forward as oforward
from synth.workloads import Layout

from _hip import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def readme_example() -> str:
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "the README holds one Python example"
    return blocks[0]


def test_readme_example_runs_and_matches_oracle():
    env = {}
    exec(compile(readme_example(), "README.md", "exec"), env)
    torch.cuda.synchronize()
    o, lse, lens = env["o"], env["lse"], env["lens"]
    for name in ("dq", "dk", "dv"):
        g = env[name]
        assert g.shape == env[name[1]].shape and torch.isfinite(g.float()).all(), name
    # the last document, head 3, against the oracle
    s, h = len(lens) - 1, 3
    q0 = sum(lens[:s])
    sl = slice(q0, q0 + lens[s])
    qh, kh, vh = (oforward.head_slice(env[x][sl].cpu(), h) for x in ("q", "k", "v"))
    sub = Layout("readme_doc", "causal", "bf16", o.shape[1], o.shape[2], [lens[s]], [lens[s]])
    O, L = oforward.sequence_head(sub, 0, qh, kh, vh)
    got = o[sl, h].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - O)
    say(f"README example: doc {s} head {h}: max {err.max():.2e} mean {err.mean():.2e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    lerr = np.abs(lse[h, sl].cpu().numpy().astype(np.float64) - L)
    assert lerr.max() <= 2e-2
