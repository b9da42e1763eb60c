"""Gradients of masked attention (oracle; test infrastructure only).

The forward map of one (sequence, head) is O = P V with P the row softmax of
S, S_ij = scale * (q_i . k_j) on visible pairs and -inf elsewhere (Triton
from First Principles, Ch. 21, sections 21.1 and 21.2; the masks of
``masks``).  The pages print no backward formulas; the gradients here are
the derivative of that forward map for an upstream gradient dO, written out
by the chain rule (this project's reading):

  dV = P^T dO
  dP = dO V^T
  dS_ij = P_ij * (dP_ij - sum_l P_il dP_il)     (Jacobian of the row softmax)
  dQ = scale * dS K
  dK = scale * dS^T Q

A row with no visible key has P = 0 and contributes nothing.  The
xorl issue ("Block-mask attention: express shared-prefix and
strip-thinking multi-turn training that cu_seqlens cannot", section
"Correctness") compares dq, dk and dv of its routes against a dense float32
reference; this float64 version plays that role here.
"""

from __future__ import annotations

import numpy as np

from .attention import default_scale
from .forward import head_slice
from .masks import visible_for_layout


def probabilities(q, k, vis, scale):
    """P [Lq, Lk] (float64): the row softmax of the scaled, masked scores."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    vis = np.asarray(vis, bool)
    s = np.where(vis, (q @ k.T) * scale, -np.inf)
    has = vis.any(axis=1)
    m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)


def sequence_backward(q, k, v, vis, scale, do):
    """(dQ [Lq, D], dK [Lk, D], dV [Lk, Dv]) of one (sequence, head)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    p = probabilities(q, k, vis, scale)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def backward(layout, q, k, v, do, *, scale=None, heads=None):
    """dQ [total_q, H, D], dK and dV [total_k, H, D] (float64) for every
    sequence of a contiguous layout; ``heads`` restricts the heads computed
    (the others stay 0)."""
    assert not layout.paged, "the backward takes contiguous K and V"
    scale = default_scale(layout.head_dim) if not scale else scale
    H, D = layout.num_heads, layout.head_dim
    dQ = np.zeros((layout.total_q, H, D), np.float64)
    dK = np.zeros((layout.total_k, H, D), np.float64)
    dV = np.zeros((layout.total_k, H, D), np.float64)
    cq, ck = layout.cu_q, layout.cu_k
    for h in (range(H) if heads is None else heads):
        qh, kh, vh, doh = (head_slice(x, h) for x in (q, k, v, do))
        for s in range(layout.n_seqs):
            qs, qe, ks, ke = cq[s], cq[s + 1], ck[s], ck[s + 1]
            vis = visible_for_layout(layout, s)
            dq, dk, dv = sequence_backward(qh[qs:qe], kh[ks:ke], vh[ks:ke], vis, scale, doh[qs:qe])
            dQ[qs:qe, h], dK[ks:ke, h], dV[ks:ke, h] = dq, dk, dv
    return dQ, dK, dV
