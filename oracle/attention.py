"""Exact masked attention for one (sequence, head) (oracle; test infrastructure only).

``three_pass`` is the plain definition softmax(Q K^T * scale + M) V with
M = 0 on visible pairs and -inf elsewhere, in float64:

  pass 1: m_i = max over visible j of s_ij
  pass 2: l_i = sum over visible j of exp(s_ij - m_i)
  pass 3: o_i = sum over visible j of exp(s_ij - m_i) / l_i * v_j

with s_ij = (q_i . k_j) * scale and LSE_i = m_i + ln(l_i) (natural log).

Sources: Triton from First Principles, Ch. 21 "Flash Attention, MoE, and
Advanced Features": the attention definition and scale 1/sqrt(d) (section
21.1), the naive oracle that masks scores with -inf before the softmax
(section 21.2), and the three passes that the online form reduces to two
(the prerequisites of the chapter).  The log-sum-exp output is not on the
pages; its definition here (natural log of the sum of exponentials of the
scaled, masked scores) is this project's reading.  A row with no visible key
has O = 0 and LSE = -inf (also a reading).

``online_tiled`` follows section 21.1's online recurrence tile by tile (running
max, running sum, and an accumulator rescaled by alpha = exp(m_old - m_new)),
visiting non-empty kv tiles in ascending order.  It exists to pin that the
tiled result does not depend on the block sizes.
"""

from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: widen exactly
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def three_pass(q, k, v, vis, scale: float, row_block: int = 1024):
    """O [Lq, Dv] and LSE [Lq] (float64) for one head of one sequence."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    vis = np.asarray(vis, dtype=bool)
    Lq = q.shape[0]
    O = np.zeros((Lq, v.shape[1]), np.float64)
    lse = np.full(Lq, -np.inf, np.float64)
    for r0 in range(0, Lq, row_block):
        r1 = min(Lq, r0 + row_block)
        s = (q[r0:r1] @ k.T) * scale
        mask = vis[r0:r1]
        s = np.where(mask, s, -np.inf)
        has = mask.any(axis=1)
        # pass 1: running maximum over the visible keys
        m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
        # pass 2: sum of exponentials relative to the maximum
        e = np.exp(s - m[:, None])  # exp(-inf) = 0 on hidden pairs
        l = e.sum(axis=1)
        # pass 3: normalise and weight the values
        with np.errstate(invalid="ignore", divide="ignore"):
            p = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
        O[r0:r1] = p @ v
        lse[r0:r1] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, lse


def online_tiled(q, k, v, vis, scale: float, BM: int, BN: int, skip_empty: bool = True):
    """The same O and LSE through the tile-by-tile online softmax.

    Empty tiles (no visible pair) are skipped when ``skip_empty``.  A row
    whose running maximum is still -inf after a tile uses 0 in its place, so
    exp(-inf - (-inf)) never occurs (a reading; the pages' examples never
    reach it).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    vis = np.asarray(vis, dtype=bool)
    Lq, Lk = vis.shape
    O = np.zeros((Lq, v.shape[1]), np.float64)
    lse = np.full(Lq, -np.inf, np.float64)
    for r0 in range(0, Lq, BM):
        r1 = min(Lq, r0 + BM)
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, v.shape[1]))
        for c0 in range(0, Lk, BN):
            c1 = min(Lk, c0 + BN)
            blk = vis[r0:r1, c0:c1]
            if skip_empty and not blk.any():
                continue
            s = (q[r0:r1] @ k[c0:c1].T) * scale
            s = np.where(blk, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            m_use = np.where(np.isneginf(m_new), 0.0, m_new)
            alpha = np.exp(m - m_use)
            p = np.exp(s - m_use[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = acc * alpha[:, None] + p @ v[c0:c1]
            m = m_new
        has = l > 0
        O[r0:r1] = np.where(has[:, None], acc / np.where(has, l, 1.0)[:, None], 0.0)
        lse[r0:r1] = np.where(has, np.where(np.isneginf(m), 0.0, m) + np.log(np.where(has, l, 1.0)),
                              -np.inf)
    return O, lse
