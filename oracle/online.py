"""fp64 model of the tiled forward pass with the online softmax recurrence.

TEST INFRASTRUCTURE (see the oracle package header).

This follows the blocked algorithm of the "FlashAttention for trading models"
explainer (marketmaker.cc), sections "The Flash Attention algorithm" and "The
online softmax recurrence": queries are split into blocks of Br rows and keys
and values into blocks of Bc rows; for each query block a running row max m,
a running row sum l and an output accumulator are carried across the key
blocks, and whenever a new block raises the max the earlier sum and output
are rescaled by exp(m_old - m_new).  In exact arithmetic the result equals
the two-pass softmax; this model exists to check that claim against the dense
definition in ``attention.py`` and to document the recurrence the forward
kernel implements.
"""
from __future__ import annotations

import numpy as np


def online_fwd(Q, K, V, causal=True, scale=None, Br=16, Bc=16):
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    B, H, N, d = Q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    O = np.zeros_like(Q)
    LSE = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, N, Br):
                i1 = min(N, i0 + Br)
                qi = Q[b, h, i0:i1]
                qidx = np.arange(i0, i1)
                m = np.full(i1 - i0, -np.inf)      # running max of scaled scores
                l = np.zeros(i1 - i0)              # running sum
                acc = np.zeros((i1 - i0, d))       # unnormalised output
                jend = i1 if causal else N
                for j0 in range(0, jend, Bc):
                    j1 = min(N, j0 + Bc)
                    s = c * (qi @ K[b, h, j0:j1].T)
                    if causal:
                        vis = np.arange(j0, j1)[None, :] <= qidx[:, None]
                        s = np.where(vis, s, -np.inf)
                    m_blk = s.max(axis=1)
                    m_new = np.maximum(m, m_blk)
                    live = np.isfinite(m_new)      # rows that have seen a key
                    safe = np.where(live, m_new, 0.0)
                    p = np.exp(s - safe[:, None])  # exp(-inf) = 0 for masked
                    corr = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
                    l = l * corr + p.sum(axis=1)
                    acc = acc * corr[:, None] + p @ V[b, h, j0:j1]
                    m = m_new
                O[b, h, i0:i1] = acc / l[:, None]
                LSE[b, h, i0:i1] = m + np.log(l)
    return O, LSE
