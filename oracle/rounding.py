"""bf16 rounding, and an fp64 model of where a bf16 backward rounds.

TEST INFRASTRUCTURE (see the oracle package header).

The GProj page (rit.work, flashattention-bf16-gradient-gproj, section "How a
zero sum turns into a false gradient") explains a failure of the bf16
backward: the score gradient dS is rounded to bf16 before it is multiplied by
the keys, the rounded rows no longer sum to zero, and the leftover mass adds a
component along the mean key.  GProj measures each row's leftover mass on the
rounded values and subtracts that share of the attention probabilities.

``bwd_rounded`` reproduces only those rounding points, in fp64 otherwise, so the
claim can be checked on the CPU:  with R the fp32 -> bf16 round-to-nearest-even,
    r_i  = sum_j R(dS)_ij
    dQ   = c (R(dS) K - gproj * r_i R(P) K)
It is a model of the rounding, not the parity reference: the reference for
dQ is the exact ``attention.bwd``.
"""
from __future__ import annotations

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), returned as float64.
    The value is first rounded to fp32 (as a float32 register would hold it);
    finite inputs only."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def bwd_rounded(Q, K, V, dO, gproj: bool, causal=True, scale=None, heads=None,
                row_idx=None, round_o=True):
    """dQ rows of a backward that rounds dS (and P for the GProj term) to bf16
    before the products with K.  O is rounded to bf16 as a stored forward
    output would be when ``round_o``.  Returns (len(heads), len(rows), d)."""
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    B, H, N, d = Q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    idx = np.arange(N) if row_idx is None else np.asarray(row_idx, dtype=np.int64)
    out = []
    for (b, h) in heads:
        q, k, v, do = Q[b, h][idx], K[b, h], V[b, h], dO[b, h][idx]
        s = q @ k.T
        vis = (np.arange(N)[None, :] <= idx[:, None]) if causal else np.ones((idx.size, N), bool)
        s_vis = np.where(vis, s, -np.inf)
        m = s_vis.max(axis=1, keepdims=True)
        e = np.exp(c * (s_vis - m))
        p = e / e.sum(axis=1, keepdims=True)
        o = p @ v
        if round_o:
            o = bf16_round(o)
        D = np.einsum("ia,ia->i", do, o)
        dS = p * (do @ v.T - D[:, None])
        rdS = bf16_round(dS)
        dq = rdS @ k
        if gproj:
            r = rdS.sum(axis=1)
            dq = dq - r[:, None] * (bf16_round(p) @ k)
        out.append(c * dq)
    return np.stack(out)
