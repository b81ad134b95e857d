"""fp64 CPU oracle for exact softmax attention, its backward and its
backward-over-backward.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline may import this module.  It shares no code with the HIP library and
imports nothing from it.

Everything here is the plain definition, written out densely per (batch, head)
with NumPy in float64.  Rows are processed in chunks so that no more than
``chunk`` full rows of the N x N matrices exist at a time; chunking only
bounds memory, each row is still computed from its full definition.

Notation (per head): Q, K, V, dO are N x d; c is the softmax scale; S = Q K^T
is the raw score matrix; the causal mask keeps key j for query i iff j <= i.

Sources (pages, with the section each definition follows):
  * forward: "FlashAttention for trading models" explainer (marketmaker.cc),
    sections "Why is attention tied to memory" (softmax(QK^T/sqrt(d_k)) V) and
    "The Flash Attention algorithm" (per-row max m and sum l);
  * LSE: the row statistics (m, l) kept for the backward, same page, section
    "Backward pass: recompute instead of store";
  * backward: same section; zero row sums of the score gradient from the GProj
    page (rit.work, flashattention-bf16-gradient-gproj), section "How a zero sum
    turns into a false gradient";
  * backward-over-backward: the FlashBoB page (rit.work,
    flashbob-second-order-attention), section "Why go backward through an
    already computed gradient": the derivative of the first backward's
    gradients with respect to the attention inputs and the incoming gradient.
    The pages give no formula; the closed forms below are derived from that
    definition (vector-Jacobian product of (Q, K, V, dO) -> (dQ, dK, dV)).
"""
from __future__ import annotations

import numpy as np

__all__ = ["probs", "fwd", "bwd", "bob", "hvp", "rows", "last_columns", "gproj_project",
           "max_prob", "expand_kv", "reduce_kv", "fwd_gqa", "bwd_gqa", "bob_gqa"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _visible(rows_idx: np.ndarray, ncols: int, causal: bool, window: int = 0,
             starts=None, blocks=None) -> np.ndarray:
    """Boolean (len(rows_idx), ncols): True where query rows_idx[a] sees key j:
    j <= i when causal, and additionally j > i - window for a sliding window
    (window > 0) and j >= starts[i] for document masks (starts: this batch
    row's first position of each query's document); blocks (this batch row's
    (nb, nb) block-sparse mask over 128 x 128 blocks) further hides key j
    from query i where blocks[i // 128, j // 128] == 0.  These are the
    flexible masks the FlashBoB page names among its next extensions (closing
    paragraph)."""
    j = np.arange(ncols)[None, :]
    if causal:
        vis = j <= rows_idx[:, None]
        if window > 0:
            vis &= j > rows_idx[:, None] - window
        if starts is not None:
            vis &= j >= np.asarray(starts)[rows_idx][:, None]
    else:
        assert window == 0 and starts is None, "window and document masks need the causal mask"
        vis = np.ones((rows_idx.size, ncols), dtype=bool)
    if blocks is not None:
        bl = np.asarray(blocks) != 0
        vis &= bl[rows_idx // 128][:, np.arange(ncols) // 128]
    return vis


def _row_softmax(q_rows, k, rows_idx, causal, scale, window=0, starts=None, blocks=None):
    """P rows and LSE for the given query rows against keys k.

    m_i is the row max of the raw scores over visible keys; the exponent is
    taken as c * (S - m), i.e. the max is subtracted before scaling, so the
    largest entry is exactly exp(0) = 1 (GProj page, section "Why the error
    shows up at the end of training").  LSE_i = c m_i + ln l_i.  A row with
    no visible key (possible only under a block-sparse mask) is the empty
    softmax: P = 0 and LSE = -inf (the log of an empty sum)."""
    s = q_rows @ k.T
    vis = _visible(rows_idx, k.shape[0], causal, window, starts, blocks)
    empty = ~vis.any(axis=1)
    s_vis = np.where(vis, s, -np.inf)
    m = np.where(empty[:, None], 0.0, s_vis.max(axis=1, keepdims=True))
    e = np.exp(scale * (s_vis - m))        # masked keys: exp(-inf) = 0
    l = e.sum(axis=1, keepdims=True)
    p = e / np.where(empty[:, None], 1.0, l)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, scale * m[:, 0] + np.log(l[:, 0]))
    return p, lse


def probs(Q, K, causal=True, scale=None):
    """Dense softmax probabilities P, shape (B, H, N, N).  Small inputs only."""
    Q, K = _f64(Q), _f64(K)
    B, H, N, d = Q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, H, N, N))
    idx = np.arange(N)
    for b in range(B):
        for h in range(H):
            out[b, h], _ = _row_softmax(Q[b, h], K[b, h], idx, causal, c)
    return out


def max_prob(Q, K, causal=True, scale=None, heads=None, row_idx=None, chunk=1024):
    """max_j P_ij for the selected rows of the selected heads, shape
    (len(heads), len(rows)).  Used to place a workload in the near one-hot
    regime described on the GProj page."""
    Q, K = _f64(Q), _f64(K)
    B, H, N, d = Q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    idx_all = np.arange(N) if row_idx is None else np.asarray(row_idx, dtype=np.int64)
    out = np.zeros((len(heads), idx_all.size))
    for n, (b, h) in enumerate(heads):
        for a0 in range(0, idx_all.size, chunk):
            idx = idx_all[a0:a0 + chunk]
            ncols = int(idx.max()) + 1 if causal else N
            p, _ = _row_softmax(Q[b, h][idx], K[b, h][:ncols], idx, causal, c)
            out[n, a0:a0 + idx.size] = p.max(axis=1)
    return out


def _head(q, k, v, do, a, bk, cv, rows_idx, causal, c, want_bwd, want_bob, window=0,
          starts=None, blocks=None):
    """All outputs of one head for the query rows ``rows_idx``.

    Row outputs (O, LSE, D, dQ, alpha, beta, gQ, gdO) are complete for those
    rows.  Column outputs (dK, dV, gK, gV) are the contributions of those rows
    only; summing them over a partition of all rows gives the full result."""
    ncols = k.shape[0]
    if causal:
        ncols = int(rows_idx.max()) + 1
    kk, vv = k[:ncols], v[:ncols]
    qr = q[rows_idx]
    p, lse = _row_softmax(qr, kk, rows_idx, causal, c, window, starts, blocks)
    o = p @ vv
    r = {"O": o, "LSE": lse}
    if not (want_bwd or want_bob):
        return r, ncols
    dor = do[rows_idx]
    # D_i = sum_a dO_ia O_ia (equals sum_j P_ij dP_ij in exact arithmetic)
    D = np.einsum("ia,ia->i", dor, o)
    dP = dor @ vv.T
    dS = p * (dP - D[:, None])
    r["D"] = D
    if want_bwd:
        r["dQ"] = c * (dS @ kk)
        r["dK"] = c * (dS.T @ qr)
        r["dV"] = p.T @ dor
    if want_bob:
        ar = a[rows_idx]
        bkk, cc = bk[:ncols], cv[:ncols]
        vis = _visible(rows_idx, ncols, causal, window, starts, blocks)
        # Phi = <A, dQ> + <Bk, dK> + <C, dV> = <dS, W> + <P, U>
        W = np.where(vis, c * (ar @ kk.T + qr @ bkk.T), 0.0)
        U = np.where(vis, dor @ cc.T, 0.0)
        # through dP (P held fixed): dPhi/d(dP) = P o (W - alpha)
        alpha = np.einsum("ij,ij->i", p, W)
        Hm = p * (W - alpha[:, None])
        # through P (dP, W, U held fixed): dPhi/dP = G
        G = W * (dP - D[:, None]) - alpha[:, None] * dP + U
        # softmax Jacobian on the scaled scores s = c S
        beta = np.einsum("ij,ij->i", p, G)
        Sh = p * (G - beta[:, None])
        r["alpha"], r["beta"] = alpha, beta
        r["gQ"] = c * (Sh @ kk + dS @ bkk)
        r["gK"] = c * (Sh.T @ qr + dS.T @ ar)
        r["gV"] = Hm.T @ dor
        r["gdO"] = Hm @ vv + p @ cc
    return r, ncols


_ROW_KEYS = ("O", "LSE", "D", "dQ", "alpha", "beta", "gQ", "gdO")
_COL_KEYS = ("dK", "dV", "gK", "gV")


def _run(Q, K, V, dO=None, A=None, Bk=None, C=None, causal=True, scale=None,
         want_bwd=False, want_bob=False, chunk=1024, heads=None, window=0, docs=None,
         block_mask=None):
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, d = Q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    dO = None if dO is None else _f64(dO)
    A = None if A is None else _f64(A)
    Bk = None if Bk is None else _f64(Bk)
    C = None if C is None else _f64(C)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    keys = ["O", "LSE"]
    if want_bwd or want_bob:
        keys += ["D"]
    if want_bwd:
        keys += ["dQ", "dK", "dV"]
    if want_bob:
        keys += ["alpha", "beta", "gQ", "gK", "gV", "gdO"]
    out = {}
    for key in keys:
        shp = (B, H, N) if key in ("LSE", "D", "alpha", "beta") else (B, H, N, d)
        out[key] = np.zeros(shp)
    for (b, h) in heads:
        args = (Q[b, h], K[b, h], V[b, h],
                None if dO is None else dO[b, h],
                None if A is None else A[b, h],
                None if Bk is None else Bk[b, h],
                None if C is None else C[b, h])
        for r0 in range(0, N, chunk):
            idx = np.arange(r0, min(N, r0 + chunk))
            r, ncols = _head(*args, idx, causal, c, want_bwd, want_bob, window,
                             None if docs is None else np.asarray(docs)[b],
                             None if block_mask is None else np.asarray(block_mask)[b])
            for key, val in r.items():
                if key in _ROW_KEYS:
                    out[key][b, h, idx] = val
                else:
                    out[key][b, h, :ncols] += val
    return out


def fwd(Q, K, V, causal=True, scale=None, heads=None, chunk=1024, window=0, docs=None,
        block_mask=None):
    """O = softmax(c Q K^T + mask) V and LSE_i = c m_i + ln l_i per row."""
    r = _run(Q, K, V, causal=causal, scale=scale, chunk=chunk, heads=heads, window=window,
             docs=docs, block_mask=block_mask)
    return r["O"], r["LSE"]


def bwd(Q, K, V, dO, causal=True, scale=None, heads=None, chunk=1024, window=0, docs=None,
        block_mask=None):
    """Gradients of <dO, O(Q, K, V)>:  dP = dO V^T, D = rowsum(dO o O),
    dS = P o (dP - D), dQ = c dS K, dK = c dS^T Q, dV = P^T dO.
    Returns dict with O, LSE, D, dQ, dK, dV."""
    return _run(Q, K, V, dO, causal=causal, scale=scale, want_bwd=True,
                heads=heads, chunk=chunk, window=window, docs=docs, block_mask=block_mask)


def bob(Q, K, V, dO, gdQ, gdK, gdV, causal=True, scale=None, heads=None,
        chunk=1024, with_bwd=False, window=0, docs=None, block_mask=None):
    """Backward-over-backward: the gradient of
    Phi = <gdQ, dQ> + <gdK, dK> + <gdV, dV> with respect to (Q, K, V, dO),
    where (dQ, dK, dV) is the first backward of ``bwd``.  With A = gdQ,
    Bk = gdK, C = gdV:
        W = c (A K^T + Q Bk^T),  U = dO C^T              (masked)
        alpha_i = sum_j P_ij W_ij,   H = P o (W - alpha)
        G = W o (dP - D) - alpha o dP + U
        beta_i  = sum_j P_ij G_ij,   Sh = P o (G - beta)
        gQ = c (Sh K + dS Bk),   gK = c (Sh^T Q + dS^T A)
        gV = H^T dO,             gdO = H V + P C
    alpha and beta are the two per-row scalar states.  Returns a dict with
    O, LSE, D, alpha, beta, gQ, gK, gV, gdO (and dQ, dK, dV if with_bwd)."""
    return _run(Q, K, V, dO, gdQ, gdK, gdV, causal=causal, scale=scale,
                want_bwd=with_bwd, want_bob=True, heads=heads, chunk=chunk, window=window,
                docs=docs, block_mask=block_mask)


def hvp(Q, K, V, dO, vQ, vK, vV, causal=True, scale=None, heads=None, chunk=1024):
    """Hessian of Phi(Q, K, V) = <dO, O(Q, K, V)>, dO held fixed, applied to
    v = (vQ, vK, vV) (FlashBoB page, section "Why go backward through an
    already computed gradient": the Hessian-vector products second-order
    methods consume).  The gradient of Phi is (dQ, dK, dV) of ``bwd``, so H v
    is the vector-Jacobian product of (Q, K, V) -> (dQ, dK, dV) with
    cotangents v: the Q, K, V parts of ``bob`` with (gdQ, gdK, gdV) = v.  The
    dO part (HvdO) is the mixed derivative of <v, grad Phi> in dO.  Returns a
    dict with O, LSE, HvQ, HvK, HvV, HvdO."""
    r = bob(Q, K, V, dO, vQ, vK, vV, causal=causal, scale=scale, heads=heads, chunk=chunk)
    return {"O": r["O"], "LSE": r["LSE"], "HvQ": r["gQ"], "HvK": r["gK"], "HvV": r["gV"],
            "HvdO": r["gdO"]}


# ----------------------------------------------------- shared keys and values
# Grouped-query attention (FlashBoB page, closing paragraph: shared keys and
# values are named among the next extensions).  Query head h of a batch reads
# key/value head h // g, g = H / Hkv; the model is multi-head attention on the
# expanded K, V, and by the chain rule the gradient of a shared key-side
# tensor is the sum of its copies' gradients.

def expand_kv(X, group):
    """(B, Hkv, N, d) -> (B, Hkv * group, N, d): head h is a copy of h // group."""
    return np.repeat(_f64(X), group, axis=1)


def reduce_kv(G, group):
    """(B, H, N, d) per-query-head gradients -> (B, H / group, N, d) group sums."""
    B, H, N, d = G.shape
    return G.reshape(B, H // group, group, N, d).sum(axis=2)


def _group(Q, K):
    H, Hkv = np.shape(Q)[1], np.shape(K)[1]
    assert H % Hkv == 0
    return H // Hkv


def fwd_gqa(Q, K, V, causal=True, scale=None, window=0, docs=None, block_mask=None):
    g = _group(Q, K)
    return fwd(Q, expand_kv(K, g), expand_kv(V, g), causal=causal, scale=scale, window=window,
               docs=docs, block_mask=block_mask)


def bwd_gqa(Q, K, V, dO, causal=True, scale=None, window=0, docs=None, block_mask=None):
    g = _group(Q, K)
    r = bwd(Q, expand_kv(K, g), expand_kv(V, g), dO, causal=causal, scale=scale, window=window,
            docs=docs, block_mask=block_mask)
    r["dK"], r["dV"] = reduce_kv(r["dK"], g), reduce_kv(r["dV"], g)
    return r


def bob_gqa(Q, K, V, dO, gdQ, gdK, gdV, causal=True, scale=None, with_bwd=False, window=0,
            docs=None, block_mask=None):
    """BoB of the grouped-query map: <gdK, dK> with dK summed over a group is
    <expand(gdK), dK per query head>, so the cotangents expand like K and V
    and the key-side outputs reduce like dK, dV."""
    g = _group(Q, K)
    r = bob(Q, expand_kv(K, g), expand_kv(V, g), dO, gdQ, expand_kv(gdK, g), expand_kv(gdV, g),
            causal=causal, scale=scale, with_bwd=with_bwd, window=window, docs=docs,
            block_mask=block_mask)
    for k in ("gK", "gV") + (("dK", "dV") if with_bwd else ()):
        r[k] = reduce_kv(r[k], g)
    return r


def rows(Q, K, V, dO=None, gdQ=None, gdK=None, gdV=None, row_idx=None,
         causal=True, scale=None, heads=None, window=0, docs=None):
    """Row outputs (O, LSE, D, dQ, alpha, beta, gQ, gdO) for selected rows of
    selected heads, each row computed exactly from its own definition.
    ``row_idx`` is a sorted 1-D array of query positions; ``window`` and
    ``docs`` (each batch row's document starts) are the masks of ``fwd``.
    Returns a dict of arrays shaped (len(heads), len(row_idx)[, d])."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, d = Q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    row_idx = np.asarray(row_idx, dtype=np.int64)
    want_bwd = dO is not None
    want_bob = gdQ is not None
    res = {}
    for n, (b, h) in enumerate(heads):
        g = lambda X: None if X is None else _f64(X[b, h])
        r, _ = _head(Q[b, h], K[b, h], V[b, h], g(dO), g(gdQ), g(gdK), g(gdV),
                     row_idx, causal, c, want_bwd, want_bob, window,
                     None if docs is None else np.asarray(docs)[b])
        for key, val in r.items():
            if key in _ROW_KEYS:
                res.setdefault(key, []).append(val)
    return {k: np.stack(v) for k, v in res.items()}


def last_columns(Q, K, V, dO, gdQ=None, gdK=None, gdV=None, ncols_tail=256,
                 scale=None, heads=None, chunk=256, window=0, docs=None):
    """Column outputs for the last ``ncols_tail`` keys of a causal head: dK and
    dV, or gK and gV when the cotangents are given.  Under the causal mask key j is
    seen only by queries i >= j (a window or document mask only removes some of
    them), so the rows N - ncols_tail .. N - 1 hold every contribution to these
    columns.  Returns arrays (len(heads), ncols_tail, d)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, H, N, d = Q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    want_bob = gdQ is not None
    n0 = N - ncols_tail
    res = {}
    for (b, h) in heads:
        g = lambda X: None if X is None else _f64(X[b, h])
        acc = {}
        for r0 in range(n0, N, chunk):
            idx = np.arange(r0, min(N, r0 + chunk))
            r, ncols = _head(Q[b, h], K[b, h], V[b, h], g(dO), g(gdQ), g(gdK),
                             g(gdV), idx, True, c, not want_bob, want_bob, window,
                             None if docs is None else np.asarray(docs)[b])
            for key, val in r.items():
                if key in _COL_KEYS:
                    tail = np.zeros((ncols_tail, d))
                    tail[: ncols - n0] = val[n0:ncols]
                    acc[key] = acc.get(key, 0.0) + tail
        for key, val in acc.items():
            res.setdefault(key, []).append(val)
    return {k: np.stack(v) for k, v in res.items()}


def gproj_project(X, P):
    """GProj projection of a score-gradient block X against probabilities P
    (GProj page, section "How a zero sum turns into a false gradient"): the
    residual mass of each row, r_i = sum_k X_ik, is removed in proportion to
    the attention probabilities,  Pi_P(X)_ij = X_ij - r_i P_ij.  When each row
    of P sums to 1 every projected row sums to 0."""
    X, P = _f64(X), _f64(P)
    r = X.sum(axis=-1, keepdims=True)
    return X - r * P
