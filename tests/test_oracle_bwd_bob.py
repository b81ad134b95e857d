"""Pins of the oracle's backward, GProj projection and backward-over-backward
(CPU only).

The backward is pinned by central finite differences of <dO, O> and by the
invariants of softmax attention; the backward-over-backward by finite
differences of Phi = <A, dQ> + <Bk, dK> + <C, dV>, symmetry of the
Hessian-vector product, Euler identities of the homogeneous parts, the
key-shift and Q/K-rescaling invariances, the single-token closed form, and
torch's autograd double backward in fp64."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.rounding import bf16_round, bwd_rounded


def rnd(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def inputs(B, H, N, d, seed, std=1.0):
    return [rnd((B, H, N, d), seed + i, std) for i in range(7)]   # Q K V dO A Bk C


def dot(x, y):
    return float(np.sum(x * y))


# ---------------------------------------------------------------- backward
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_finite_differences(causal):
    Q, K, V, dO = inputs(1, 1, 6, 3, 100)[:4]
    g = oracle.bwd(Q, K, V, dO, causal=causal)
    f = lambda q, k, v: dot(dO, oracle.fwd(q, k, v, causal=causal)[0])
    h = 1e-6
    for name, X, G in (("Q", Q, g["dQ"]), ("K", K, g["dK"]), ("V", V, g["dV"])):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = {"Q": Q, "K": K, "V": V}
            args_m = dict(args_p)
            args_p[name], args_m[name] = Xp, Xm
            num[idx] = (f(args_p["Q"], args_p["K"], args_p["V"]) -
                        f(args_m["Q"], args_m["K"], args_m["V"])) / (2 * h)
        assert np.linalg.norm(num - G) <= 1e-6 * np.linalg.norm(G), name


def test_bwd_invariants():
    Q, K, V, dO = inputs(2, 2, 31, 8, 110)[:4]
    g = oracle.bwd(Q, K, V, dO)
    O = g["O"]
    # score-gradient rows sum to 0  ->  dK sums to 0 over keys
    assert np.allclose(g["dK"].sum(axis=2), 0.0, atol=1e-12)
    # dV = P^T dO and P rows sum to 1  ->  sum_j dV_j = sum_i dO_i
    assert np.allclose(g["dV"].sum(axis=2), dO.sum(axis=2), atol=1e-12)
    # O is linear in V:  <V, dV> = <O, dO>
    assert dot(V, g["dV"]) == pytest.approx(dot(O, dO), rel=1e-12)
    # S is invariant under Q -> tQ, K -> K/t:  <Q, dQ> = <K, dK>
    assert dot(Q, g["dQ"]) == pytest.approx(dot(K, g["dK"]), rel=1e-10)
    # row 0 sees a single key: its softmax has no freedom, dQ_0 = 0
    assert np.allclose(g["dQ"][:, :, 0], 0.0, atol=1e-13)
    # D = rowsum(dO o O)
    assert np.allclose(g["D"], np.einsum("bhnd,bhnd->bhn", dO, O), atol=1e-13)


def test_score_gradient_rows_sum_to_zero():
    Q, K, V, dO = inputs(1, 2, 25, 8, 120)[:4]
    P = oracle.probs(Q, K)
    g = oracle.bwd(Q, K, V, dO)
    dP = dO @ np.swapaxes(V, -1, -2)
    dS = P * (dP - g["D"][..., None])
    assert np.allclose(dS.sum(-1), 0.0, atol=1e-13)
    c = 1 / math.sqrt(8)
    assert np.allclose(c * dS @ K, g["dQ"], atol=1e-13)


def torch_attention(q, k, v, causal, c):
    s = c * (q @ k.transpose(-1, -2))
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    return torch.softmax(s, dim=-1) @ v


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_and_bob_against_torch_double_backward(causal):
    Q, K, V, dO, A, Bk, C = inputs(2, 2, 19, 8, 130)
    c = 1 / math.sqrt(8)
    tq, tk, tv, tdo = (torch.tensor(x, requires_grad=True) for x in (Q, K, V, dO))
    out = torch_attention(tq, tk, tv, causal, c)
    gq, gk, gv = torch.autograd.grad(out, (tq, tk, tv), tdo, create_graph=True)
    phi = (gq * torch.from_numpy(A)).sum() + (gk * torch.from_numpy(Bk)).sum() + \
        (gv * torch.from_numpy(C)).sum()
    hq, hk, hv, hdo = torch.autograd.grad(phi, (tq, tk, tv, tdo))
    r = oracle.bob(Q, K, V, dO, A, Bk, C, causal=causal, with_bwd=True)
    for mine, ref in ((r["dQ"], gq), (r["dK"], gk), (r["dV"], gv), (r["gQ"], hq),
                      (r["gK"], hk), (r["gV"], hv), (r["gdO"], hdo)):
        ref = ref.detach().numpy()
        assert np.linalg.norm(mine - ref) <= 1e-12 * max(1.0, np.linalg.norm(ref))


@pytest.mark.parametrize("H,Hkv", [(4, 2), (4, 1), (3, 3)])
def test_grouped_query_against_torch_double_backward(H, Hkv):
    # shared keys and values: torch's autograd differentiates through
    # repeat_interleave (its own sum over each group), independently of the
    # oracle's expand/reduce
    g = H // Hkv
    rng = np.random.default_rng(135)
    Q, dO, A = (rng.standard_normal((1, H, 13, 8)) for _ in range(3))
    K, V, Bk, C = (rng.standard_normal((1, Hkv, 13, 8)) for _ in range(4))
    c = 1 / math.sqrt(8)
    tq, tk, tv, tdo = (torch.tensor(x, requires_grad=True) for x in (Q, K, V, dO))
    out = torch_attention(tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1),
                          True, c)
    gq, gk, gv = torch.autograd.grad(out, (tq, tk, tv), tdo, create_graph=True)
    phi_ = (gq * torch.from_numpy(A)).sum() + (gk * torch.from_numpy(Bk)).sum() + \
        (gv * torch.from_numpy(C)).sum()
    hq, hk, hv, hdo = torch.autograd.grad(phi_, (tq, tk, tv, tdo))
    o, lse = oracle.fwd_gqa(Q, K, V)
    r = oracle.bob_gqa(Q, K, V, dO, A, Bk, C, with_bwd=True)
    assert np.linalg.norm(o - out.detach().numpy()) <= 1e-12 * np.linalg.norm(o)
    for mine, ref in ((r["dQ"], gq), (r["dK"], gk), (r["dV"], gv), (r["gQ"], hq),
                      (r["gK"], hk), (r["gV"], hv), (r["gdO"], hdo)):
        ref = ref.detach().numpy()
        assert mine.shape == ref.shape
        assert np.linalg.norm(mine - ref) <= 1e-12 * max(1.0, np.linalg.norm(ref))
    b = oracle.bwd_gqa(Q, K, V, dO)
    assert np.linalg.norm(b["dK"] - r["dK"]) <= 1e-13 * np.linalg.norm(b["dK"])


@pytest.mark.parametrize("window", [1, 3, 7])
def test_sliding_window_against_torch_double_backward(window):
    # a causal sliding window as an explicit boolean mask in torch (fp64
    # autograd, double backward), independent of the oracle's _visible
    Q, K, V, dO, A, Bk, C = inputs(1, 2, 15, 8, 137)
    c = 1 / math.sqrt(8)
    n = 15
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    hide = (j > i) | (j <= i - window)
    tq, tk, tv, tdo = (torch.tensor(x, requires_grad=True) for x in (Q, K, V, dO))
    s_ = (c * (tq @ tk.transpose(-1, -2))).masked_fill(hide, float("-inf"))
    out = torch.softmax(s_, dim=-1) @ tv
    gq, gk, gv = torch.autograd.grad(out, (tq, tk, tv), tdo, create_graph=True)
    phi_ = (gq * torch.from_numpy(A)).sum() + (gk * torch.from_numpy(Bk)).sum() + \
        (gv * torch.from_numpy(C)).sum()
    hq, hk, hv, hdo = torch.autograd.grad(phi_, (tq, tk, tv, tdo))
    r = oracle.bob(Q, K, V, dO, A, Bk, C, with_bwd=True, window=window)
    o, _ = oracle.fwd(Q, K, V, window=window)
    assert np.linalg.norm(o - out.detach().numpy()) <= 1e-12 * np.linalg.norm(o)
    for mine, ref in ((r["dQ"], gq), (r["dK"], gk), (r["dV"], gv), (r["gQ"], hq),
                      (r["gK"], hk), (r["gV"], hv), (r["gdO"], hdo)):
        ref = ref.detach().numpy()
        assert np.linalg.norm(mine - ref) <= 1e-12 * max(1.0, np.linalg.norm(ref))


def test_document_mask_against_torch_and_independent_documents():
    # packed documents: torch fp64 double backward with an explicit mask; and
    # the packed result equals running each document on its own
    Q, K, V, dO, A, Bk, C = inputs(1, 2, 16, 8, 139)
    bounds = [0, 5, 6, 13, 16]                       # documents [0,5) [5,6) [6,13) [13,16)
    starts = np.zeros(16, dtype=np.int64)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        starts[lo:hi] = lo
    docs = starts[None, :]
    c = 1 / math.sqrt(8)
    i = torch.arange(16)[:, None]
    j = torch.arange(16)[None, :]
    hide = (j > i) | (j < torch.from_numpy(starts)[:, None])
    tq, tk, tv, tdo = (torch.tensor(x, requires_grad=True) for x in (Q, K, V, dO))
    s_ = (c * (tq @ tk.transpose(-1, -2))).masked_fill(hide, float("-inf"))
    out = torch.softmax(s_, dim=-1) @ tv
    gq, gk, gv = torch.autograd.grad(out, (tq, tk, tv), tdo, create_graph=True)
    phi_ = (gq * torch.from_numpy(A)).sum() + (gk * torch.from_numpy(Bk)).sum() + \
        (gv * torch.from_numpy(C)).sum()
    hq, hk, hv, hdo = torch.autograd.grad(phi_, (tq, tk, tv, tdo))
    r = oracle.bob(Q, K, V, dO, A, Bk, C, with_bwd=True, docs=docs)
    for mine, ref in ((r["dQ"], gq), (r["dK"], gk), (r["dV"], gv), (r["gQ"], hq),
                      (r["gK"], hk), (r["gV"], hv), (r["gdO"], hdo)):
        ref = ref.detach().numpy()
        assert np.linalg.norm(mine - ref) <= 1e-12 * max(1.0, np.linalg.norm(ref))
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        sl = slice(lo, hi)
        own = oracle.bob(Q[..., sl, :], K[..., sl, :], V[..., sl, :], dO[..., sl, :],
                         A[..., sl, :], Bk[..., sl, :], C[..., sl, :], with_bwd=True)
        for k in ("O", "dQ", "dK", "dV", "gQ", "gK", "gV", "gdO"):
            assert np.allclose(r[k][..., sl, :], own[k], rtol=1e-12, atol=1e-13), (k, lo)


def _torch_masked_double_backward(Q, K, V, dO, A, Bk, C, hide, c):
    """fp64 torch autograd: outputs and BoB of softmax attention with an
    explicit boolean mask (True hides), query rows Q may be a subset."""
    tq, tk, tv, tdo = (torch.tensor(x, requires_grad=True) for x in (Q, K, V, dO))
    s_ = (c * (tq @ tk.transpose(-1, -2))).masked_fill(torch.from_numpy(hide), float("-inf"))
    out = torch.softmax(s_, dim=-1) @ tv
    gq, gk, gv = torch.autograd.grad(out, (tq, tk, tv), tdo, create_graph=True)
    phi_ = (gq * torch.from_numpy(A)).sum() + (gk * torch.from_numpy(Bk)).sum() + \
        (gv * torch.from_numpy(C)).sum()
    hq, hk, hv, hdo = torch.autograd.grad(phi_, (tq, tk, tv, tdo))
    return {k: t.detach().numpy() for k, t in (("O", out), ("dQ", gq), ("dK", gk), ("dV", gv),
                                               ("gQ", hq), ("gK", hk), ("gV", hv),
                                               ("gdO", hdo))}


@pytest.mark.parametrize("causal", [True, False])
def test_block_sparse_mask_against_torch_double_backward(causal):
    # a (B, nb, nb) mask over 128 x 128 blocks (N = 300: blocks of 128, 128
    # and 44 rows), expanded to an explicit element mask for torch; every row
    # keeps a visible key (diagonal blocks kept when causal)
    N, d = 300, 8
    Q, K, V, dO, A, Bk, C = inputs(1, 2, N, d, 141)
    c = 1 / math.sqrt(d)
    bm = np.array([[[1, 0, 1], [0, 1, 0], [1, 1, 1]]], dtype=np.uint8)
    if not causal:
        bm[0, 1, 2] = 1
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    hide = bm[0][i // 128, j // 128] == 0
    if causal:
        hide |= j > i
    ref = _torch_masked_double_backward(Q, K, V, dO, A, Bk, C, hide, c)
    r = oracle.bob(Q, K, V, dO, A, Bk, C, causal=causal, with_bwd=True, block_mask=bm)
    o, _ = oracle.fwd(Q, K, V, causal=causal, block_mask=bm)
    assert np.linalg.norm(o - ref["O"]) <= 1e-12 * np.linalg.norm(o)
    for k in ("dQ", "dK", "dV", "gQ", "gK", "gV", "gdO"):
        assert np.linalg.norm(r[k] - ref[k]) <= 1e-12 * max(1.0, np.linalg.norm(ref[k])), k
    # a mask of ones is no mask, bit for bit
    ones = np.ones((1, 3, 3), dtype=np.uint8)
    full = oracle.bob(Q, K, V, dO, A, Bk, C, causal=causal, with_bwd=True)
    same = oracle.bob(Q, K, V, dO, A, Bk, C, causal=causal, with_bwd=True, block_mask=ones)
    for k in full:
        assert np.array_equal(full[k], same[k]), k


def test_block_sparse_empty_rows():
    # query block 0 keeps no key block: its rows are empty softmax rows (O = 0,
    # LSE = -inf, zero row gradients) and contribute nothing to the key side;
    # the other rows and the key-side outputs equal torch on the remaining
    # query rows against all keys
    N, d = 300, 8
    Q, K, V, dO, A, Bk, C = inputs(1, 1, N, d, 142)
    c = 1 / math.sqrt(d)
    bm = np.array([[[0, 0, 0], [1, 0, 1], [0, 1, 1]]], dtype=np.uint8)
    r = oracle.bob(Q, K, V, dO, A, Bk, C, causal=False, with_bwd=True, block_mask=bm)
    assert np.all(r["O"][..., :128, :] == 0) and np.all(np.isneginf(r["LSE"][..., :128]))
    for k in ("dQ", "gQ", "gdO"):
        assert np.all(r[k][..., :128, :] == 0), k
    i = np.arange(128, N)[:, None]
    j = np.arange(N)[None, :]
    hide = bm[0][i // 128, j // 128] == 0
    sub = slice(128, N)
    ref = _torch_masked_double_backward(Q[..., sub, :], K, V, dO[..., sub, :], A[..., sub, :],
                                        Bk, C, hide, c)
    for k in ("O", "dQ", "gQ", "gdO"):
        assert np.linalg.norm(r[k][..., sub, :] - ref[k]) <= 1e-12 * np.linalg.norm(ref[k]), k
    for k in ("dK", "dV", "gK", "gV"):
        assert np.linalg.norm(r[k] - ref[k]) <= 1e-12 * np.linalg.norm(ref[k]), k


def test_window_of_one_closed_form_and_wide_window_is_causal():
    Q, K, V, dO, A, Bk, C = inputs(1, 1, 9, 4, 138)
    c = 0.5
    r = oracle.bwd(Q, K, V, dO, scale=c, window=1)
    # each row sees only its own key: O = V, LSE = c q.k, dS = 0, dV = dO
    assert np.allclose(r["O"], V, atol=1e-15)
    assert np.allclose(r["LSE"], c * np.einsum("bhnd,bhnd->bhn", Q, K), atol=1e-14)
    assert np.abs(r["dQ"]).max() < 1e-14 and np.abs(r["dK"]).max() < 1e-14
    assert np.allclose(r["dV"], dO, atol=1e-15)
    full = oracle.bob(Q, K, V, dO, A, Bk, C, with_bwd=True)
    wide = oracle.bob(Q, K, V, dO, A, Bk, C, with_bwd=True, window=9)
    for k in full:
        assert np.array_equal(full[k], wide[k]), k


# ---------------------------------------------------------------- BoB
def phi(Q, K, V, dO, A, Bk, C, causal=True):
    g = oracle.bwd(Q, K, V, dO, causal=causal)
    return dot(A, g["dQ"]) + dot(Bk, g["dK"]) + dot(C, g["dV"])


@pytest.mark.parametrize("causal", [True, False])
def test_bob_finite_differences(causal):
    Q, K, V, dO, A, Bk, C = inputs(1, 1, 5, 3, 140)
    r = oracle.bob(Q, K, V, dO, A, Bk, C, causal=causal)
    base = {"Q": Q, "K": K, "V": V, "dO": dO}
    h = 1e-6
    for name, G in (("Q", r["gQ"]), ("K", r["gK"]), ("V", r["gV"]), ("dO", r["gdO"])):
        X = base[name]
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            p, m = dict(base), dict(base)
            p[name], m[name] = X.copy(), X.copy()
            p[name][idx] += h
            m[name][idx] -= h
            num[idx] = (phi(p["Q"], p["K"], p["V"], p["dO"], A, Bk, C, causal) -
                        phi(m["Q"], m["K"], m["V"], m["dO"], A, Bk, C, causal)) / (2 * h)
        assert np.linalg.norm(num - G) <= 1e-6 * np.linalg.norm(G), name


def test_bob_hvp_symmetry():
    # (gQ, gK, gV) is the Hessian of <dO, O(Q, K, V)> applied to v = (A, Bk, C)
    Q, K, V, dO, A1, B1, C1 = inputs(1, 2, 17, 8, 150)
    _, _, _, _, A2, B2, C2 = inputs(1, 2, 17, 8, 160)
    h1 = oracle.bob(Q, K, V, dO, A1, B1, C1)
    h2 = oracle.bob(Q, K, V, dO, A2, B2, C2)
    lhs = dot(A1, h2["gQ"]) + dot(B1, h2["gK"]) + dot(C1, h2["gV"])
    rhs = dot(A2, h1["gQ"]) + dot(B2, h1["gK"]) + dot(C2, h1["gV"])
    assert lhs == pytest.approx(rhs, rel=1e-11)


@pytest.mark.parametrize("causal", [True, False])
def test_hvp_is_derivative_of_the_gradient(causal):
    # H v = d/de grad<dO, O>(x + e v) at e = 0, by central differences of the
    # (separately pinned) backward: independent of the BoB closed forms
    Q, K, V, dO, vQ, vK, vV = inputs(1, 2, 9, 6, 155)
    r = oracle.hvp(Q, K, V, dO, vQ, vK, vV, causal=causal)
    h = 1e-5
    gp = oracle.bwd(Q + h * vQ, K + h * vK, V + h * vV, dO, causal=causal)
    gm = oracle.bwd(Q - h * vQ, K - h * vK, V - h * vV, dO, causal=causal)
    for name, key in (("dQ", "HvQ"), ("dK", "HvK"), ("dV", "HvV")):
        num = (gp[name] - gm[name]) / (2 * h)
        assert np.linalg.norm(num - r[key]) <= 1e-7 * np.linalg.norm(r[key]), key
    # the dO part: derivative of <v, grad> in dO; grad is linear in dO
    g1 = oracle.bwd(Q, K, V, dO + 1.0 * vQ, causal=causal)
    g0 = oracle.bwd(Q, K, V, dO, causal=causal)
    lhs = dot(vQ, g1["dQ"] - g0["dQ"]) + dot(vK, g1["dK"] - g0["dK"]) + dot(vV, g1["dV"] - g0["dV"])
    assert lhs == pytest.approx(dot(vQ, r["HvdO"]), rel=1e-10)


def test_bob_identities():
    Q, K, V, dO, A, Bk, C = inputs(2, 2, 23, 8, 170)
    r = oracle.bob(Q, K, V, dO, A, Bk, C, with_bwd=True)
    Phi = dot(A, r["dQ"]) + dot(Bk, r["dK"]) + dot(C, r["dV"])
    # Phi is linear in dO (Euler, degree 1)
    assert dot(dO, r["gdO"]) == pytest.approx(Phi, rel=1e-11)
    # dQ, dK are linear in V and dV does not depend on V
    assert dot(V, r["gV"]) == pytest.approx(dot(A, r["dQ"]) + dot(Bk, r["dK"]), rel=1e-11)
    # Phi is invariant under a common shift of all keys
    assert np.allclose(r["gK"].sum(axis=2), 0.0, atol=1e-11)
    # Q -> tQ, K -> K/t scales dQ by 1/t and dK by t
    assert dot(Q, r["gQ"]) - dot(K, r["gK"]) == pytest.approx(
        dot(Bk, r["dK"]) - dot(A, r["dQ"]), rel=1e-10, abs=1e-10)
    # the row states: alpha = sum P o W, beta = sum P o G with D = rowsum(dO o O)
    P = oracle.probs(Q, K)
    c = 1 / math.sqrt(8)
    W = c * (A @ np.swapaxes(K, -1, -2) + Q @ np.swapaxes(Bk, -1, -2))
    assert np.allclose(r["alpha"], np.sum(P * W, -1), atol=1e-12)
    dP = dO @ np.swapaxes(V, -1, -2)
    U = dO @ np.swapaxes(C, -1, -2)
    beta2 = np.sum(P * (W * dP + U), -1) - 2 * r["alpha"] * r["D"]
    assert np.allclose(r["beta"], beta2, atol=1e-11)


def test_bob_single_token_closed_form():
    Q, K, V, dO, A, Bk, C = inputs(1, 3, 1, 4, 180)
    r = oracle.bob(Q, K, V, dO, A, Bk, C)
    assert np.allclose(r["gdO"], C, atol=1e-15)
    for key in ("gQ", "gK", "gV"):
        assert np.allclose(r[key], 0.0, atol=1e-15)


def test_bob_linear_in_cotangents():
    Q, K, V, dO, A, Bk, C = inputs(1, 2, 13, 8, 190)
    _, _, _, _, A2, B2, C2 = inputs(1, 2, 13, 8, 200)
    r1 = oracle.bob(Q, K, V, dO, A, Bk, C)
    r2 = oracle.bob(Q, K, V, dO, A2, B2, C2)
    r3 = oracle.bob(Q, K, V, dO, 2 * A - A2, 2 * Bk - B2, 2 * C - C2)
    for key in ("gQ", "gK", "gV", "gdO"):
        assert np.allclose(r3[key], 2 * r1[key] - r2[key], atol=1e-12)


# ------------------------------------------------- sampled rows / columns
def test_rows_and_last_columns_match_dense():
    Q, K, V, dO, A, Bk, C = inputs(1, 2, 57, 8, 210)
    full = oracle.bob(Q, K, V, dO, A, Bk, C, with_bwd=True, chunk=13)
    idx = np.array([0, 5, 31, 56])
    r = oracle.rows(Q, K, V, dO, A, Bk, C, row_idx=idx)
    for key in ("O", "LSE", "D", "dQ", "alpha", "beta", "gQ", "gdO"):
        assert np.allclose(r[key], full[key][0][:, idx], atol=1e-13), key
    t = oracle.last_columns(Q, K, V, dO, A, Bk, C, ncols_tail=10, chunk=4)
    assert np.allclose(t["gK"], full["gK"][0][:, -10:], atol=1e-12)
    assert np.allclose(t["gV"], full["gV"][0][:, -10:], atol=1e-12)
    t = oracle.last_columns(Q, K, V, dO, ncols_tail=7)
    assert np.allclose(t["dK"], full["dK"][0][:, -7:], atol=1e-12)
    assert np.allclose(t["dV"], full["dV"][0][:, -7:], atol=1e-12)
    h = oracle.bob(Q, K, V, dO, A, Bk, C, heads=[(0, 1)])
    assert np.allclose(h["gK"][0, 1], full["gK"][0, 1], atol=1e-13)
    assert np.all(h["gK"][0, 0] == 0.0)



@pytest.mark.parametrize("window,with_docs", [(33, False), (0, True), (20, True)])
def test_rows_and_last_columns_match_dense_under_masks(window, with_docs):
    """The row and column samplers with a sliding window or document starts
    give the dense oracle's rows and last columns (the masks only drop keys,
    so the last rows still hold every contribution to the last keys)."""
    Q, K, V, dO, A, Bk, C = inputs(1, 2, 200, 8, 211)
    starts = None
    if with_docs:
        starts = np.zeros((1, 200), dtype=np.int64)
        starts[0, 70:] = 70
        starts[0, 150:] = 150
    full = oracle.bob(Q, K, V, dO, A, Bk, C, with_bwd=True, chunk=37, window=window,
                      docs=starts)
    idx = np.array([0, 5, 69, 70, 100, 149, 150, 199])
    r = oracle.rows(Q, K, V, dO, A, Bk, C, row_idx=idx, window=window, docs=starts)
    for key in ("O", "LSE", "D", "dQ", "alpha", "beta", "gQ", "gdO"):
        assert np.allclose(r[key], full[key][0][:, idx], atol=1e-12), key
    t = oracle.last_columns(Q, K, V, dO, ncols_tail=64, chunk=16, window=window, docs=starts)
    for key in ("dK", "dV"):
        assert np.allclose(t[key], full[key][0][:, -64:], atol=1e-12), key
    t = oracle.last_columns(Q, K, V, dO, A, Bk, C, ncols_tail=64, chunk=16, window=window,
                            docs=starts)
    for key in ("gK", "gV"):
        assert np.allclose(t[key], full[key][0][:, -64:], atol=1e-11), key

# ---------------------------------------------------------------- GProj
def test_gproj_projection_properties():
    Q, K = rnd((1, 2, 30, 8), 220), rnd((1, 2, 30, 8), 221)
    P = oracle.probs(Q, K)
    X = rnd(P.shape, 222) * (P > 0)
    Y = oracle.gproj_project(X, P)
    assert np.allclose(Y.sum(-1), 0.0, atol=1e-13)            # zero row mass
    assert np.allclose(oracle.gproj_project(Y, P), Y, atol=1e-13)  # idempotent
    V, dO = rnd((1, 2, 30, 8), 223), rnd((1, 2, 30, 8), 224)
    g = oracle.bwd(Q, K, V, dO)
    dS = P * (dO @ np.swapaxes(V, -1, -2) - g["D"][..., None])
    assert np.allclose(oracle.gproj_project(dS, P), dS, atol=1e-13)  # exact dS is fixed


def test_bf16_round_matches_torch_and_ties_to_even():
    x = rnd((4096,), 230, 100.0)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_round(x), ref)
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1)
    assert bf16_round(1 + 2 ** -8) == 1.0
    assert bf16_round(1 + 3 * 2 ** -8) == 1 + 2 ** -6


def test_gproj_model_large_key_regime():
    # The GProj page's failure: keys share a large mean and attention is near
    # one-hot.  Rounding dS to bf16 then gives a large median dQ error; the
    # projection brings it back to the fp32 level.  One head, N = 1024.
    N, d = 1024, 64
    rng = np.random.default_rng(240)
    u = rng.standard_normal(d)
    mu = 8.0 * u / np.linalg.norm(u)
    Q = 32.0 * rng.standard_normal((1, 1, N, d))
    K = rng.standard_normal((1, 1, N, d)) + mu
    V, dO = rng.standard_normal((1, 1, N, d)), rng.standard_normal((1, 1, N, d))
    Q, K, V, dO = (bf16_round(x) for x in (Q, K, V, dO))
    exact = oracle.bwd(Q, K, V, dO)["dQ"][0, 0]
    rows_ = np.arange(1, N)

    def median_rel(dq):
        e = np.linalg.norm(dq[0][rows_] - exact[rows_], axis=1)
        n = np.linalg.norm(exact[rows_], axis=1)
        return float(np.median(e[n > 0] / n[n > 0]))

    plain = median_rel(bwd_rounded(Q, K, V, dO, gproj=False))
    proj = median_rel(bwd_rounded(Q, K, V, dO, gproj=True))
    assert plain > 0.05
    assert proj < 0.01
    assert proj < plain / 10


def test_hutchinson_average_over_all_sign_vectors_is_the_hessian_diagonal():
    """Hutchinson's estimate diag(H) ~ mean of z o (H z) over random sign
    vectors z (the estimate second-order methods such as Sophia-H build on the
    FlashBoB page's Hessian-vector products) is exact when the mean runs over
    all 2^n sign vectors: E[z_i z_j] = [i = j].  Checked on a problem small
    enough to enumerate them (n = 3 N d = 6) against the diagonal from the
    Hessian's columns H e_j."""
    import itertools
    rng = np.random.default_rng(99)
    N, d = 2, 1
    Q, K, V, dO = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    n = 3 * N * d

    def hv(vec):
        vq, vk, vv = (vec[i * N * d:(i + 1) * N * d].reshape(1, 1, N, d) for i in range(3))
        r = oracle.hvp(Q, K, V, dO, vq, vk, vv, causal=False)
        return np.concatenate([r["HvQ"].ravel(), r["HvK"].ravel(), r["HvV"].ravel()])

    Hm = np.stack([hv(e) for e in np.eye(n)], axis=1)
    np.testing.assert_allclose(Hm, Hm.T, atol=1e-12)       # a Hessian is symmetric
    est = np.zeros(n)
    for signs in itertools.product((-1.0, 1.0), repeat=n):
        z = np.array(signs)
        est += z * hv(z)
    est /= 2 ** n
    np.testing.assert_allclose(est, np.diag(Hm), rtol=0, atol=1e-12)
    assert np.abs(np.diag(Hm)).max() > 1e-3                # not trivially zero
