"""Pins of the oracle's forward pass (CPU only).

Each test pins the dense fp64 forward to something other than itself: closed
forms, invariances of softmax attention, the pages' tiled online recurrence,
and torch's own attention and softmax routines."""
import math

import numpy as np
import pytest
import torch

import oracle



def rnd(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def test_probability_rows_sum_to_one_and_respect_mask():
    Q, K = rnd((2, 3, 37, 8), 1), rnd((2, 3, 37, 8), 2)
    P = oracle.probs(Q, K, causal=True)
    assert np.allclose(P.sum(-1), 1.0, atol=1e-13)
    iu = np.triu_indices(37, k=1)
    assert np.all(P[..., iu[0], iu[1]] == 0.0)
    assert np.all(P[..., np.arange(37), np.arange(37)] > 0.0)
    Pn = oracle.probs(Q, K, causal=False)
    assert np.allclose(Pn.sum(-1), 1.0, atol=1e-13)
    assert np.all(Pn > 0)


def test_hand_derived_two_by_two():
    # d = 1, c = 1, q = [2, 1], k = [0, ln 3], v = [4, 8].
    # Row 0 sees only key 0: P = [1, 0], O_0 = v_0 = 4, LSE_0 = q0 k0 = 0.
    # Row 1: scores q1*k = [0, ln 3]  ->  P = [1/4, 3/4];  O_1 = 4/4 + 3*8/4 = 7;
    # LSE_1 = ln(e^0 + e^{ln 3}) = ln 4.
    Q = np.array([2.0, 1.0]).reshape(1, 1, 2, 1)
    K = np.array([0.0, math.log(3.0)]).reshape(1, 1, 2, 1)
    V = np.array([4.0, 8.0]).reshape(1, 1, 2, 1)
    O, L = oracle.fwd(Q, K, V, causal=True, scale=1.0)
    assert O[0, 0, 0, 0] == pytest.approx(4.0, abs=1e-15)
    assert L[0, 0, 0] == pytest.approx(0.0, abs=1e-15)
    assert O[0, 0, 1, 0] == pytest.approx(7.0, rel=1e-14)
    assert L[0, 0, 1] == pytest.approx(math.log(4.0), rel=1e-14)


def test_single_token_closed_form():
    Q, K, V = rnd((2, 2, 1, 5), 3), rnd((2, 2, 1, 5), 4), rnd((2, 2, 1, 5), 5)
    c = 0.3
    O, L = oracle.fwd(Q, K, V, causal=True, scale=c)
    assert np.allclose(O, V, atol=1e-15)
    assert np.allclose(L, c * np.einsum("bhnd,bhnd->bhn", Q, K), atol=1e-14)


def test_zero_queries_give_prefix_means():
    N = 23
    Q = np.zeros((1, 2, N, 4))
    K, V = rnd((1, 2, N, 4), 6), rnd((1, 2, N, 4), 7)
    O, L = oracle.fwd(Q, K, V, causal=True)
    means = np.cumsum(V, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.allclose(O, means, atol=1e-14)
    assert np.allclose(L, np.log(np.arange(1, N + 1))[None, None, :], atol=1e-14)
    On, Ln = oracle.fwd(Q, K, V, causal=False)
    assert np.allclose(On, V.mean(axis=2, keepdims=True), atol=1e-14)
    assert np.allclose(Ln, math.log(N), atol=1e-14)


def test_constant_values_pass_through():
    Q, K = rnd((1, 2, 19, 6), 8, 3.0), rnd((1, 2, 19, 6), 9, 3.0)
    v = rnd((6,), 10)
    V = np.broadcast_to(v, (1, 2, 19, 6)).copy()
    O, _ = oracle.fwd(Q, K, V, causal=True)
    assert np.allclose(O, V, atol=1e-13)


def test_key_shift_moves_only_lse():
    # Adding one vector delta to every key adds c q_i.delta to row i's scores:
    # P and O are unchanged, LSE_i moves by exactly c q_i.delta.
    Q, K, V = rnd((1, 3, 29, 8), 11), rnd((1, 3, 29, 8), 12), rnd((1, 3, 29, 8), 13)
    delta = rnd((8,), 14, 2.0)
    c = 1 / math.sqrt(8)
    O1, L1 = oracle.fwd(Q, K, V)
    O2, L2 = oracle.fwd(Q, K + delta, V)
    assert np.allclose(O1, O2, atol=1e-12)
    assert np.allclose(L2 - L1, c * Q @ delta, atol=1e-12)


def test_causal_prefix_property():
    Q, K, V = rnd((1, 2, 40, 8), 15), rnd((1, 2, 40, 8), 16), rnd((1, 2, 40, 8), 17)
    O, L = oracle.fwd(Q, K, V)
    Op, Lp = oracle.fwd(Q[:, :, :17], K[:, :, :17], V[:, :, :17])
    assert np.allclose(O[:, :, :17], Op, atol=1e-14)
    assert np.allclose(L[:, :, :17], Lp, atol=1e-14)


def test_noncausal_key_permutation_invariance():
    Q, K, V = rnd((1, 1, 21, 8), 18), rnd((1, 1, 21, 8), 19), rnd((1, 1, 21, 8), 20)
    perm = np.random.default_rng(21).permutation(21)
    O1, L1 = oracle.fwd(Q, K, V, causal=False)
    O2, L2 = oracle.fwd(Q, K[:, :, perm], V[:, :, perm], causal=False)
    assert np.allclose(O1, O2, atol=1e-13) and np.allclose(L1, L2, atol=1e-13)


def test_max_entry_is_exactly_one_before_normalising():
    # Subtracting the max before scaling makes the largest unnormalised weight
    # exactly exp(0) = 1, so l_i >= 1 and LSE_i >= c m_i with equality only
    # for a single visible key.
    Q, K = rnd((1, 1, 50, 8), 22, 30.0), rnd((1, 1, 50, 8), 23, 30.0)
    V = rnd((1, 1, 50, 8), 24)
    _, L = oracle.fwd(Q, K, V)
    S = Q[0, 0] @ K[0, 0].T
    m = np.array([S[i, : i + 1].max() for i in range(50)])
    c = 1 / math.sqrt(8)
    assert L[0, 0, 0] == c * m[0]
    assert np.all(L[0, 0] - c * m >= 0.0)


@pytest.mark.parametrize("Br,Bc", [(16, 16), (8, 32), (32, 8), (7, 5), (64, 64)])
def test_online_recurrence_equals_two_pass(Br, Bc):
    Q, K, V = rnd((2, 2, 45, 16), 25, 2.0), rnd((2, 2, 45, 16), 26, 2.0), rnd((2, 2, 45, 16), 27)
    for causal in (True, False):
        O, L = oracle.fwd(Q, K, V, causal=causal)
        Ot, Lt = oracle.online_fwd(Q, K, V, causal=causal, Br=Br, Bc=Bc)
        assert np.allclose(O, Ot, atol=1e-12, rtol=0)
        assert np.allclose(L, Lt, atol=1e-12, rtol=0)


def test_against_torch_attention_fp64():
    Q, K, V = rnd((2, 3, 33, 16), 28), rnd((2, 3, 33, 16), 29), rnd((2, 3, 33, 16), 30)
    tq, tk, tv = (torch.from_numpy(x) for x in (Q, K, V))
    for causal in (True, False):
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
        O, L = oracle.fwd(Q, K, V, causal=causal)
        assert np.allclose(O, ref.numpy(), atol=1e-13)
        s = (tq @ tk.transpose(-1, -2)) / 4.0
        if causal:
            s = s.masked_fill(torch.ones(33, 33, dtype=torch.bool).triu(1), float("-inf"))
        assert np.allclose(L, torch.logsumexp(s, dim=-1).numpy(), atol=1e-13)


def test_chunking_does_not_change_results():
    Q, K, V = rnd((1, 2, 70, 8), 31), rnd((1, 2, 70, 8), 32), rnd((1, 2, 70, 8), 33)
    a = oracle.fwd(Q, K, V, chunk=1024)
    b = oracle.fwd(Q, K, V, chunk=9)
    assert np.allclose(a[0], b[0], atol=1e-14) and np.allclose(a[1], b[1], atol=1e-14)
