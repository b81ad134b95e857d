"""The stored large-key tau fixture agrees with the oracle on a row sample."""
import json
import os

import numpy as np

import oracle
import synthetic
from synthetic import to_f64

HERE = os.path.dirname(os.path.abspath(__file__))


def load_tau():
    with open(os.path.join(HERE, "golden", "large_key_tau.json")) as f:
        return json.load(f)


def test_large_key_tau_is_near_one_hot_and_minimal():
    g = load_tau()
    tau = g["tau"]
    assert tau & (tau - 1) == 0
    rows = np.sort(np.random.default_rng(7).choice(np.arange(1, 16384), 256, replace=False))
    meds = {}
    for t in (tau // 2, tau):
        w = synthetic.WORKLOADS[3].with_(tau=float(t))
        x = synthetic.make_inputs(w, ("q", "k"))
        mp = oracle.max_prob(to_f64(x["q"]), to_f64(x["k"]), row_idx=rows,
                             heads=[(0, 0), (0, 5)])
        meds[t] = float(np.median(mp))
    assert meds[tau] > 0.95, meds
    assert meds[tau // 2] < 0.95, meds


def test_max_prob_against_brute_force_and_closed_form():
    """oracle.max_prob (which places the large-key workload) against its
    definition written as plain loops: P_ij = exp(c S_ij) / sum_{k <= i}
    exp(c S_ik) over the causal row, max over j; and against the closed form
    for Q = 0, where every visible key has the same weight: max_j P_ij =
    1 / (i + 1) causal, 1 / N without the mask."""
    import math
    rng = np.random.default_rng(11)
    B, H, N, d = 1, 2, 9, 64
    q = rng.standard_normal((B, H, N, d)) * 3
    k = rng.standard_normal((B, H, N, d))
    c = 0.125
    for causal in (True, False):
        mp = oracle.max_prob(q, k, causal=causal, scale=c)
        for h in range(H):
            for i in range(N):
                js = range(i + 1) if causal else range(N)
                s = [c * sum(q[0, h, i, t] * k[0, h, j, t] for t in range(d)) for j in js]
                e = [math.exp(x) for x in s]
                want = max(e) / sum(e)
                assert abs(mp[h, i] - want) <= 1e-13 * want
        z = oracle.max_prob(np.zeros_like(q), k, causal=causal, scale=c)
        want = 1.0 / (np.arange(N) + 1.0) if causal else np.full(N, 1.0 / N)
        np.testing.assert_allclose(z, np.broadcast_to(want, z.shape), rtol=1e-14)
    # selected rows and heads pick the same entries
    sel = oracle.max_prob(q, k, scale=c, heads=[(0, 1)], row_idx=[2, 7])
    np.testing.assert_array_equal(sel, oracle.max_prob(q, k, scale=c)[1:2, [2, 7]])
