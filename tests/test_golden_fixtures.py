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
