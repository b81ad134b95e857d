"""Seeded random combinations of the supported forms against the fp64 oracle.

The other GPU tests fix one form at a time at a scale of 1/8.  Here each case
draws every option at once from its own seed, so that interactions are
exercised too: the dtype, batch, query and key/value heads (grouped-query and
multi-query), a ragged length, causal or not, a sliding window, packed
documents, a block-sparse mask (with or without its diagonal, so rows may be
left with no visible key), GProj, and a softmax scale that is not a power of
two.  Each case runs attn_fwd, attn_bwd and attn_bob on the same inputs (and,
for half the cases, attn_hvp with the cotangents as the direction) and holds
every output to the tolerance of its dtype, whole tensor and per row."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import (block_masks, check, check_lse_with_empty_rows, doc_starts, inputs, say,
                      tol)

pytestmark = pytest.mark.gpu

NCASES = 32


def draw(i):
    """The options of case i, from a generator seeded by i alone."""
    rng = np.random.default_rng(52000 + i)
    dtype = "bf16" if i % 2 == 0 else "fp32"
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 3]))
    grp = int(rng.choice([1, 2, 4]))
    # lengths around the 32-, 64- and 128-row tile edges, and plain ragged ones
    N = int(rng.choice([2, 31, 33, 64, 65, 127, 129, 255, 257])
            if rng.random() < 0.4 else rng.integers(2, 700))
    causal = bool(rng.random() < 0.75)
    window = int(rng.integers(2, N + 2)) if causal and rng.random() < 0.4 else 0
    mean_len = int(rng.integers(4, 200)) if causal and rng.random() < 0.3 else 0
    density = float(rng.uniform(0.3, 0.8)) if rng.random() < 0.3 else 0.0
    keep_diag = bool(rng.random() < 0.5)
    scale = float(rng.uniform(0.05, 0.22))
    gproj = bool(rng.random() < 0.5)
    hvp = bool(rng.random() < 0.5)
    return dict(dtype=dtype, B=B, H=Hkv * grp, Hkv=Hkv, N=N, causal=causal, window=window,
                mean_len=mean_len, density=density, keep_diag=keep_diag, scale=scale,
                gproj=gproj, hvp=hvp)


@pytest.mark.parametrize("i", range(NCASES))
def test_random_configuration(i):
    import fwd_bwd_double_amd as fbd
    c = draw(i)
    say(f"[gpu] random case {i}: {c}")
    B, H, Hkv, N, dtype = c["B"], c["H"], c["Hkv"], c["N"], c["dtype"]
    w = synthetic.Workload(f"random-{i}", B, H, N, 64, dtype, 53000 + i, causal=c["causal"],
                           qkv_std=1.0)
    x, g, a = inputs(w)
    for n in ("k", "v", "g_dk", "g_dv"):
        g[n] = g[n][:, :Hkv].contiguous()
        a[n] = a[n][:, :Hkv]
    docs = doc_starts(B, N, 54000 + i, c["mean_len"]) if c["mean_len"] else None
    bm = block_masks(B, N, 55000 + i, c["density"], c["keep_diag"]) if c["density"] else None
    ds = torch.from_numpy(docs.astype(np.int32)).cuda() if docs is not None else None
    bmt = torch.from_numpy(bm).cuda() if bm is not None else None
    opts = dict(causal=c["causal"], scale=c["scale"], window=c["window"], doc_start=ds,
                block_mask=bmt)

    o, lse = fbd.attn_fwd(g["q"], g["k"], g["v"], **opts)
    dq, dk, dv = fbd.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], gproj=c["gproj"], **opts)
    gq, gk, gv, gdo = fbd.attn_bob(g["q"], g["k"], g["v"], o, lse, g["do"], g["g_dq"],
                                   g["g_dk"], g["g_dv"], gproj=c["gproj"], **opts)
    h = None
    if c["hvp"]:
        h = fbd.attn_hvp(g["q"], g["k"], g["v"], g["do"], g["g_dq"], g["g_dk"], g["g_dv"],
                         gproj=c["gproj"], **opts)
    torch.cuda.synchronize()

    ref = oracle.bob_gqa(a["q"], a["k"], a["v"], a["do"], a["g_dq"], a["g_dk"], a["g_dv"],
                         causal=c["causal"], scale=c["scale"], with_bwd=True,
                         window=c["window"], docs=docs, block_mask=bm)
    t1, t2 = tol(dtype), tol(dtype, bob=True)
    f64 = synthetic.to_f64
    got = {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv, "gQ": gq, "gK": gk, "gV": gv,
           "gdO": gdo}
    if h is not None:
        got.update({"hvp O": h["O"], "hvp LSE": h["LSE"], "hvp dQ": h["dQ"], "hvp dK": h["dK"],
                    "hvp dV": h["dV"], "hvp gQ": h["Hv_q"], "hvp gK": h["Hv_k"],
                    "hvp gV": h["Hv_v"], "hvp gdO": h["Hv_do"]})
    for name, t in got.items():
        key = name.split()[-1]
        assert t.shape == (B, H if key not in ("dK", "dV", "gK", "gV") else Hkv, N) + (
            () if key == "LSE" else (64,)), (name, tuple(t.shape))
        if key == "LSE":
            check_lse_with_empty_rows(f64(t), ref["LSE"], t1)
        else:
            check(name, f64(t), ref[key], t2 if key.startswith("g") else t1)
