"""The Hessian-vector product call with bf16 operands and the gradient
requested runs one row pass for the first backward and BoB together: BoB's
row pass sums R(dS) K and R(P) K, which are the backward row pass's dQ terms.
These tests hold that call to the separate attn_fwd, attn_bwd and attn_bob
calls on the same inputs, every output bit for bit:

- O, LSE, dQ, dK and dV (the same products over the same bf16 values,
  accumulated in the same order; the backward's column pass reads the same
  D, r and -LSE log2(e));
- Hv_Q, Hv_K, Hv_V and Hv_dO (attn_bob's row pass forms the same sums, and
  its column pass reads the same alpha and kappa), with the same gproj,
  which also projects g_Q's and g_dO's residual row sums;

and Hv_Q, attn_bob's g_Q and dQ within the BoB and first-order tolerances of
the fp64 oracle where the oracle is run.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import block_masks, check, doc_starts, inputs, say

pytestmark = pytest.mark.gpu

CASES = {
    # name: B, H, Hkv, N, causal, window, mean_len, density, gproj, oracle
    "one-token": (2, 3, 3, 1, True, 0, 0, 0.0, True, True),
    "causal": (2, 3, 3, 300, True, 0, 0, 0.0, True, True),
    "causal-no-gproj": (2, 3, 3, 300, True, 0, 0, 0.0, False, True),
    "full": (2, 3, 3, 200, False, 0, 0, 0.0, True, True),
    "gqa-window": (2, 4, 2, 333, True, 100, 0, 0.0, True, True),
    "docs": (2, 4, 4, 300, True, 0, 60, 0.0, True, True),
    "block-sparse": (2, 2, 2, 1000, True, 0, 0, 0.5, True, True),
    # diagonal blocks dropped too: rows with no visible key (LSE = -inf)
    "block-sparse-empty-rows": (1, 2, 2, 700, True, 0, 0, -0.4, True, True),
    # the backward's row pass takes 8-wave (256-row) blocks from N = 65536
    # and a partly filled last block here; the fused pass keeps 128-row blocks
    "long": (1, 2, 2, 65613, True, 0, 0, 0.0, True, False),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", list(CASES))
def test_fused_hvp_matches_separate_calls(case):
    import fwd_bwd_double_amd as fbd
    B, H, Hkv, N, causal, window, mean_len, density, gproj, with_oracle = CASES[case]
    w = synthetic.Workload(f"hvp-fused-{case}", B, H, N, 64, "bf16", 7100 + N + H + Hkv,
                           causal=causal, qkv_std=0.5)
    x, g, a = inputs(w)
    for n in ("k", "v", "g_dk", "g_dv"):
        g[n] = g[n][:, :Hkv].contiguous()
        a[n] = a[n][:, :Hkv]
    docs = doc_starts(B, N, 77 + N, mean_len) if mean_len else None
    # a negative density keeps each block with probability |density| and
    # drops the diagonal blocks' guarantee
    bm = block_masks(B, N, 88 + N, abs(density), density > 0) if density else None
    masks = dict(window=window,
                 doc_start=torch.from_numpy(docs.astype(np.int32)).cuda() if docs is not None else None,
                 block_mask=torch.from_numpy(bm).cuda() if bm is not None else None)
    say(f"[gpu] fused attn_hvp vs separate calls: {case} B={B} H={H} Hkv={Hkv} N={N} "
        f"causal={causal} window={window} mean_len={mean_len} density={density} gproj={gproj}")
    q, k, v, do = g["q"], g["k"], g["v"], g["do"]
    vq, vk, vv = g["g_dq"], g["g_dk"], g["g_dv"]
    ws_h = torch.empty(fbd.load().attn_hvp_ex_workspace_bytes(B, H, Hkv, N) // 4, device="cuda")
    ws_b = torch.empty(fbd.bob_ex_workspace_bytes(B, H, Hkv, N) // 4, device="cuda")
    ws_g = torch.empty(fbd.bwd_ex_workspace_bytes(B, H, Hkv, N) // 4, device="cuda")
    r = fbd.attn_hvp(q, k, v, do, vq, vk, vv, causal=causal, scale=w.scale, gproj=gproj,
                     workspace=ws_h, **masks)
    o, lse = fbd.attn_fwd(q, k, v, causal=causal, scale=w.scale, **masks)
    dq, dk, dv = fbd.attn_bwd(q, k, v, o, lse, do, causal=causal, scale=w.scale, gproj=gproj,
                              workspace=ws_g, **masks)
    gq, gk, gv, gdo = fbd.attn_bob(q, k, v, o, lse, do, vq, vk, vv, causal=causal,
                                   scale=w.scale, workspace=ws_b, gproj=gproj, **masks)
    torch.cuda.synchronize()
    # the fp32 row states both row passes leave behind (D, alpha, beta,
    # -LSE log2(e), -kappa), and the backward's GProj row sums r: any rounding
    # difference shows here, before a bf16 rounding can hide it
    bhn = B * H * N
    for i, name in enumerate(("D", "alpha", "beta", "-LSE log2(e)", "-kappa")):
        same = torch.equal(ws_h[i * bhn:(i + 1) * bhn], ws_b[i * bhn:(i + 1) * bhn])
        say(f"    row state {name}: bit-identical {same}")
        assert same, name
    if gproj:
        same = torch.equal(ws_h[5 * bhn:6 * bhn], ws_g[bhn:2 * bhn])
        say(f"    GProj row sums r: bit-identical {same}")
        assert same, "r"
    for name, got, ref in (("O", r["O"], o), ("LSE", r["LSE"], lse), ("dQ", r["dQ"], dq),
                           ("dK", r["dK"], dk), ("dV", r["dV"], dv), ("Hv_q", r["Hv_q"], gq),
                           ("Hv_k", r["Hv_k"], gk), ("Hv_v", r["Hv_v"], gv),
                           ("Hv_do", r["Hv_do"], gdo)):
        same = torch.equal(got, ref)
        say(f"    {name}: bit-identical {same}")
        assert same, name
    f64 = synthetic.to_f64
    if with_oracle:
        ref = oracle.bob_gqa(a["q"], a["k"], a["v"], a["do"], a["g_dq"], a["g_dk"], a["g_dv"],
                             causal=causal, window=window, docs=docs, block_mask=bm)
        check("Hv_q against the oracle", f64(r["Hv_q"]), ref["gQ"], 5e-2)
        check("attn_bob gQ against the oracle", f64(gq), ref["gQ"], 5e-2)
    else:
        # seeded rows, the first row and the last (partly filled) blocks
        rng = np.random.default_rng(7101)
        rows = np.unique(np.concatenate([rng.choice(np.arange(N), 250, replace=False),
                                         [0, 1, 127, 128, N - 78, N - 1]]))
        ref = oracle.rows(a["q"], a["k"], a["v"], a["do"], a["g_dq"], a["g_dk"], a["g_dv"],
                          row_idx=rows, causal=causal, scale=w.scale)
        check("Hv_q rows against the oracle", f64(r["Hv_q"])[0][:, rows], ref["gQ"], 5e-2)
        check("attn_bob gQ rows against the oracle", f64(gq)[0][:, rows], ref["gQ"], 5e-2)
        check("dQ rows against the oracle", f64(r["dQ"])[0][:, rows], ref["dQ"], 2e-2)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tau_key", ["tau", "tau_strict"])
def test_gproj_projection_of_bob_gq_in_the_large_key_regime(tau_key):
    """The large-key regime (keys shifted by one shared vector of norm 8,
    queries scaled by the power of two that makes most rows near one-hot,
    from the committed oracle fixture), B1 H2 N1024 against the fp64 oracle on
    full tensors.  There g_Q is formed from large terms that nearly cancel, and
    the residual row sum of its bf16 key weights carries a false multiple of
    the keys' large mean into it (the GProj page's mechanism, in BoB's row
    pass); g_dO, whose weights of V sum to zero too, the same along O.
    Asserted:
      * with the projections (attn_bob with gproj, and attn_hvp with gproj,
        whose fused pass gives the same g_Q and g_dO bit for bit): g_Q and
        g_dO within the BoB bound of the oracle, row by row;
      * without them (attn_bob): g_Q's worst row at least 3 times further
        off, g_dO's further off;
      * the fused call's other outputs bit for bit equal to the separate
        calls'; g_K, g_V (unchanged by the flag) within the BoB bound as
        whole tensors, worst rows printed."""
    import json
    import os
    import fwd_bwd_double_amd as fbd
    from gpu_util import rel_l2, row_errors
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "large_key_tau.json")))
    w = synthetic.Workload(f"bob-large-key-{tau_key}", 1, 2, 1024, 64, "bf16", 7300,
                           qkv_std=1.0, do_std=1.0, cot_std=1.0, mean_norm=8.0,
                           tau=float(gold[tau_key]))
    x, g, a = inputs(w)
    say(f"[gpu] BoB g_Q projection, large-key regime: tau={w.tau} B1 H2 N1024")
    q, k, v, do = g["q"], g["k"], g["v"], g["do"]
    vq, vk, vv = g["g_dq"], g["g_dk"], g["g_dv"]
    r = fbd.attn_hvp(q, k, v, do, vq, vk, vv, causal=True, scale=w.scale, gproj=True)
    o, lse = fbd.attn_fwd(q, k, v, causal=True, scale=w.scale)
    dq, dk, dv = fbd.attn_bwd(q, k, v, o, lse, do, causal=True, scale=w.scale, gproj=True)
    gq, gk, gv, gdo = fbd.attn_bob(q, k, v, o, lse, do, vq, vk, vv, causal=True,
                                   scale=w.scale, gproj=True)
    gq0, gk0, gv0, gdo0 = fbd.attn_bob(q, k, v, o, lse, do, vq, vk, vv, causal=True,
                                       scale=w.scale)
    torch.cuda.synchronize()
    for name, got, ref in (("O", r["O"], o), ("LSE", r["LSE"], lse), ("dQ", r["dQ"], dq),
                           ("dK", r["dK"], dk), ("dV", r["dV"], dv), ("Hv_q", r["Hv_q"], gq),
                           ("Hv_k", r["Hv_k"], gk), ("Hv_v", r["Hv_v"], gv),
                           ("Hv_do", r["Hv_do"], gdo),
                           ("g_K without projection", gk0, gk), ("g_V", gv0, gv)):
        assert torch.equal(got, ref), name
    say("    the projections change g_Q and g_dO only; the fused call's other outputs "
        "equal the separate calls' bit for bit")
    f64 = synthetic.to_f64
    ref = oracle.bob(a["q"], a["k"], a["v"], a["do"], a["g_dq"], a["g_dk"], a["g_dv"],
                     causal=True, scale=w.scale)
    check("Hv_q (fused, projected) against the oracle", f64(r["Hv_q"]), ref["gQ"], 5e-2)
    check("attn_bob g_Q (projected) against the oracle", f64(gq), ref["gQ"], 5e-2)
    check("Hv_do (fused, projected) against the oracle", f64(r["Hv_do"]), ref["gdO"], 5e-2)
    check("attn_bob g_dO (projected) against the oracle", f64(gdo), ref["gdO"], 5e-2)
    w0 = float(row_errors(f64(gq0), ref["gQ"]).max())
    w1 = float(row_errors(f64(gq), ref["gQ"]).max())
    say(f"    attn_bob g_Q without the projection: rel-L2 {rel_l2(f64(gq0), ref['gQ']):.3e}, "
        f"worst row {w0:.3e} ({w0 / w1:.1f} x the projected)")
    assert w0 >= 3 * w1, (w0, w1)
    o0 = float(row_errors(f64(gdo0), ref["gdO"]).max())
    o1 = float(row_errors(f64(gdo), ref["gdO"]).max())
    say(f"    attn_bob g_dO without the projection: rel-L2 "
        f"{rel_l2(f64(gdo0), ref['gdO']):.3e}, worst row {o0:.3e} ({o0 / o1:.1f} x the projected)")
    assert o0 > o1, (o0, o1)
    for key, got in (("g_K", gk), ("g_V", gv)):
        e = rel_l2(f64(got), ref[key[0] + key[2:]])
        say(f"    {key}: rel-L2 {e:.3e} (tol 5e-02), worst row "
            f"{float(row_errors(f64(got), ref[key[0] + key[2:]]).max()):.3e}")
        assert e <= 5e-2, key
