"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle."""
import sys

import numpy as np
import torch

import fwd_bwd_double_amd as fbd
from synthetic import make_inputs, to_f64

# Tolerances on rel-L2 = |x - y|_2 / |y|_2 over the compared tensor, y from
# the oracle: fp32 inputs 1e-5; bf16 inputs with fp32 accumulation 2e-2 for
# O, LSE and the first-order gradients and 5e-2 for the BoB cotangents.
TOL_FP32 = 1e-5
TOL_BF16 = 2e-2
TOL_BF16_BOB = 5e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    n = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / n) if n > 0 else float(np.linalg.norm(x))


def to_gpu(x):
    return {k: v.cuda() for k, v in x.items()}


def f64(x):
    return {k: to_f64(v) for k, v in x.items()}


def tol(dtype, bob=False):
    if dtype == "fp32":
        return TOL_FP32
    return TOL_BF16_BOB if bob else TOL_BF16


def run_all(w, g, gproj=False, ops=("fwd", "bwd", "bob")):
    """Run the requested ops of workload w on GPU tensors g; returns a dict of
    CPU fp64 arrays."""
    say(f"[gpu] {w.name} B={w.B} H={w.H} N={w.N} dtype={w.dtype} causal={w.causal} "
        f"gproj={gproj} ops={ops}")
    out = {}
    o, lse = fbd.attn_fwd(g["q"], g["k"], g["v"], causal=w.causal, scale=w.scale)
    if "bwd" in ops:
        ws = torch.empty(fbd.bwd_workspace_bytes(w.B, w.H, w.N) // 4, device="cuda")
        dq, dk, dv = fbd.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=w.causal,
                                  scale=w.scale, gproj=gproj, workspace=ws)
    if "bob" in ops:
        wsb = torch.empty(fbd.bob_workspace_bytes(w.B, w.H, w.N) // 4, device="cuda")
        gq, gk, gv, gdo = fbd.attn_bob(g["q"], g["k"], g["v"], o, lse, g["do"], g["g_dq"],
                                       g["g_dk"], g["g_dv"], causal=w.causal, scale=w.scale,
                                       workspace=wsb)
    torch.cuda.synchronize()
    out["O"], out["LSE"] = to_f64(o), to_f64(lse)
    if "bwd" in ops:
        out["dQ"], out["dK"], out["dV"] = to_f64(dq), to_f64(dk), to_f64(dv)
        n = w.B * w.H * w.N
        wsn = to_f64(ws)
        out["D_bwd"] = wsn[:n].reshape(w.B, w.H, w.N)
        if gproj:
            out["r"] = wsn[n:2 * n].reshape(w.B, w.H, w.N)
    if "bob" in ops:
        out["gQ"], out["gK"], out["gV"], out["gdO"] = (to_f64(t) for t in (gq, gk, gv, gdo))
        n = w.B * w.H * w.N
        wsn = to_f64(wsb)
        out["D"] = wsn[:n].reshape(w.B, w.H, w.N)
        out["alpha"] = wsn[n:2 * n].reshape(w.B, w.H, w.N)
        out["beta"] = wsn[2 * n:3 * n].reshape(w.B, w.H, w.N)
    return out


def inputs(w, names=("q", "k", "v", "do", "g_dq", "g_dk", "g_dv")):
    x = make_inputs(w, names)
    return x, to_gpu(x), f64(x)
