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


# Per-row bound beside the whole-tensor rel-L2.  One wholly wrong row of an
# N x d tensor moves the whole-tensor rel-L2 by only about 1/sqrt(N), so each
# row is also held to its own relative error
#     e_i = |x_i - y_i|_2 / max(|y_i|_2, ROW_FLOOR * rms_i |y_i|_2)
# with a limit of ROW_FACTOR times the tensor's tolerance.  A row is the last
# axis of a (.., N, 64) tensor, one element of a row-statistic array.  The
# floor keeps rows whose exact value is (nearly) zero -- the first query's dQ,
# the one-key rows of BoB -- from being measured against their own tiny norm:
# there the error is the rounding of terms of typical size, not of the row.
# The BoB row pass forms g_Q from two row scalars applied after the row is
# complete (X - alpha Z - beta Y, each a sum of bf16-rounded products), so on
# rows with few visible keys those terms are much larger than g_Q and cancel:
# measured up to 0.07 rms there (bf16), against about 1 rms for a row that is
# wholly wrong -- the floor of rms / 2 and the limit of 5 tol (0.25 for BoB)
# separate the two by a factor of two on each side.  An all-zero reference
# (the exact gradients of one-key inputs) is compared in absolute terms, as
# rel_l2 does.
ROW_FACTOR = 5.0
ROW_FLOOR = 0.5


def row_errors(x, y):
    """Relative error of every row (see ROW_FACTOR), as a flat array."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if y.ndim >= 1 and y.shape[-1] == 64:
        err = np.linalg.norm(x - y, axis=-1).ravel()
        ref = np.linalg.norm(y, axis=-1).ravel()
    else:
        err = np.abs(x - y).ravel()
        ref = np.abs(y).ravel()
    if ref.size == 0:
        return err
    floor = ROW_FLOOR * float(np.sqrt(np.mean(ref ** 2)))
    if floor == 0.0:
        return err
    den = np.maximum(ref, floor)
    return np.where(den > 0, err / np.where(den > 0, den, 1.0), np.where(err > 0, np.inf, 0.0))


def check(name, got, ref, t):
    """Whole-tensor rel-L2 <= t and every row's relative error <= ROW_FACTOR t
    (row_errors: a single wrong row cannot hide under the tensor norm)."""
    e = rel_l2(got, ref)
    re = row_errors(got, ref)
    worst = float(re.max()) if re.size else 0.0
    say(f"    {name}: rel-L2 {e:.3e} (tol {t:.0e}); worst row {worst:.3e} at "
        f"{int(re.argmax()) if re.size else -1} (limit {ROW_FACTOR * t:.0e})")
    assert np.all(np.isfinite(got)), name
    assert e <= t, (name, e, t)
    assert worst <= ROW_FACTOR * t, (name, "worst row", worst, ROW_FACTOR * t)
    return e


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


def doc_starts(B, N, seed, mean_len):
    """Seeded packed-document layout: (B, N) int first position of each row's
    document, document lengths ~ geometric with the given mean (some of
    length 1)."""
    rng = np.random.default_rng(seed)
    out = np.zeros((B, N), dtype=np.int64)
    for b in range(B):
        i = 0
        while i < N:
            n = int(min(N - i, rng.geometric(1.0 / mean_len)))
            out[b, i:i + n] = i
            i += n
    return out


def block_masks(B, N, seed, density, keep_diag):
    """Seeded (B, nb, nb) uint8 block mask, nb = ceil(N / 128): each block kept
    with the given probability; the diagonal blocks kept when asked."""
    rng = np.random.default_rng(seed)
    nb = (N + 127) // 128
    m = (rng.random((B, nb, nb)) < density).astype(np.uint8)
    if keep_diag:
        m[:, np.arange(nb), np.arange(nb)] = 1
    return m


def check_lse_with_empty_rows(got, ref, t):
    """Rows with no visible key have LSE = -inf on both sides; the others are
    compared by rel-L2."""
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), "empty rows differ"
    say(f"    empty rows: {int(empty.sum())}")
    check("LSE", got[~empty], ref[~empty], t)
