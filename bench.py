"""Throughput of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  attn_fwd -> attn_bwd (row pass, column pass; GProj on) -> attn_bob (row
  pass, column pass), causal, on the BoB workload B=4, H=12, N=4096, d=64,
  bf16 inputs with fp32 accumulation (Q, K, V, dO ~ 0.5 N(0,1), cotangents
  ~ N(0,1), seeded).  Inputs are resident in device memory before timing.

Prints ONE JSON line.  `value` is the step's model TFLOP/s under the FLOP
convention (per unmasked causal (query, key) pair and head: forward 4d,
backward 10d, backward-over-backward 38d); `roofline` is the dominant kernel's
executed contraction FLOPs per launch over its HIP-event-timed duration against
the bf16 dense MFMA peak; `cpu_baseline` is the fp64 oracle timed on a bounded
sample of the same workload on this host.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]

`--fp8` times the FP8 forward (rotated quantisation pre-pass + E4M3 forward)
on the same workload instead of the step, one JSON line.

`--sweep` instead times each operation separately over sequence lengths
1k .. 256k (H=12, d=64, B = max(1, 16384/N), causal, GProj on), the other
workload shapes and the extended forms (grouped-query heads, a sliding window,
packed documents, a block-sparse mask, the HVP call), printing one JSON line
per case; it includes the FP8 forward (quantisation pre-pass and the forward
on the codes, against the fp8 peak).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (published)
HBM_PEAK_GBS = 8000.0
METRIC = "attn fwd/bwd/BoB TFLOP/s & % bf16 MFMA peak, GPT-2S head shape, N≤262k"

# Contraction units (N x N x d products, 2d FLOP per unmasked pair) executed
# by each kernel; GProj adds one unit to each backward pass.
UNITS = {"fwd": 2, "bwd_row": 4, "bwd_col": 5, "bob_row": 11, "bob_col": 8}
# FLOP convention per unmasked pair, in units of d
CONV = {"fwd": 4, "bwd": 10, "bob": 38}
# Algorithmic HBM bytes per launch as (tensors, row arrays): (B, H, N, d)
# tensors read or written once, and (B, H, N) fp32 arrays.  fwd: Q, K, V, O
# and LSE.  bwd_row: Q, K, V, O, dO, dQ; LSE in, D, r, -LSE log2(e) out.
# bwd_col: Q, K, V, dO, dK, dV; -LSE log2(e), D, r.  bob_row: Q, K, V, O, dO
# and the three cotangents in, g_Q and g_dO out; LSE in, D, alpha, beta,
# -LSE log2(e), -kappa out.  bob_col: Q, K, V, dO, g_dQ, g_dK, g_dV in, g_K,
# g_V out; -LSE log2(e), D, alpha, -kappa.
ALG_BYTES = {"fwd": (4, 1), "bwd_row": (6, 4), "bwd_col": (6, 3), "bob_row": (10, 6),
             "bob_col": (9, 4)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=48,
                   help="heads of the workload the oracle baseline runs on")
    p.add_argument("--sweep", action="store_true",
                   help="time fwd, bwd and BoB separately over N = 1k .. 256k and the other "
                        "workload shapes (one JSON line per case) instead of the step")
    p.add_argument("--case", default=None,
                   help="with --sweep: only the named cases (comma-separated), e.g. "
                        "sweep-N262144 for a counter run on the longest sequence")
    p.add_argument("--fp8", action="store_true",
                   help="time the FP8 forward (rotated quantisation pre-pass + E4M3 forward) on "
                        "the step's workload instead of the step (one JSON line)")
    p.add_argument("--workload", default="bob-B4H12N4096",
                   choices=["bob-B4H12N4096", "gpt2s-layer-B8H12N1024"],
                   help="workload the step runs on: the BoB workload (the reported line) or "
                        "the GPT-2-Small layer shape, where each kernel is short and the "
                        "memory traffic matters (for counter runs)")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="first run one device-to-device copy of this many MiB (a plain copy "
                        "kernel of known size, to calibrate memory counters)")
    return p.parse_args()


def main():
    args = parse()
    if args.sweep and args.gpus == 1:
        return sweep(args.case)
    if args.fp8 and args.gpus == 1:
        return fp8_bench(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fwd_bwd_double_amd as fbd
    import synthetic

    w = {x.name: x for x in synthetic.WORKLOADS.values()}[args.workload]
    B, H, N, d = w.B, w.H, w.N, w.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = synthetic.make_inputs(w)
    g = {k: v.to(dev) for k, v in x.items()}
    q, k, v, do = g["q"], g["k"], g["v"], g["do"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    gq, gk, gv, gdo = (torch.empty_like(q) for _ in range(4))
    ws_b = torch.empty(fbd.bwd_workspace_bytes(B, H, N) // 4, device=dev)
    ws_bb = torch.empty(fbd.bob_workspace_bytes(B, H, N) // 4, device=dev)
    sc = w.scale

    names = ["fwd", "bwd_row", "bwd_col", "bob_row", "bob_col"]

    def step(ev):
        ev[0].record()
        fbd.attn_fwd(q, k, v, causal=True, scale=sc, out=o, lse=lse)
        ev[1].record()
        fbd.attn_bwd(q, k, v, o, lse, do, causal=True, scale=sc, gproj=True, workspace=ws_b,
                     outs=(dq, dk, dv), passes=1)
        ev[2].record()
        fbd.attn_bwd(q, k, v, o, lse, do, causal=True, scale=sc, gproj=True, workspace=ws_b,
                     outs=(dq, dk, dv), passes=2)
        ev[3].record()
        fbd.attn_bob(q, k, v, o, lse, do, g["g_dq"], g["g_dk"], g["g_dv"], causal=True,
                     scale=sc, workspace=ws_bb, outs=(gq, gk, gv, gdo), passes=1)
        ev[4].record()
        fbd.attn_bob(q, k, v, o, lse, do, g["g_dq"], g["g_dk"], g["g_dv"], causal=True,
                     scale=sc, workspace=ws_bb, outs=(gq, gk, gv, gdo), passes=2)
        ev[5].record()

    if args.copy_mb > 0:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)]
           for _ in range(max(args.steps, 1))]
    for _ in range(args.warmup):
        step(evs[0])
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr,
          flush=True)
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    kern_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs[:args.steps]]))
               for i, n in enumerate(names)}

    pairs = B * H * N * (N + 1) / 2          # unmasked causal pairs over all heads
    unit = 2 * d * pairs                     # FLOP of one N x N x d contraction unit
    step_flop = sum(CONV.values()) * d * pairs
    value = step_flop / (ms_step * 1e-3) / 1e12
    per_kernel = {n: {"ms": kern_ms[n],
                      "executed_tflops": UNITS[n] * unit / (kern_ms[n] * 1e-3) / 1e12}
                  for n in names}
    # algorithmic bytes: one touch of every input and output, in units of one
    # (B, H, N, d) tensor (t) and one (B, H, N) fp32 row-statistic array (r)
    t_b, r_b = B * H * N * d * x["q"].element_size(), B * H * N * 4
    alg_bytes = {n: a * t_b + b * r_b for n, (a, b) in ALG_BYTES.items()}
    for n in names:
        per_kernel[n]["frac_mfma_peak"] = per_kernel[n]["executed_tflops"] / PEAK_BF16_TFLOPS
        per_kernel[n]["alg_bytes"] = alg_bytes[n]
        per_kernel[n]["alg_gbs"] = alg_bytes[n] / (kern_ms[n] * 1e-3) / 1e9
        per_kernel[n]["frac_hbm_peak"] = per_kernel[n]["alg_gbs"] / HBM_PEAK_GBS
    op_ms = {"fwd": kern_ms["fwd"], "bwd": kern_ms["bwd_row"] + kern_ms["bwd_col"],
             "bob": kern_ms["bob_row"] + kern_ms["bob_col"]}
    per_op = {op: {"ms": op_ms[op],
                   "conv_tflops": CONV[op] * d * pairs / (op_ms[op] * 1e-3) / 1e12}
              for op in op_ms}
    for op in per_op:
        per_op[op]["frac_mfma_peak"] = per_op[op]["conv_tflops"] / PEAK_BF16_TFLOPS
    dom = max(names, key=lambda n: kern_ms[n])
    ach = per_kernel[dom]["executed_tflops"]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                "traffic": stored_traffic(dom, w.name), "traffic_unit": "bytes per launch",
                "flop_per_launch": UNITS[dom] * unit}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, w, min(args.cpu_heads, B * H))

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": True,
                   "gproj": True, "step": "fwd + bwd(row, col) + bob(row, col)",
                   "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "per_kernel": per_kernel, "per_op": per_op,
        "peak_mem_gb": torch.cuda.max_memory_allocated() / 1e9,
    }
    print(json.dumps(line), flush=True)


def fp8_bench(args):
    """The FP8 forward on the step's workload (B4 H12 N4096, causal, bf16 Q, K,
    V from its seeded generator, rotation signs from its seed): W untimed then
    K timed repetitions of the rotated quantisation pre-pass followed by the
    E4M3 forward, each launch bracketed by HIP events on the launch stream.
    `value` is the forward's model TFLOP/s (4d per unmasked pair) over the
    whole (pre-pass + forward); `per_op` gives each part, the forward against
    the 5 PFLOP/s fp8 peak and the pre-pass in GB/s of its algorithmic bytes
    (11 per element: Q, K, V read, V read again for its column maxima, codes
    written)."""
    import numpy as np
    import torch

    import fwd_bwd_double_amd as fbd
    import synthetic

    w = {x.name: x for x in synthetic.WORKLOADS.values()}[args.workload]
    B, H, N, d = w.B, w.H, w.N, w.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = synthetic.make_inputs(w, ("q", "k", "v"))
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    signs = synthetic.sign_mask(w.seed)
    ws = torch.empty(fbd.fp8_workspace_bytes(B, H, H, N), device=dev, dtype=torch.uint8)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)

    def once(ev):
        ev[0].record()
        fbd.attn_fp8_quantize(q, k, v, signs, ws)
        ev[1].record()
        fbd.attn_fwd_fp8_codes(ws, B, H, H, N, torch.bfloat16, True, w.scale, out=o, lse=lse)
        ev[2].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(args.warmup + args.steps)]
    for i in range(args.warmup):
        once(evs[i])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        once(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    timed = evs[args.warmup:]
    qms = float(np.mean([e[0].elapsed_time(e[1]) for e in timed]))
    fms = float(np.mean([e[1].elapsed_time(e[2]) for e in timed]))
    pairs = B * H * N * (N + 1) / 2
    conv = CONV["fwd"] * d * pairs
    line = {
        "metric": "fp8 attention forward TFLOP/s (rotated E4M3 pre-pass + forward)",
        "value": conv / wall / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3", "data": "synthetic",
        "config": {"workload": w.name + " forward", "B": B, "H": H, "N": N, "d": d,
                   "causal": True, "rotation": True},
        "per_op": {
            "quantize": {"ms": qms, "gbs": B * H * N * d * 11 / (qms * 1e-3) / 1e9},
            "fwd_fp8": {"ms": fms, "conv_tflops": conv / (fms * 1e-3) / 1e12,
                        "executed_frac_fp8_peak":
                            UNITS["fwd"] * 2 * d * pairs / (fms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS},
        },
    }
    print(json.dumps(line), flush=True)


def sweep(only=None):
    """Each operation timed on its own (HIP events on the launch stream; median
    of the repetitions after a warm-up) for N = 1k .. 256k with H = 12, d = 64,
    B = max(1, 16384 / N), for the gpt2s-layer (B8 H12 N1024) and large-key
    (B1 H12 N16384) shapes, and for the extended forms: grouped-query heads,
    a sliding window, packed documents, a block-sparse mask and the HVP call.
    Inputs: seeded device-side normal draws with the BoB workload's
    distributions (Q, K, V, dO ~ 0.5 N(0,1), cotangents ~ N(0,1)), rounded to
    bf16.  FLOP rates count the (query, key) pairs each case leaves visible."""
    import numpy as np
    import torch

    import fwd_bwd_double_amd as fbd

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def case(name, B, H, N, **kw):
        return dict(name=name, B=B, H=H, N=N, Hkv=kw.get("Hkv", H), window=kw.get("window", 0),
                    mean_doc=kw.get("mean_doc", 0), density=kw.get("density", 0.0),
                    hvp=kw.get("hvp", False))

    cases = [case("gpt2s-layer", 8, 12, 1024), case("large-key", 1, 12, 16384)]
    cases += [case(f"sweep-N{n}", max(1, 16384 // n), 12, n)
              for n in (1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072, 262144)]
    cases += [
        # grouped-query: 12 query heads over 4 key/value heads
        case("gqa3-N16384", 1, 12, 16384, Hkv=4),
        # causal sliding window of 4096 keys
        case("window4k-N65536", 1, 12, 65536, window=4096),
        # packed documents, lengths ~ geometric with mean 4096 (seeded)
        case("docs4k-N65536", 1, 12, 65536, mean_doc=4096),
        # block-sparse: each 128 x 128 block below the diagonal kept with
        # probability 1/2 (seeded), diagonal blocks kept
        case("bsparse-N16384", 1, 12, 16384, density=0.5),
        # the Hessian-vector product call (fwd, bwd, BoB in one call)
        case("hvp-N4096", 4, 12, 4096, hvp=True),
    ]
    d = 64
    if only:
        cases = [c for c in cases if c["name"] in only.split(",")]
        if not cases:
            raise SystemExit(f"--case {only}: no such sweep case")
    for cs in cases:
        name, B, H, N, Hkv = cs["name"], cs["B"], cs["H"], cs["N"], cs["Hkv"]
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 + N)

        def draw(std, heads=H):
            return (torch.randn((B, heads, N, d), generator=gen, device=dev) * std).to(
                torch.bfloat16)

        q, k, v, do = draw(0.5), draw(0.5, Hkv), draw(0.5, Hkv), draw(0.5)
        a, bk, c = draw(1.0), draw(1.0, Hkv), draw(1.0, Hkv)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
        gq, gk, gv, gdo = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(k),
                           torch.empty_like(q))
        # grouped-query sizes: room for the split column passes' partial sums
        ws_b = torch.empty(fbd.bwd_ex_workspace_bytes(B, H, Hkv, N) // 4, device=dev)
        ws_bb = torch.empty(fbd.bob_ex_workspace_bytes(B, H, Hkv, N) // 4, device=dev)
        i = np.arange(N, dtype=np.float64)
        vis = i + 1                                   # visible keys per query row
        bm = ds = None
        win = cs["window"]
        if win:
            vis = np.minimum(vis, win)
        if cs["mean_doc"]:
            rng = np.random.default_rng(77)
            starts = np.zeros((B, N), dtype=np.int64)
            for b in range(B):
                r = 0
                while r < N:
                    n = int(min(N - r, rng.geometric(1.0 / cs["mean_doc"])))
                    starts[b, r:r + n] = r
                    r += n
            ds = torch.from_numpy(starts.astype(np.int32)).to(dev)
            vis = (np.arange(N)[None] - starts + 1).astype(np.float64)
        pairs = H * float(np.broadcast_to(vis, (B, N)).sum())
        if cs["density"]:
            nb = (N + 127) // 128
            rng = np.random.default_rng(2024)
            keep = (rng.random((B, nb, nb)) < cs["density"]) | np.eye(nb, dtype=bool)[None]
            bm = torch.from_numpy(keep.astype(np.uint8)).to(dev)
            pairs = H * float((np.tril(keep.astype(np.float64), -1)).sum() * 128 * 128 +
                              keep[:, np.arange(nb), np.arange(nb)].sum() * 128 * 129 / 2)
        sc = 1.0 / 8.0
        mk = dict(window=win, doc_start=ds, block_mask=bm)
        ops = {
            "fwd": lambda: fbd.attn_fwd(q, k, v, causal=True, scale=sc, out=o, lse=lse, **mk),
            "bwd": lambda: fbd.attn_bwd(q, k, v, o, lse, do, causal=True, scale=sc, gproj=True,
                                        workspace=ws_b, outs=(dq, dk, dv), **mk),
            "bob": lambda: fbd.attn_bob(q, k, v, o, lse, do, a, bk, c, causal=True, scale=sc,
                                        workspace=ws_bb, outs=(gq, gk, gv, gdo), **mk),
        }
        plain = Hkv == H and not (win or cs["mean_doc"] or cs["density"] or cs["hvp"])
        if plain:
            ws8 = torch.empty(fbd.fp8_workspace_bytes(B, H, H, N), device=dev, dtype=torch.uint8)
            o8 = torch.empty_like(q)
            signs = 0x9E3779B97F4A7C15
            # FP8 forward: the quantisation pre-pass (rotated) and the forward on the codes
            ops["fp8_quant"] = lambda: fbd.attn_fp8_quantize(q, k, v, signs, ws8)
            ops["fp8_fwd"] = lambda: fbd.attn_fwd_fp8_codes(ws8, B, H, H, N, torch.bfloat16,
                                                            True, sc, out=o8, lse=lse)
        if cs["hvp"]:
            ws_h = torch.empty(fbd.hvp_workspace_bytes(B, H, N) // 4, device=dev)
            ops = {"hvp": lambda: fbd.attn_hvp(q, k, v, do, a, bk, c, causal=True, scale=sc,
                                               gproj=True, workspace=ws_h)}
        exec_units = {"fwd": UNITS["fwd"], "bwd": UNITS["bwd_row"] + UNITS["bwd_col"],
                      "bob": UNITS["bob_row"] + UNITS["bob_col"], "fp8_fwd": UNITS["fwd"]}
        exec_units["hvp"] = exec_units["fwd"] + exec_units["bwd"] + exec_units["bob"]
        conv = {"fwd": CONV["fwd"], "bwd": CONV["bwd"], "bob": CONV["bob"],
                "fp8_fwd": CONV["fwd"], "hvp": CONV["fwd"] + CONV["bwd"] + CONV["bob"]}
        reps = 3 if N >= 65536 else 10
        res = {}
        for op, fn in ops.items():
            fn()
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            for r in range(reps):
                ev[r].record()
                fn()
            ev[reps].record()
            torch.cuda.synchronize()
            ms = float(np.median([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]))
            if op == "fp8_quant":
                # reads Q, K, V (bf16) and V again for its column maxima, writes the codes
                nbytes = B * H * N * d * (2 * 4 + 3)
                res[op] = {"ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9}
                continue
            peak = PEAK_FP8_TFLOPS if op == "fp8_fwd" else PEAK_BF16_TFLOPS
            res[op] = {"ms": ms,
                       "conv_tflops": conv[op] * d * pairs / (ms * 1e-3) / 1e12,
                       "executed_frac_mfma_peak":
                           exec_units[op] * 2 * d * pairs / (ms * 1e-3) / 1e12 / peak}
        line = {"case": name, "B": B, "H": H, "Hkv": Hkv, "N": N, "d": d, "causal": True,
                "gproj": True, "window": win, "mean_doc": cs["mean_doc"],
                "block_density": cs["density"], "pairs": pairs,
                "dtype": "bf16", "data": "synthetic", "ops": res,
                "peak_mem_gb": torch.cuda.max_memory_allocated() / 1e9}
        print(json.dumps(line), flush=True)
        print(f"[sweep] {name:15s} " + "  ".join(
            f"{op} {r['ms']:9.3f} ms " + (f"{r['gbs']:7.0f} GB/s" if "gbs" in r else
                                          f"{r['conv_tflops']:7.1f} TF "
                                          f"{100 * r['executed_frac_mfma_peak']:5.1f}%")
            for op, r in res.items()), file=sys.stderr, flush=True)
        del q, k, v, do, a, bk, c, o, lse, dq, dk, dv, gq, gk, gv, gdo, ws_b, ws_bb, ops
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()


# Which sources define each kernel: a stored counter figure is used only while
# these files are unchanged since the counters were taken.
KERNEL_SOURCES = {
    "fwd": ["fwd.hip"], "bwd_row": ["bwd.hip"], "bwd_col": ["bwd.hip"],
    "bob_row": ["bob_kernels.hpp", "bob.hip"], "bob_col": ["bob_kernels.hpp", "bob.hip"],
}
COMMON_SOURCES = ["tile.hpp", "launch.hpp", "../build.py"]


def kernel_source_sha(kernel):
    import hashlib
    csrc = os.path.join(HERE, "fwd_bwd_double_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + COMMON_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the stored rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (each scaled by the same counter's reading for a copy
    kernel of known size), or None when no summary exists for the current
    kernel source."""
    path = os.path.join(HERE, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != kernel_source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(x, w, nheads):
    """The fp64 oracle (fwd + bwd + BoB, untuned) on the first `nheads` heads."""
    import numpy as np
    import oracle
    from synthetic import to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    heads = [(hh // w.H, hh % w.H) for hh in range(nheads)]
    a = {k: to_f64(v) for k, v in x.items()}
    t0 = time.perf_counter()
    oracle.bob(a["q"], a["k"], a["v"], a["do"], a["g_dq"], a["g_dk"], a["g_dv"], heads=heads,
               with_bwd=True)
    dt = time.perf_counter() - t0
    pairs = nheads * w.N * (w.N + 1) / 2
    flop = sum(CONV.values()) * w.d * pairs
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": dt,
            "sample": f"{nheads} of {w.B * w.H} heads of {w.name}: fwd+bwd+BoB in fp64 NumPy, "
                      f"same FLOP convention"}


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--source-sha":
        print(kernel_source_sha(sys.argv[2]))
    else:
        main()
