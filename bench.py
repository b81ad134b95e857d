"""Throughput of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  attn_fwd -> attn_bwd (row pass, column pass; GProj on) -> attn_bob (row
  pass, column pass), causal, bf16 inputs with fp32 accumulation, d = 64,
  seeded inputs (Q, K, V, dO ~ 0.5 N(0,1), cotangents ~ N(0,1)) resident in
  device memory before timing.  The reported line runs on the long-context
  workload B=1, H=12, N=262144 (the FlashBoB page's 262k tokens).

Prints ONE JSON line.  `value` is the step's model TFLOP/s under the FLOP
convention (per unmasked causal (query, key) pair and head: forward 4d,
backward 10d, backward-over-backward 38d -- the 19 contraction units of the
two-pass scheme); `value_min_work` counts the backward-over-backward as the
12 units a single dense pass would need (24d).  `roofline` is the dominant
kernel's executed contraction FLOPs per launch over its HIP-event-timed
duration against the bf16 dense MFMA peak; `cpu_baseline` is the fp64 oracle
timed on a bounded sample of the same workload on this host.  `extra` holds
the B4 H12 N4096 step, the GPT-2-Small layer shape B8 H12 N1024 timed with
the caches flushed before every kernel (HBM-bound: achieved GB/s of its
algorithmic bytes), the backward's time with GProj off and on, and the same
step's outputs from the one Hessian-vector-product call (`hvp_fused`:
attn_hvp with the BoB cotangents as the direction, whose single row pass
finishes BoB's row outputs and the backward's dQ together), with its time and
how its outputs compare with the separate calls'.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2] [--no-cpu-baseline]
                    [--no-extra] [--workload NAME]

`--fp8` times the FP8 forward (rotated quantisation pre-pass + E4M3 forward)
on the B4 H12 N4096 workload instead of the step, one JSON line.

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
HEADLINE = "bob-long-B1H12N262144"
FLUSH_BYTES = 512 << 20     # written between kernels: evicts L2 (8 x 4 MB) and MALL (256 MB)

# Contraction units (N x N x d products, 2d FLOP per unmasked pair) executed
# by each kernel; GProj adds one unit to each backward pass.
UNITS = {"fwd": 2, "bwd_row": 4, "bwd_col": 5, "bob_row": 11, "bob_col": 8}
UNITS_NO_GPROJ = {"bwd_row": 3, "bwd_col": 4}
# FLOP convention per unmasked pair, in units of d
CONV = {"fwd": 4, "bwd": 10, "bob": 38}
# minimal work: a backward-over-backward in one dense pass (S, dP, W twice, U,
# then g_Q, g_K twice each, g_V, g_dO twice) is 12 units
CONV_MIN = {"fwd": 4, "bwd": 10, "bob": 24}
# Algorithmic HBM bytes per launch as (tensors, row arrays): (B, H, N, d)
# tensors read or written once, and (B, H, N) fp32 arrays.  fwd: Q, K, V, O
# and LSE.  bwd_row: Q, K, V, O, dO, dQ; LSE in, D, r, -LSE log2(e) out.
# bwd_col: Q, K, V, dO, dK, dV; -LSE log2(e), D, r.  bob_row: Q, K, V, O, dO
# and the three cotangents in, g_Q and g_dO out; LSE in, D, alpha, beta,
# -LSE log2(e), -kappa out.  bob_col: Q, K, V, dO, g_dQ, g_dK, g_dV in, g_K,
# g_V out; -LSE log2(e), D, alpha, -kappa.
ALG_BYTES = {"fwd": (4, 1), "bwd_row": (6, 4), "bwd_col": (6, 3), "bob_row": (10, 6),
             "bob_col": (9, 4)}
KERNELS = ["fwd", "bwd_row", "bwd_col", "bob_row", "bob_col"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the extra workloads (B4 H12 N4096 step, flushed GPT-2-Small "
                        "layer, GProj on/off)")
    p.add_argument("--sweep", action="store_true",
                   help="time fwd, bwd and BoB separately over N = 1k .. 256k and the other "
                        "workload shapes (one JSON line per case) instead of the step")
    p.add_argument("--case", default=None,
                   help="with --sweep: only the named cases (comma-separated), e.g. "
                        "sweep-N262144 for a counter run on the longest sequence")
    p.add_argument("--fp8", action="store_true",
                   help="time the FP8 forward (rotated quantisation pre-pass + E4M3 forward) on "
                        "the B4 H12 N4096 workload instead of the step (one JSON line)")
    p.add_argument("--workload", default=HEADLINE,
                   choices=[HEADLINE, "bob-B4H12N4096", "gpt2s-layer-B8H12N1024"],
                   help="workload the step runs on: the long-context workload (the reported "
                        "line), the B4 H12 N4096 BoB workload, or the GPT-2-Small layer "
                        "shape (for counter runs)")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="first run one device-to-device copy of this many MiB (a plain copy "
                        "kernel of known size, to calibrate memory counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def workload(name):
    import synthetic
    return {x.name: x for x in synthetic.WORKLOADS.values()}[name]


class Step:
    """Device tensors and the five launches of one step on workload w."""

    def __init__(self, w, x, dev):
        import torch
        import fwd_bwd_double_amd as fbd
        self.fbd, self.w = fbd, w
        B, H, N = w.B, w.H, w.N
        self.g = {k: v.to(dev) for k, v in x.items()}
        q = self.g["q"]
        self.o = torch.empty_like(q)
        self.lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
        self.dq, self.dk, self.dv = (torch.empty_like(q) for _ in range(3))
        self.has_bob = "g_dq" in self.g
        if self.has_bob:
            self.gq, self.gk, self.gv, self.gdo = (torch.empty_like(q) for _ in range(4))
            self.ws_bb = torch.empty(fbd.bob_workspace_bytes(B, H, N) // 4, device=dev)
        self.ws_b = torch.empty(fbd.bwd_workspace_bytes(B, H, N) // 4, device=dev)
        self.names = KERNELS if self.has_bob else KERNELS[:3]

    def launch(self, name, gproj=True):
        g, sc, f = self.g, self.w.scale, self.fbd
        if name == "fwd":
            f.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=sc, out=self.o, lse=self.lse)
        elif name.startswith("bwd"):
            f.attn_bwd(g["q"], g["k"], g["v"], self.o, self.lse, g["do"], causal=True, scale=sc,
                       gproj=gproj, workspace=self.ws_b, outs=(self.dq, self.dk, self.dv),
                       passes=1 if name == "bwd_row" else 2)
        else:
            f.attn_bob(g["q"], g["k"], g["v"], self.o, self.lse, g["do"], g["g_dq"], g["g_dk"],
                       g["g_dv"], causal=True, scale=sc, workspace=self.ws_bb,
                       outs=(self.gq, self.gk, self.gv, self.gdo),
                       passes=1 if name == "bob_row" else 2)

    def run(self, ev=None, gproj=True, flush=None):
        """One step; ev: HIP events recorded around each kernel (on torch's
        current stream, the one the library launches on); flush: a buffer
        written before every kernel (outside the events)."""
        for i, n in enumerate(self.names):
            if flush is not None:
                flush.fill_(i + 1)
            if ev is not None:
                ev[2 * i].record()
            self.launch(n, gproj)
            if ev is not None:
                ev[2 * i + 1].record()


def timed_steps(st, steps, warmup, gproj=True, flush=None, wall=True):
    """W untimed then K timed steps; returns (wall ms per step, {kernel: mean
    event ms}).  The timed region is bracketed by device synchronisations."""
    import numpy as np
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(st.names))]
           for _ in range(max(steps, 1))]
    for _ in range(warmup):
        st.run(gproj=gproj, flush=flush)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        st.run(evs[s], gproj=gproj, flush=flush)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = {n: float(np.mean([e[2 * i].elapsed_time(e[2 * i + 1]) for e in evs[:steps]]))
            for i, n in enumerate(st.names)}
    kmed = {n: float(np.median([e[2 * i].elapsed_time(e[2 * i + 1]) for e in evs[:steps]]))
            for i, n in enumerate(st.names)}
    return (t1 - t0) * 1e3 / max(steps, 1), kern, kmed


def report(w, names, kern_ms, ms_step, elt, gproj=True):
    """Per-kernel and per-operation rates of one step on workload w."""
    d = w.d
    pairs = w.B * w.H * w.N * (w.N + 1) / 2      # unmasked causal pairs over all heads
    unit = 2 * d * pairs                         # FLOP of one N x N x d contraction unit
    units = dict(UNITS, **({} if gproj else UNITS_NO_GPROJ))
    t_b, r_b = w.B * w.H * w.N * d * elt, w.B * w.H * w.N * 4
    per_kernel = {}
    for n in names:
        ms = kern_ms[n]
        ex = units[n] * unit / (ms * 1e-3) / 1e12
        a, b = ALG_BYTES[n]
        ab = a * t_b + b * r_b
        per_kernel[n] = {"ms": ms, "executed_tflops": ex, "frac_mfma_peak": ex / PEAK_BF16_TFLOPS,
                         "flop_per_launch": units[n] * unit, "alg_bytes": ab,
                         "alg_gbs": ab / (ms * 1e-3) / 1e9,
                         "frac_hbm_peak": ab / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    op_ms = {"fwd": kern_ms["fwd"], "bwd": kern_ms["bwd_row"] + kern_ms["bwd_col"]}
    if "bob_row" in names:
        op_ms["bob"] = kern_ms["bob_row"] + kern_ms["bob_col"]
    per_op = {}
    for op, ms in op_ms.items():
        per_op[op] = {"ms": ms, "conv_tflops": CONV[op] * d * pairs / (ms * 1e-3) / 1e12,
                      "min_work_tflops": CONV_MIN[op] * d * pairs / (ms * 1e-3) / 1e12}
        per_op[op]["frac_mfma_peak"] = per_op[op]["conv_tflops"] / PEAK_BF16_TFLOPS
    out = {"per_kernel": per_kernel, "per_op": per_op, "pairs": pairs}
    if ms_step is not None:
        out["ms_per_step"] = ms_step
        out["value"] = sum(CONV[op] for op in op_ms) * d * pairs / (ms_step * 1e-3) / 1e12
        out["value_min_work"] = (sum(CONV_MIN[op] for op in op_ms) * d * pairs /
                                 (ms_step * 1e-3) / 1e12)
    return out


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

    import torch

    import synthetic

    w = workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"{w.name}: drawing the seeded inputs")
    x = synthetic.make_inputs(w)
    st = Step(w, x, dev)
    if args.copy_mb > 0:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"{w.name}: {args.warmup} warm-up + {args.steps} timed steps")
    ms_step, kern_ms, _ = timed_steps(st, args.steps, args.warmup)
    rep = report(w, st.names, kern_ms, ms_step, x["q"].element_size())
    log(f"{w.name}: {ms_step:.3f} ms per step, {rep['value']:.1f} TFLOP/s")
    dom = max(st.names, key=lambda n: kern_ms[n])
    pk = rep["per_kernel"][dom]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": pk["executed_tflops"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": pk["executed_tflops"] / PEAK_BF16_TFLOPS,
                "traffic": stored_traffic(dom, w.name), "traffic_unit": "bytes per launch",
                "flop_per_launch": pk["flop_per_launch"], "ms_per_launch": pk["ms"]}
    peak_mem = torch.cuda.max_memory_allocated() / 1e9

    extra = None
    if not args.no_extra:
        extra = {"gproj_overhead": {w.name: gproj_overhead(st, 3 if w.N > 65536 else 20)}}
        extra["hvp_fused"] = {w.name: hvp_fused(st, 3 if w.N > 65536 else 20, ms_step, rep)}
        del st
        torch.cuda.empty_cache()
        extra.update(extra_workloads(dev, w.name, extra["gproj_overhead"]))

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        cpu = cpu_baseline(x, w)

    line = {
        "metric": METRIC, "value": rep["value"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": True,
                   "gproj": True, "step": "fwd + bwd(row, col) + bob(row, col)",
                   "parallelism": "single GPU"},
        "value_min_work": rep["value_min_work"],
        "roofline": roofline, "cpu_baseline": cpu, "per_kernel": rep["per_kernel"],
        "per_op": rep["per_op"], "peak_mem_gb": peak_mem, "extra": extra,
    }
    print(json.dumps(line), flush=True)


def hvp_fused(st, reps, ms_sep, rep):
    """The same step's outputs from the one Hessian-vector-product call
    (attn_hvp with v = the BoB cotangents, GProj on): forward, one row pass
    that finishes BoB's row outputs and the backward's dQ together, then the
    backward's and BoB's column passes.  Median ms of `reps` calls (HIP events
    on the launch stream), the rate under the same FLOP convention as the
    step, and the comparison of its outputs with the separate calls' (the
    step just run): O, LSE, dQ, dK, dV, Hv_K, Hv_V bit for bit; Hv_Q and
    Hv_dO as rel-L2 (GProj in the Hessian-vector product also projects
    their bf16 weights' residual row sums, which the step's attn_bob does
    not, and the fused pass regroups Hv_Q's alpha term)."""
    import numpy as np
    import torch
    g, f, w = st.g, st.fbd, st.w
    ws = torch.empty(f.hvp_workspace_bytes(w.B, w.H, w.N) // 4, device=g["q"].device)
    call = lambda: f.attn_hvp(g["q"], g["k"], g["v"], g["do"], g["g_dq"], g["g_dk"], g["g_dv"],
                              causal=True, scale=w.scale, gproj=True, workspace=ws)
    r = call()
    st.run()          # the separate calls, for the comparison
    torch.cuda.synchronize()
    same = {k: bool(torch.equal(r[k], t)) for k, t in (
        ("O", st.o), ("LSE", st.lse), ("dQ", st.dq), ("dK", st.dk), ("dV", st.dv),
        ("Hv_k", st.gk), ("Hv_v", st.gv))}
    rel = lambda x, y: float((x.double() - y.double()).norm() / y.double().norm())
    dif, dif_do = rel(r["Hv_q"], st.gq), rel(r["Hv_do"], st.gdo)
    del r
    times = []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        call()
        ev[1].record()
        torch.cuda.synchronize()
        times.append(ev[0].elapsed_time(ev[1]))
    ms = float(np.median(times))
    conv = sum(CONV[op] for op in ("fwd", "bwd", "bob")) * w.d * rep["pairs"]
    out = {"ms": ms, "conv_tflops": conv / (ms * 1e-3) / 1e12, "separate_ms_per_step": ms_sep,
           "speedup": ms_sep / ms, "bit_identical": same, "hv_q_rel_l2_vs_separate": dif,
           "hv_do_rel_l2_vs_separate": dif_do}
    log(f"{w.name} fused HVP: {ms:.3f} ms ({out['conv_tflops']:.1f} TFLOP/s), "
        f"{out['speedup']:.3f}x the separate calls; identical {same}; Hv_q rel-L2 {dif:.2e}, "
        f"Hv_do rel-L2 {dif_do:.2e}")
    return out


def gproj_overhead(st, reps):
    """The backward (row + column pass) with GProj off and on, alternating,
    `reps` times each: median ms and the relative cost of the projection."""
    import numpy as np
    import torch
    res = {False: [], True: []}
    for _ in range(reps):
        for gp in (False, True):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
            st.launch("bwd_row", gp)
            ev[1].record()
            st.launch("bwd_col", gp)
            ev[2].record()
            torch.cuda.synchronize()
            res[gp].append((ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])))
    med = {gp: np.median(np.array(v), axis=0) for gp, v in res.items()}
    off, on = float(med[False].sum()), float(med[True].sum())
    out = {"reps": reps, "bwd_ms_gproj_off": off, "bwd_ms_gproj_on": on,
           "bwd_row_ms": [float(med[False][0]), float(med[True][0])],
           "bwd_col_ms": [float(med[False][1]), float(med[True][1])],
           "bwd_overhead_frac": on / off - 1.0}
    log(f"{st.w.name}: bwd {off:.3f} ms without GProj, {on:.3f} ms with (+{100 * (on / off - 1):.1f}%)")
    return out


def extra_workloads(dev, headline, gp):
    """The B4 H12 N4096 step (20 steps after 5 warm-ups), its GProj cost, the
    same outputs from the fused Hessian-vector-product call, and
    the GPT-2-Small layer shape B8 H12 N1024 (forward + backward) with a
    512 MiB buffer written before every kernel so that each reads its inputs
    from HBM (median of 20 steps)."""
    import torch
    import synthetic
    out = {}
    if headline != "bob-B4H12N4096":
        w = workload("bob-B4H12N4096")
        x = synthetic.make_inputs(w)
        st = Step(w, x, dev)
        ms, kern, _ = timed_steps(st, 20, 5)
        rep = report(w, st.names, kern, ms, 2)
        rep["stored_traffic"] = {n: stored_traffic(n, w.name) for n in st.names}
        out[w.name] = rep
        gp[w.name] = gproj_overhead(st, 20)
        log(f"{w.name}: {ms:.3f} ms per step, {rep['value']:.1f} TFLOP/s")
        rep["hvp_fused"] = hvp_fused(st, 20, ms, rep)
        del st
    w = workload("gpt2s-layer-B8H12N1024")
    x = synthetic.make_inputs(w, ("q", "k", "v", "do"))
    st = Step(w, x, dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    _, kern_warm, _ = timed_steps(st, 20, 5)
    _, _, kern_cold = timed_steps(st, 20, 3, flush=flush)
    rep = report(w, st.names, kern_cold, None, 2)
    rep["flushed_bytes_before_each_kernel"] = FLUSH_BYTES
    rep["per_kernel_warm_ms"] = kern_warm
    rep["stored_traffic"] = {n: stored_traffic(n, w.name) for n in st.names}
    rep["floor_us"] = {n: v["alg_bytes"] / (HBM_PEAK_GBS * 1e9) * 1e6
                       for n, v in rep["per_kernel"].items()}
    out[w.name + " (flushed)"] = rep
    log(f"{w.name} flushed: " + ", ".join(
        f"{n} {v['ms'] * 1e3:.1f} us ({v['alg_gbs']:.0f} GB/s)" for n, v in rep["per_kernel"].items()))
    del st, flush
    torch.cuda.empty_cache()
    return out


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

    w = workload("bob-B4H12N4096")
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


def cpu_baseline(x, w):
    """The fp64 oracle (untuned) on a bounded sample of workload w, on this
    host's cores.  Long sequences (N > 8192): the first 2048 rows of every
    head (fwd, bwd and BoB of the causal prefix, which depends only on its
    own keys), 128 seeded random rows of every head beyond them (each row's
    outputs from its own definition) and the key-side BoB outputs of the last
    64 keys of heads 0, 4, 7 and 11 (only the last 64 rows see them).  Shorter
    sequences: whole heads, as many as take about 10 s.  The rate counts the
    (query, key) pairs the sample evaluates under the same FLOP convention
    (52d per pair where fwd, bwd and BoB quantities are formed, 42d for the
    key-side columns, which need no first-order gradients)."""
    import numpy as np
    import oracle
    from synthetic import to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    d = w.d
    conv_all = sum(CONV.values()) * d
    flop = 0.0
    t0 = time.perf_counter()
    if w.N > 8192:
        n0 = 2048
        pre = {k: to_f64(v[:, :, :n0]) for k, v in x.items()}
        oracle.bob(pre["q"], pre["k"], pre["v"], pre["do"], pre["g_dq"], pre["g_dk"],
                   pre["g_dv"], with_bwd=True)
        flop += conv_all * w.B * w.H * n0 * (n0 + 1) / 2
        rng = np.random.default_rng(5005)
        rows = np.sort(rng.choice(np.arange(n0, w.N), 128, replace=False))
        for h in range(w.H):
            a = {k: to_f64(v[:, h:h + 1, : rows[-1] + 1]) for k, v in x.items()}
            oracle.rows(a["q"], a["k"], a["v"], a["do"], a["g_dq"], a["g_dk"], a["g_dv"],
                        row_idx=rows)
            flop += conv_all * float((rows + 1).sum())
        for h in (0, 4, 7, 11):
            a = {k: to_f64(v[:, h:h + 1]) for k, v in x.items()}
            oracle.last_columns(a["q"], a["k"], a["v"], a["do"], a["g_dq"], a["g_dk"],
                                a["g_dv"], ncols_tail=64, chunk=64)
            flop += (CONV["fwd"] + CONV["bob"]) * d * 64 * w.N
        sample = (f"{w.name}: rows 0..2047 of all {w.H} heads (fwd+bwd+BoB), 128 random rows "
                  f"per head beyond them, BoB key-side outputs of the last 64 keys of 4 heads")
    else:
        per_head = w.N * (w.N + 1) / 2
        nheads = max(1, min(w.B * w.H, int(10.0 * 2e10 / (conv_all * per_head))))
        heads = [(hh // w.H, hh % w.H) for hh in range(nheads)]
        a = {k: to_f64(v) for k, v in x.items()}
        if "g_dq" in a:
            oracle.bob(a["q"], a["k"], a["v"], a["do"], a["g_dq"], a["g_dk"], a["g_dv"],
                       heads=heads, with_bwd=True)
            flop += conv_all * nheads * per_head
            sample = f"{nheads} of {w.B * w.H} heads of {w.name}: fwd+bwd+BoB"
        else:
            oracle.bwd(a["q"], a["k"], a["v"], a["do"], heads=heads)
            flop += (CONV["fwd"] + CONV["bwd"]) * d * nheads * per_head
            sample = f"{nheads} of {w.B * w.H} heads of {w.name}: fwd+bwd"
    dt = time.perf_counter() - t0
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": dt,
            "sample": sample + " in fp64 NumPy, same FLOP convention"}


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--source-sha":
        print(kernel_source_sha(sys.argv[2]))
    else:
        main()
