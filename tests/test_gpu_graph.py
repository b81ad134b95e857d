"""The library's calls under HIP graph capture (torch.cuda.graph): a captured
forward, backward (GProj) and backward-over-backward, or the same outputs from
one Hessian-vector-product call (its fused row pass), multi-head and
grouped-query (split column passes, whose partial sums another kernel adds),
replayed several times with new inputs written in between and eager work
between the replays; every replay must equal the eager calls on the same
inputs bit for bit (the kernels are deterministic and allocate nothing; the
binding's output and workspace tensors come from the graph's memory pool)."""
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


def step(fbd, x, Hkv):
    q, k, v, do, a, bk, c = x
    o, lse = fbd.attn_fwd(q, k, v, causal=True, scale=0.125)
    dq, dk, dv = fbd.attn_bwd(q, k, v, o, lse, do, causal=True, scale=0.125, gproj=True)
    gq, gk, gv, gdo = fbd.attn_bob(q, k, v, o, lse, do, a, bk, c, causal=True, scale=0.125)
    return [o, lse, dq, dk, dv, gq, gk, gv, gdo]


def hvp_step(fbd, x, Hkv):
    q, k, v, do, a, bk, c = x
    r = fbd.attn_hvp(q, k, v, do, a, bk, c, causal=True, scale=0.125, gproj=True)
    return [r[n] for n in ("O", "LSE", "dQ", "dK", "dV", "Hv_q", "Hv_k", "Hv_v", "Hv_do")]


@pytest.mark.parametrize("mode", ["calls", "hvp"])
@pytest.mark.parametrize("H,Hkv,N", [(4, 4, 700), (6, 2, 513)])
def test_graph_replays_match_eager(H, Hkv, N, mode):
    import fwd_bwd_double_amd as fbd
    B = 1
    gen = torch.Generator(device="cuda").manual_seed(3000 + N)
    shapes = [H, Hkv, Hkv, H, H, Hkv, Hkv]

    def fill(x):
        for t, h in zip(x, shapes):
            t.copy_((0.5 * torch.randn(B, h, N, 64, device="cuda", generator=gen)).bfloat16())

    x = [torch.empty(B, h, N, 64, device="cuda", dtype=torch.bfloat16) for h in shapes]
    fill(x)
    say(f"[gpu] graph capture B={B} H={H} Hkv={Hkv} N={N} mode={mode}")
    step = globals()["hvp_step" if mode == "hvp" else "step"]
    step(fbd, x, Hkv)                                  # warm-up (library load, allocator)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(fbd, x, Hkv)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step(fbd, x, Hkv)
    for rep in range(3):
        fill(x)                                        # new inputs, eager work between replays
        ref = [t.clone() for t in step(fbd, x, Hkv)]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV", "gQ", "gK", "gV", "gdO"), outs, ref):
            assert torch.equal(a, b), (rep, name)
        say(f"    replay {rep}: all nine outputs equal the eager calls")
