"""attn_bob_noalloc (backward-over-backward with its row states in the
library's own device array) against attn_bob with a caller workspace, through
the C ABI: the same kernels on the same inputs, so the outputs must agree bit
for bit.  Two calls in a row per dtype, the second on a smaller input, so the
array still holds the first call's states when the second runs."""
import pytest
import torch

import fwd_bwd_double_amd as fbd
import synthetic
from gpu_util import inputs, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bob_noalloc_matches_workspace_call(dtype):
    for B, H, N, causal in ((2, 3, 777, True), (1, 2, 300, False)):
        w = synthetic.Workload(f"noalloc-{dtype}", B, H, N, 64, dtype, 7300 + N, causal=causal,
                               qkv_std=0.5)
        x, g, a = inputs(w)
        say(f"[gpu] attn_bob_noalloc B={B} H={H} N={N} causal={causal} {dtype}")
        o, lse = fbd.attn_fwd(g["q"], g["k"], g["v"], causal=causal, scale=w.scale)
        args = (g["q"], g["k"], g["v"], o, lse, g["do"], g["g_dq"], g["g_dk"], g["g_dv"])
        ref = fbd.attn_bob(*args, causal=causal, scale=w.scale)
        outs = tuple(torch.full_like(g["q"], 3.0) for _ in range(4))
        got = fbd.attn_bob_noalloc(*args, causal=causal, scale=w.scale, outs=outs)
        torch.cuda.synchronize()
        assert all(a_ is b_ for a_, b_ in zip(got, outs))
        for name, r, t in zip(("g_Q", "g_K", "g_V", "g_dO"), ref, got):
            same = torch.equal(r, t)
            say(f"    {name}: bit-identical {same}")
            assert same, name


def test_bob_noalloc_rejects_oversize():
    # beyond the array's rows: an error before anything is enqueued; the
    # outputs keep their contents
    B, H, N = 1, 1, (3 << 20) + 1
    q = torch.zeros(B, H, N, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(B, H, N, device="cuda")
    outs = tuple(torch.full_like(q, 5.0) for _ in range(4))
    with pytest.raises(fbd.AttnError) as e:
        fbd.attn_bob_noalloc(q, q.clone(), q.clone(), q.clone(), lse, q.clone(), q.clone(),
                             q.clone(), q.clone(), outs=outs)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert all(bool((t == 5.0).all()) for t in outs)
