"""The autograd glue of fwd_bwd_double_amd.attention, on the CPU: the three
library calls it makes are stood in for by the fp64 oracle (test
infrastructure only), and first and second derivatives through
torch.autograd -- gradient, Hessian-vector product, and the Gauss-Newton
term a loss nonlinear in O brings in -- are compared with torch's own double
backward of a plain fp64 attention.  This checks that the glue routes
tensors, cotangents and the dO path correctly; the kernels themselves are
checked on the GPU."""
import numpy as np
import pytest
import torch

import oracle
from fwd_bwd_double_amd import _lib, autograd


def _np(t):
    return None if t is None else t.detach().double().cpu().numpy()


@pytest.fixture
def oracle_backed(monkeypatch):
    def fwd(q, k, v, causal=True, scale=None, out=None, lse=None, window=0, doc_start=None,
            block_mask=None):
        o, l = oracle.fwd_gqa(_np(q), _np(k), _np(v), causal=causal, scale=scale,
                              window=window, docs=_np(doc_start), block_mask=_np(block_mask))
        return torch.from_numpy(o), torch.from_numpy(l)

    def bwd(q, k, v, o, lse, do, causal=True, scale=None, gproj=False, workspace=None,
            outs=None, passes=3, window=0, doc_start=None, block_mask=None):
        r = oracle.bwd_gqa(_np(q), _np(k), _np(v), _np(do), causal=causal, scale=scale,
                           window=window, docs=_np(doc_start), block_mask=_np(block_mask))
        return tuple(torch.from_numpy(r[n]) for n in ("dQ", "dK", "dV"))

    def bob(q, k, v, o, lse, do, g_dq, g_dk, g_dv, causal=True, scale=None, workspace=None,
            outs=None, passes=3, window=0, doc_start=None, block_mask=None, gproj=False):
        # (the projections only remove bf16 rounding residuals: exact
        # arithmetic needs none)
        r = oracle.bob_gqa(_np(q), _np(k), _np(v), _np(do), _np(g_dq), _np(g_dk), _np(g_dv),
                           causal=causal, scale=scale, window=window, docs=_np(doc_start),
                           block_mask=_np(block_mask))
        return tuple(torch.from_numpy(r[n]) for n in ("gQ", "gK", "gV", "gdO"))

    monkeypatch.setattr(_lib, "attn_fwd", fwd)
    monkeypatch.setattr(_lib, "attn_bwd", bwd)
    monkeypatch.setattr(_lib, "attn_bob", bob)


def torch_attention(q, k, v, causal, scale, window=0):
    g = q.shape[1] // k.shape[1]
    k, v = k.repeat_interleave(g, dim=1), v.repeat_interleave(g, dim=1)
    s = scale * q @ k.transpose(-1, -2)
    n = q.shape[2]
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    hide = torch.zeros(n, n, dtype=torch.bool)
    if causal:
        hide |= j > i
    if window:
        hide |= j <= i - window
    s = s.masked_fill(hide, float("-inf"))
    return torch.softmax(s, -1) @ v


@pytest.mark.parametrize("causal,H,Hkv,window,loss", [
    (True, 2, 2, 0, "linear"), (False, 2, 2, 0, "linear"), (True, 4, 2, 0, "square"),
    (True, 2, 1, 3, "square")])
def test_double_backward_matches_torch(oracle_backed, causal, H, Hkv, window, loss):
    rng = np.random.default_rng(7 + H + Hkv + window)
    B, N, d, scale = 1, 9, 64, 0.125
    r = lambda h: torch.from_numpy(rng.standard_normal((B, h, N, d)))
    q0, k0, v0, do, vq = r(H), r(Hkv), r(Hkv), r(H), r(H)
    vk, vv = r(Hkv), r(Hkv)

    def derivs(fn):
        q, k, v = (t.clone().requires_grad_() for t in (q0, k0, v0))
        o = fn(q, k, v)
        L = (do * o).sum() if loss == "linear" else 0.5 * (o * o).sum()
        g = torch.autograd.grad(L, (q, k, v), create_graph=True)
        s = sum((a * b).sum() for a, b in zip(g, (vq, vk, vv)))
        h = torch.autograd.grad(s, (q, k, v))
        return [t.detach() for t in g], list(h)

    got_g, got_h = derivs(lambda q, k, v: autograd.attention(q, k, v, causal=causal, scale=scale,
                                                             window=window))
    ref_g, ref_h = derivs(lambda q, k, v: torch_attention(q, k, v, causal, scale, window))
    for a, b in zip(got_g + got_h, ref_g + ref_h):
        assert a.shape == b.shape
        assert torch.allclose(a, b, rtol=1e-9, atol=1e-11), float((a - b).abs().max())
