"""Attention as a twice-differentiable torch operation.

`attention(q, k, v, ...)` returns O and registers two autograd functions, so
that torch's autograd reaches every kernel of the library:

- the gradient of O is the recompute backward (`attn_bwd`, optionally with
  GProj);
- the gradient of that backward -- what `torch.autograd.grad(...,
  create_graph=True)` followed by a second differentiation asks for, as in a
  Hessian-vector product or a second-order optimiser -- is the two-pass
  backward-over-backward (`attn_bob`).  This is the FlashBoB page's use case
  (rit.work, flashbob-second-order-attention, section "Why go backward through
  an already computed gradient"): second-order training signals without the
  quadratic intermediates that autodiff through the backward would keep.

The backward-over-backward is the derivative of the whole first-backward map
(Q, K, V, dO) -> (dQ, dK, dV), with O and LSE taken as the functions of
(Q, K, V) they are: its Q, K, V outputs already contain the paths through O
and LSE, so no gradient is passed to the saved O and LSE themselves.  GProj
(a rounding correction that is the identity in exact arithmetic) is not
differentiated: the second derivative is that of the exact map.

Only marshalling lives here; every step runs in the library's HIP kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib


def _zeros_if_none(g, like):
    return torch.zeros_like(like) if g is None else g.contiguous()


class _AttnBackward(torch.autograd.Function):
    """(q, k, v, o, lse, do) -> (dq, dk, dv); its own backward is BoB."""

    @staticmethod
    def forward(ctx, q, k, v, o, lse, do, opts):
        dq, dk, dv = _lib.attn_bwd(q, k, v, o, lse, do, causal=opts["causal"],
                                   scale=opts["scale"], gproj=opts["gproj"],
                                   window=opts["window"], doc_start=opts["doc_start"],
                                   block_mask=opts["block_mask"])
        ctx.save_for_backward(q, k, v, o, lse, do)
        ctx.opts = opts
        return dq, dk, dv

    @staticmethod
    def backward(ctx, g_dq, g_dk, g_dv):
        q, k, v, o, lse, do = ctx.saved_tensors
        opts = ctx.opts
        g_dq, g_dk, g_dv = (_zeros_if_none(g, t) for g, t in ((g_dq, q), (g_dk, k), (g_dv, v)))
        gq, gk, gv, gdo = _lib.attn_bob(q, k, v, o, lse, do, g_dq, g_dk, g_dv,
                                        causal=opts["causal"], scale=opts["scale"],
                                        window=opts["window"], doc_start=opts["doc_start"],
                                        block_mask=opts["block_mask"], gproj=opts["gproj"])
        # O and LSE are functions of (q, k, v): their paths are inside gq, gk, gv
        return gq, gk, gv, None, None, gdo, None


class _Attn(torch.autograd.Function):
    """(q, k, v) -> O; its backward runs through _AttnBackward, so it is
    differentiable once more."""

    @staticmethod
    def forward(ctx, q, k, v, opts):
        o, lse = _lib.attn_fwd(q, k, v, causal=opts["causal"], scale=opts["scale"],
                               window=opts["window"], doc_start=opts["doc_start"],
                               block_mask=opts["block_mask"])
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.opts = opts
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _g_lse):
        q, k, v, o, lse = ctx.saved_tensors
        if do is None:
            return None, None, None, None
        dq, dk, dv = _AttnBackward.apply(q, k, v, o.detach(), lse, do.contiguous(), ctx.opts)
        return dq, dk, dv, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
              scale: Optional[float] = None, gproj: bool = False, window: int = 0,
              doc_start: Optional[torch.Tensor] = None,
              block_mask: Optional[torch.Tensor] = None, return_lse: bool = False):
    """O = softmax(scale q k^T + mask) v for q (B, H, N, 64) and k, v (B, Hkv,
    N, 64), bf16 or fp32 on the GPU, differentiable twice through the
    library's kernels (first backward: `attn_bwd`, with GProj when `gproj`;
    second: `attn_bob`, which then also projects the residual row sums of
    g_Q's and g_dO's bf16 weights).  The masks are those of `attn_fwd`.  With
    `return_lse`, the row log-sum-exp is returned too (not differentiable)."""
    opts = dict(causal=causal, scale=scale, gproj=gproj, window=int(window),
                doc_start=doc_start, block_mask=block_mask)
    o, lse = _Attn.apply(q.contiguous(), k.contiguous(), v.contiguous(), opts)
    return (o, lse) if return_lse else o
