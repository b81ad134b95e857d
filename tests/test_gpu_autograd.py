"""torch.autograd through the library (fwd_bwd_double_amd.attention): the
first derivatives come from the backward kernels and the second from the
backward-over-backward kernels.  Checked against the fp64 oracle: the
gradient against its backward, and Hessian-vector products (double backward
through autograd) against its BoB, for a loss linear in O and for one that is
not (where the HVP also needs the Jacobian-vector product of O, BoB's g_dO)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import check, inputs, say, tol

pytestmark = pytest.mark.gpu


def leaves(g, Hkv):
    q = g["q"].clone().requires_grad_()
    k = g["k"][:, :Hkv].contiguous().requires_grad_()
    v = g["v"][:, :Hkv].contiguous().requires_grad_()
    return q, k, v


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("causal,H,Hkv,N,gproj", [(True, 2, 2, 200, False),
                                                  (False, 2, 2, 130, True),
                                                  (True, 4, 2, 300, False)])
def test_autograd_gradient_and_hvp(causal, H, Hkv, N, gproj, dtype):
    # Phi = <dO, O(q, k, v)> with dO fixed: autograd's gradient is the
    # backward, and the gradient of <grad Phi, v> is H v (BoB, cotangents v)
    import fwd_bwd_double_amd as fbd
    w = synthetic.Workload(f"autograd-{dtype}", 1, H, N, 64, dtype, 6100 + N + H,
                           causal=causal, qkv_std=0.5)
    x, g, a = inputs(w)
    for n in ("k", "v", "g_dk", "g_dv"):
        a[n] = a[n][:, :Hkv]
    vq, vk, vv = g["g_dq"], g["g_dk"][:, :Hkv].contiguous(), g["g_dv"][:, :Hkv].contiguous()
    say(f"[gpu] autograd B=1 H={H} Hkv={Hkv} N={N} causal={causal} gproj={gproj} {dtype}")
    q, k, v = leaves(g, Hkv)
    o = fbd.attention(q, k, v, causal=causal, scale=w.scale, gproj=gproj)
    phi = (g["do"] * o).sum()
    gq, gk, gv = torch.autograd.grad(phi, (q, k, v), create_graph=True)
    s = (gq * vq).sum() + (gk * vk).sum() + (gv * vv).sum()
    hq, hk, hv = torch.autograd.grad(s, (q, k, v))
    torch.cuda.synchronize()
    ref = oracle.bob_gqa(a["q"], a["k"], a["v"], a["do"], a["g_dq"], a["g_dk"], a["g_dv"],
                         causal=causal, with_bwd=True)
    f64 = synthetic.to_f64
    t1, t2 = tol(dtype), tol(dtype, bob=True)
    check("O", f64(o.detach()), ref["O"], t1)
    for name, t, rk in (("dQ", gq, "dQ"), ("dK", gk, "dK"), ("dV", gv, "dV")):
        check(name, f64(t.detach()), ref[rk], t1)
    for name, t, rk in (("Hv_q", hq, "gQ"), ("Hv_k", hk, "gK"), ("Hv_v", hv, "gV")):
        check(name, f64(t), ref[rk], t2)


def test_autograd_hvp_of_a_loss_nonlinear_in_o():
    # L = |O|^2 / 2: grad L = J^T O, so H v = J^T (J v) + [BoB with dO = O and
    # cotangents v]; J v, the Jacobian-vector product of O along v, is BoB's
    # g_dO output, and J^T (J v) is the backward with dO = J v
    import fwd_bwd_double_amd as fbd
    w = synthetic.Workload("autograd-gn-fp32", 1, 2, 160, 64, "fp32", 6400, causal=True,
                           qkv_std=0.5)
    x, g, a = inputs(w)
    say(f"[gpu] autograd |O|^2/2 B=1 H=2 N=160 fp32")
    q, k, v = leaves(g, 2)
    o = fbd.attention(q, k, v, scale=w.scale)
    loss = 0.5 * (o * o).sum()
    gq, gk, gv = torch.autograd.grad(loss, (q, k, v), create_graph=True)
    s = (gq * g["g_dq"]).sum() + (gk * g["g_dk"]).sum() + (gv * g["g_dv"]).sum()
    hq, hk, hv = torch.autograd.grad(s, (q, k, v))
    torch.cuda.synchronize()
    O, _ = oracle.fwd(a["q"], a["k"], a["v"])
    r1 = oracle.bob(a["q"], a["k"], a["v"], O, a["g_dq"], a["g_dk"], a["g_dv"])
    r2 = oracle.bwd(a["q"], a["k"], a["v"], r1["gdO"])
    f64 = synthetic.to_f64
    for name, t, rk in (("dQ", gq, "dQ"), ("dK", gk, "dK"), ("dV", gv, "dV")):
        check(name, f64(t.detach()), oracle.bwd(a["q"], a["k"], a["v"], O)[rk], 1e-5)
    for name, t, k1, k2 in (("Hv_q", hq, "gQ", "dQ"), ("Hv_k", hk, "gK", "dK"),
                            ("Hv_v", hv, "gV", "dV")):
        check(name, f64(t), r1[k1] + r2[k2], 1e-5)
