"""GPU parity of the FP8 forward (quantisation pre-pass and E4M3 forward)
against the oracle's FP8 model (oracle/fp8.py).

Codes and exponents: without rotation both sides quantise the same fp32
values and must agree bit for bit.  With rotation the oracle quantises the
exact values x R, while the kernel rotates in fp32 with the fast transform;
its codes must equal the oracle's except where the exact value lies within
that transform's rounding bound of a rounding boundary, and there be the code
on the other side (check_row_codes).  The output differs from the
model's exact attention on the dequantised operands by the kernel's E4M3
rounding of the probabilities (at most 2^-4 W + 2^-18 U elementwise, W and U
from the model), by the limited precision of the matrix instruction's sum
(through A), by fp32 accumulation and by the output's own rounding."""
import numpy as np
import pytest
import torch

import fwd_bwd_double_amd as fbd
import oracle
import synthetic
from gpu_util import block_masks, doc_starts, rel_l2, say
from oracle import fp8
from synthetic import to_f64

pytestmark = pytest.mark.gpu


def unpermute_vt(vt, N):
    """(B, Hkv, 64, NP) stored V codes -> (B, Hkv, N, 64): stored word w of a
    64-key group holds keys 4s .. 4s+3, s = 2 (w % 8) + w / 8."""
    B, Hk, d, NP = vt.shape
    g = vt.reshape(B, Hk, d, NP // 64, 16, 4)
    w = np.arange(16)
    s = 2 * (w % 8) + w // 8
    out = np.empty_like(g)
    out[..., s, :] = g[..., w, :]
    return out.reshape(B, Hk, d, NP).transpose(0, 1, 3, 2)[:, :, :N, :], \
        out.reshape(B, Hk, d, NP)[..., N:]


def quantize_on_gpu(x, signs):
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    ws = fbd.attn_fp8_quantize(q, k, v, signs)
    torch.cuda.synchronize()
    B, H, N, _ = q.shape
    parts = fbd.fp8_parts(ws, B, H, k.shape[1], N)
    return ws, {k_: t.cpu().numpy() for k_, t in parts.items()}


U32 = 2.0 ** -24


def check_row_codes(codes, exps, x, signs, label):
    """Q or K codes and block exponents from the kernel against the oracle's
    quantisation of the same rows (x: fp64 values of the inputs, (..., N, 64)).

    Unrotated: bit for bit.  Rotated: the kernel forms each rotated value as
    a signed sum of the row's 64 inputs (times exact signs) with the fast
    transform, six rounded fp32 additions on any path, then multiplies by
    1/8 exactly; so its value lies within beta = gamma_6 sum_k |x_k| / 8 of
    the exact x R (gamma_6 = 6u / (1 - 6u), u = 2^-24).  Hence:
      * a block exponent may differ from the exact one by one only where the
        block's exact largest magnitude lies within its largest beta of a
        power of two;
      * each code, taken at the kernel's exponent, must be the code of some
        value within beta of the exact one: one of encode(z - beta) and
        encode(z + beta) (rounding is monotone, and beta is far below the
        format's spacing, so that is at most one boundary).
    Returns the number of codes that differ from the oracle's."""
    cx, ex = fp8.quantize_rows(x, signs)
    if signs is None:
        np.testing.assert_array_equal(exps, ex, err_msg=label)
        np.testing.assert_array_equal(codes, cx, err_msg=label)
        return 0
    N = x.shape[-2]
    z = fp8.rotate(x, signs)
    g6 = 6 * U32 / (1 - 6 * U32)
    beta = g6 * np.abs(x).sum(axis=-1) / 8.0                     # (..., N)
    nb = exps.shape[-1]
    pad = nb * 64 - N
    zb = np.pad(np.abs(z).max(axis=-1), [(0, 0)] * (z.ndim - 2) + [(0, pad)])
    bb = np.pad(beta, [(0, 0)] * (z.ndim - 2) + [(0, pad)])
    amax = zb.reshape(zb.shape[:-1] + (nb, 64)).max(axis=-1)
    bmax = bb.reshape(bb.shape[:-1] + (nb, 64)).max(axis=-1)
    exps = np.asarray(exps).astype(np.int64)
    edge = np.abs(amax - np.exp2(np.maximum(exps, ex) + 7.0)) <= bmax
    ok_e = (exps == ex) | ((np.abs(exps - ex) == 1) & edge)
    assert ok_e.all(), (label, "block exponents", int((~ok_e).sum()))
    e_rows = np.repeat(exps, 64, axis=-1)[..., :N, None]
    zs = np.ldexp(z, -e_rows)
    bs = np.ldexp(beta[..., None] * np.ones_like(z), -e_rows)
    lo, hi = fp8.e4m3_encode(zs - bs), fp8.e4m3_encode(zs + bs)
    codes = np.asarray(codes)
    ok = (codes == lo) | (codes == hi)
    assert ok.all(), (label, "codes", int((~ok).sum()))
    ndiff = int((codes != cx).sum())
    say(f"    {label}: {codes.size} codes, {ndiff} one step from the exact rotation's "
        f"(all at rounding boundaries within the fp32 transform's bound); "
        f"{int((exps != ex).sum())} exponents differ")
    return ndiff


CODE_CASES = [(1, 1, 1, 1), (1, 2, 2, 17), (1, 2, 1, 130), (2, 4, 2, 333), (1, 3, 3, 1000)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rot", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N", CODE_CASES)
def test_codes_bit_exact(B, H, Hkv, N, rot, dtype):
    say(f"[gpu] fp8 codes B={B} H={H} Hkv={Hkv} N={N} rotate={rot} {dtype}")
    x = synthetic.fp8_inputs(8100 + N, B, H, Hkv, N, dtype, outlier_channels=(5,),
                             outlier_mag=30.0)
    signs = synthetic.sign_mask(N) if rot else None
    _, got = quantize_on_gpu(x, signs)
    a = {k: to_f64(v) for k, v in x.items()}
    check_row_codes(got["q"], got["eq"], a["q"], signs, "Q")
    check_row_codes(got["k"], got["ek"], a["k"], signs, "K")
    cv, ev = fp8.quantize_cols(a["v"])
    np.testing.assert_array_equal(got["ev"], ev)
    vt, pad = unpermute_vt(got["vt"], N)
    np.testing.assert_array_equal(vt, cv)
    assert not pad.any()


# Precision of the sum inside the E4M3 matrix instruction: its 64 products are
# not summed to fp32 accuracy.  Measured on MI355X with exact host products
# (65536 + 63 x 1 returns 65592; over 3072 random E4M3 dot products the error
# reached 2^-12.3 of the sum of |terms|); the bounds use 2^-11.
MMA_EPS = 2.0 ** -11


def fwd_bound(ref, dtype):
    # P rounding, plus the score sums (relative change of P at most
    # 2 c eps A) and fp32 accumulation of the output
    ds = 2 * ref["scale"] * MMA_EPS * ref["A"][..., None]
    b = 2.0 ** -4 * ref["W"] + 2.0 ** -18 * ref["U"] + (ds + 1e-5) * (ref["W"] + np.abs(ref["O"]))
    if dtype == "bf16":
        b = b + 2.0 ** -8 * np.abs(ref["O"])
    return b


def check_fwd(o, lse, ref, dtype):
    og, lg = to_f64(o), to_f64(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg) | np.isneginf(ref["LSE"]))
    bound = fwd_bound(ref, dtype)
    err = np.abs(og - ref["O"])
    worst = float(np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                           np.where(err > 0, np.inf, 0.0)).max())
    fin = np.isfinite(ref["LSE"])
    e_o, e_l = rel_l2(og, ref["O"]), rel_l2(lg[fin], ref["LSE"][fin])
    dl = float(np.abs(lg[fin] - ref["LSE"][fin]).max()) if fin.any() else 0.0
    say(f"    O rel-L2 {e_o:.3e}, max err / bound {worst:.3f}; LSE rel-L2 {e_l:.2e} "
        f"max abs {dl:.2e}; empty rows {int((~fin).sum())}")
    assert worst <= 1.0, worst
    # LSE: the score sums (c eps A) plus exp2 / log2 rounding; rows a block
    # mask leaves empty are -inf on both sides
    empty = np.isneginf(ref["LSE"])
    assert np.array_equal(np.isneginf(lg), empty)
    lsafe = np.where(empty, 0.0, ref["LSE"])
    lb = ref["scale"] * MMA_EPS * ref["A"] + 4e-6 * (1 + np.abs(lsafe))
    lw = float((np.abs(np.where(empty, 0.0, lg) - lsafe) / lb).max())
    say(f"    LSE max err / bound {lw:.3f}")
    assert lw <= 1.0, lw
    return e_o


FWD_CASES = [(1, 1, 1, 1, True), (1, 2, 2, 17, True), (1, 2, 2, 17, False),
             (1, 2, 1, 200, True), (2, 2, 2, 333, False), (1, 4, 2, 1000, True),
             (1, 1, 1, 1000, False)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rot", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,causal", FWD_CASES)
def test_forward_matches_model(B, H, Hkv, N, causal, rot, dtype):
    say(f"[gpu] fp8 fwd B={B} H={H} Hkv={Hkv} N={N} causal={causal} rotate={rot} {dtype}")
    x = synthetic.fp8_inputs(8200 + N, B, H, Hkv, N, dtype, outlier_channels=(9, 33),
                             outlier_mag=10.0)
    signs = synthetic.sign_mask(7 * N) if rot else None
    scale = 0.125 / 10.0
    g = {k: v.cuda() for k, v in x.items()}
    o, lse = fbd.attn_fwd_fp8(g["q"], g["k"], g["v"], causal=causal, scale=scale, signs=signs)
    torch.cuda.synchronize()
    a = {k: to_f64(v) for k, v in x.items()}
    ref = fp8.fwd_fp8(a["q"], a["k"], a["v"], causal=causal, scale=scale, signs=signs)
    check_fwd(o, lse, ref, dtype)


def test_full_size_sampled_heads():
    """The bf16 benchmark shape B4 H12 N4096, causal, rotated; all codes
    checked, the output on two heads."""
    B, H, N = 4, 12, 4096
    say(f"[gpu] fp8 full size B={B} H={H} N={N}")
    x = synthetic.fp8_inputs(8300, B, H, H, N, "bf16", std=0.5)
    signs = synthetic.sign_mask(8300)
    g = {k: v.cuda() for k, v in x.items()}
    ws = fbd.attn_fp8_quantize(g["q"], g["k"], g["v"], signs)
    o, lse = fbd.attn_fwd_fp8_codes(ws, B, H, H, N, torch.bfloat16, True, 0.125)
    torch.cuda.synchronize()
    parts = {k: t.cpu().numpy() for k, t in fbd.fp8_parts(ws, B, H, H, N).items()}
    a = {k: to_f64(v) for k, v in x.items()}
    check_row_codes(parts["q"], parts["eq"], a["q"], signs, "Q")
    check_row_codes(parts["k"], parts["ek"], a["k"], signs, "K")
    for (b, h) in [(0, 0), (3, 11)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = fp8.fwd_fp8(a["q"][sl], a["k"][sl], a["v"][sl], causal=True, scale=0.125,
                          signs=signs)
        say(f"  head ({b},{h})")
        check_fwd(o[sl], lse[sl], ref, "bf16")


def test_error_study_rotation():
    """Explainer page, section "FA3: the Hopper mechanics", item 3: rotating
    before block quantisation lowers the error when Q and K carry outliers.
    Error of the GPU FP8 forward against the exact fp64 forward on the
    original inputs, naive and rotated, with the bf16 forward beside them."""
    B, H, N = 1, 4, 2048
    res = {}
    for mag in (1.0, 20.0):
        x = synthetic.fp8_inputs(8400, B, H, H, N, "bf16", outlier_channels=(3, 17, 40),
                                 outlier_mag=mag)
        scale = 0.125 / mag
        g = {k: v.cuda() for k, v in x.items()}
        a = {k: to_f64(v) for k, v in x.items()}
        ref, _ = oracle.fwd(a["q"], a["k"], a["v"], causal=True, scale=scale)
        ob, _ = fbd.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=scale)
        on, _ = fbd.attn_fwd_fp8(g["q"], g["k"], g["v"], causal=True, scale=scale)
        orot, _ = fbd.attn_fwd_fp8(g["q"], g["k"], g["v"], causal=True, scale=scale,
                                   signs=synthetic.sign_mask(8400))
        torch.cuda.synchronize()
        e = {n: rel_l2(to_f64(t), ref) for n, t in (("bf16", ob), ("fp8", on), ("fp8+rot", orot))}
        m = {n: float(np.abs(to_f64(t) - ref).max() / np.abs(ref).max())
             for n, t in (("bf16", ob), ("fp8", on), ("fp8+rot", orot))}
        say(f"  outlier x{mag:g}: rel-L2 " + ", ".join(f"{k} {v:.3e}" for k, v in e.items()) +
            "; max rel " + ", ".join(f"{k} {v:.3e}" for k, v in m.items()) +
            f"; naive / rotated {e['fp8'] / e['fp8+rot']:.2f}")
        res[mag] = e
    assert res[20.0]["fp8+rot"] < res[20.0]["fp8"] / 1.5
    assert res[1.0]["fp8+rot"] < 0.1 and res[1.0]["fp8"] < 0.1


def test_workspace_errors():
    x = synthetic.fp8_inputs(1, 1, 2, 2, 64)
    g = {k: v.cuda() for k, v in x.items()}
    small = torch.empty(16, device="cuda", dtype=torch.uint8)
    with pytest.raises(ValueError):
        fbd.attn_fp8_quantize(g["q"], g["k"], g["v"], None, small)
    with pytest.raises(fbd.AttnError):
        fbd.attn_fwd_fp8_codes(small, 1, 2, 2, 64)


MASK_CASES = [("window", 333, 50, 0, None, 2, 2), ("docs", 1000, 0, 150, None, 2, 2),
              ("block", 300, 0, 0, 0.4, 2, 1), ("all", 1000, 200, 300, 0.6, 4, 2)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("name,N,window,mean_len,density,H,Hkv", MASK_CASES)
def test_forward_masks(name, N, window, mean_len, density, H, Hkv, dtype):
    """The FP8 forward under the bf16 forward's masks: sliding window, packed
    documents, block-sparse (with rows left empty) and all three together."""
    B = 2
    say(f"[gpu] fp8 masks {name} B={B} H={H} Hkv={Hkv} N={N} window={window} "
        f"docs={mean_len} density={density} {dtype}")
    x = synthetic.fp8_inputs(8500 + N, B, H, Hkv, N, dtype, outlier_channels=(9,),
                             outlier_mag=5.0)
    signs = synthetic.sign_mask(8500 + N)
    docs = doc_starts(B, N, 81 + N, mean_len) if mean_len else None
    bm = block_masks(B, N, 33 + N, density, False) if density else None
    g = {k: v.cuda() for k, v in x.items()}
    o, lse = fbd.attn_fwd_fp8(
        g["q"], g["k"], g["v"], causal=True, scale=0.125 / 5, signs=signs, window=window,
        doc_start=None if docs is None else torch.from_numpy(docs.astype(np.int32)).cuda(),
        block_mask=None if bm is None else torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    a = {k: to_f64(v) for k, v in x.items()}
    ref = fp8.fwd_fp8(a["q"], a["k"], a["v"], causal=True, scale=0.125 / 5, signs=signs,
                      window=window, docs=docs, block_mask=bm)
    check_fwd(o, lse, ref, dtype)
