"""Pins of the FP8 forward model (oracle/fp8.py) against things fixed outside
it: the OCP E4M3 format, as torch's float8_e4m3fn conversion implements it
(a library routine) and as codes derived by hand from the format; the
Hadamard matrix from scipy; orthogonality; exact quantisation of values the
format holds; and the direction of the explainer page's claim that rotating
before block quantisation lowers the error (section "FA3: the Hopper
mechanics", item 3)."""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from oracle import fp8

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def torch_codes(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_hand_codes():
    # 1 = 1.000 x 2^0: exponent field 7, mantissa 0 -> 0x38.  448 = 1.110 x
    # 2^8 -> 0x7E.  2^-9 is the smallest subnormal -> 0x01; 2^-10 lies halfway
    # between 0 and 2^-9 and goes to the even 0; 3 x 2^-10 lies halfway
    # between codes 1 and 2 and goes to 2.  1 + 1/16 lies halfway between
    # 1.000 and 1.001 (to 1.000); 1 + 3/16 between 1.001 and 1.010 (to
    # 1.010 = 0x3A).  240 = 1.111 x 2^7 -> 0x77.
    x = [1.0, 448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 240.0, -2.0, 0.0]
    want = [0x38, 0x7E, 0x01, 0x00, 0x02, 0x38, 0x3A, 0x77, 0xC0, 0x00]
    assert fp8.e4m3_encode(x).tolist() == want
    rounded = [1.0, 448.0, 2.0 ** -9, 0.0, 2.0 ** -8, 1.0, 1.25, 240.0, -2.0, 0.0]
    np.testing.assert_array_equal(fp8.e4m3_decode(want), np.array(rounded))
    assert np.isnan(fp8.e4m3_decode([0x7F, 0xFF])).all()


def test_encode_matches_torch_everywhere():
    # every finite code's value, every midpoint between neighbours, and a
    # log-uniform sample over the whole range, both signs
    vals = fp8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(7)
    rand = np.exp2(rng.uniform(-12, np.log2(448.0), 20000))
    x = np.concatenate([vals, mids, rand, [448.0]])
    x = np.concatenate([x, -x])
    np.testing.assert_array_equal(fp8.e4m3_encode(x), torch_codes(x))
    # decode inverts encode on every finite code
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.e4m3_encode([449.0])
    with pytest.raises(ValueError):
        fp8.e4m3_encode([np.nan])


def test_hadamard_and_rotation_match_scipy():
    # the Sylvester matrix against scipy's; the rotation against a plain
    # product with it, exactly on small integers (every fp64 step exact)
    H = scipy.linalg.hadamard(64).astype(np.float64)
    np.testing.assert_array_equal(fp8.hadamard(64), H)
    rng = np.random.default_rng(1)
    signs = 0x8000000000000001 | int(rng.integers(0, 2 ** 62))
    s = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(64)])
    xi = rng.integers(-1000, 1000, size=(5, 64)).astype(np.float64)
    np.testing.assert_array_equal(fp8.rotate(xi, signs), (xi * s) @ H / 8.0)
    np.testing.assert_array_equal(fp8.rotation(signs), np.diag(s) @ H / 8.0)


def test_rotation_is_orthogonal_with_signs():
    rng = np.random.default_rng(2)
    signs = int(rng.integers(0, 2 ** 63)) | (1 << 63)
    s = fp8.sign_vector(signs)
    assert s[63] == -1.0 and set(s.tolist()) == {-1.0, 1.0}
    R = np.diag(s) @ scipy.linalg.hadamard(64) / 8.0
    np.testing.assert_allclose(R @ R.T, np.eye(64), atol=1e-15)
    q = rng.standard_normal((40, 64))
    k = rng.standard_normal((40, 64))
    qr = fp8.rotate(q, signs)
    kr = fp8.rotate(k, signs)
    np.testing.assert_allclose(qr, q @ R, rtol=0, atol=1e-13)
    np.testing.assert_allclose(qr @ kr.T, q @ k.T, rtol=0, atol=1e-12)


def test_block_exponent_range():
    rng = np.random.default_rng(3)
    a = np.exp2(rng.uniform(-30, 30, 5000))
    a = np.concatenate([a, np.exp2(np.arange(-20, 20, dtype=np.float64))])
    e = fp8.block_exponent(a)
    r = np.ldexp(a, -e)
    assert np.all((r >= 128) & (r < 256))
    assert fp8.block_exponent(0.0) == 0


def test_quantisation_error_bound():
    # each code is the nearest value: error <= half a quantum, i.e.
    # <= 2^-4 |x| in the normal range and <= 2^-10 2^e in the subnormal one
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 3, 200, 64)) * np.exp2(rng.uniform(-8, 8, (2, 3, 1, 1)))
    x[0, 0, 5, 7] = 300.0   # an outlier sets its block's scale
    for signs in (None, 0x5A5A5A5A12345678):
        codes, exps = fp8.quantize_rows(x, signs)
        ref = x.astype(np.float32).astype(np.float64)
        if signs is not None:
            ref = fp8.rotate(x, signs)
        deq = fp8.dequantize_rows(codes, exps)
        e = np.repeat(exps, 64, axis=-1)[..., :200, None].astype(np.float64)
        bound = np.maximum(2.0 ** -4 * np.abs(ref), np.ldexp(2.0 ** -10, e.astype(np.int64)))
        assert np.all(np.abs(deq - ref) <= bound)
        # the block max lands in [128, 256) times its scale
        amax = np.abs(ref[..., :64, :]).max(axis=(-2, -1))
        r = np.ldexp(amax, -exps[..., 0])
        assert np.all((r >= 128) & (r < 256))
    codes, ev = fp8.quantize_cols(x)
    deq = fp8.dequantize_cols(codes, ev)
    ref = x.astype(np.float32).astype(np.float64)
    bound = np.maximum(2.0 ** -4 * np.abs(ref), np.ldexp(2.0 ** -10, ev[..., None, :]))
    assert np.all(np.abs(deq - ref) <= bound)


def _representable(rng, shape, per_col=False):
    """Values the format holds exactly, scaled so that every 64-row block
    (rows) or column (per_col) has its largest magnitude in [128, 256):
    quantisation then returns them unchanged."""
    codes = rng.integers(0, 0x77, size=shape).astype(np.uint8)   # magnitudes < 256
    codes |= (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)
    x = fp8.e4m3_decode(codes)
    if per_col:
        x[..., 0, :] = 128.0
        return x * np.exp2(rng.integers(-9, -5, size=shape[:-2] + (1, shape[-1])))
    for b in range(0, shape[-2], 64):
        x[..., b, 0] = -128.0
    e = rng.integers(-9, -5, size=shape[:-2] + ((shape[-2] + 63) // 64,))
    return x * np.exp2(np.repeat(e, 64, axis=-1)[..., :shape[-2], None])


@pytest.mark.parametrize("causal", [True, False])
def test_fwd_fp8_exact_on_representable_inputs(causal):
    rng = np.random.default_rng(5)
    B, H, N = 1, 2, 150
    q = _representable(rng, (B, H, N, 64))
    k = _representable(rng, (B, H, N, 64))
    v = _representable(rng, (B, H, N, 64), per_col=True)
    r = fp8.fwd_fp8(q, k, v, causal=causal, scale=0.125)
    o, lse = oracle.fwd(q, k, v, causal=causal, scale=0.125)
    np.testing.assert_array_equal(r["O"], o)
    np.testing.assert_array_equal(r["LSE"], lse)
    np.testing.assert_array_equal(fp8.e4m3_decode(r["codes"]["v"]) *
                                  np.exp2(r["codes"]["ev"])[..., None, :], v)


def test_fwd_fp8_grouped_query_and_weights():
    rng = np.random.default_rng(6)
    B, H, Hkv, N = 1, 4, 2, 90
    q = rng.standard_normal((B, H, N, 64))
    k = rng.standard_normal((B, Hkv, N, 64))
    v = rng.standard_normal((B, Hkv, N, 64))
    r = fp8.fwd_fp8(q, k, v, causal=True, scale=0.125, signs=12345)
    c = r["codes"]
    kh = oracle.expand_kv(fp8.dequantize_rows(c["k"], c["ek"]), 2)
    vh = oracle.expand_kv(fp8.dequantize_cols(c["v"], c["ev"]), 2)
    o, lse = oracle.fwd(fp8.dequantize_rows(c["q"], c["eq"]), kh, vh, causal=True, scale=0.125)
    np.testing.assert_allclose(r["O"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["LSE"], lse, rtol=0, atol=1e-12)
    # W = sum_j P |v| bounds |O| and equals it for non-negative V
    assert np.all(np.abs(r["O"]) <= r["W"] * (1 + 1e-12))
    r2 = fp8.fwd_fp8(q, k, np.abs(v), causal=True, scale=0.125, signs=12345)
    np.testing.assert_allclose(r2["O"], r2["W"], rtol=1e-12)
    # first row sees one key: U = W there
    np.testing.assert_allclose(r["U"][:, :, 0], r["W"][:, :, 0], rtol=1e-12)


def outlier_inputs(rng, B, H, N, channels=(3, 17, 40), mag=20.0):
    """N(0, 1) rows with a few large channels in Q and K (all heads)."""
    q = rng.standard_normal((B, H, N, 64))
    k = rng.standard_normal((B, H, N, 64))
    v = rng.standard_normal((B, H, N, 64))
    for ch in channels:
        q[..., ch] *= mag
        k[..., ch] *= mag
    return q, k, v


def test_rotation_lowers_error_with_outlier_channels():
    """The page reports a lower error for rotated than for naive block
    quantisation when the inputs carry outliers.  Measured here against the
    exact forward on the unquantised inputs (the model keeps P exact)."""
    rng = np.random.default_rng(8)
    q, k, v = outlier_inputs(rng, 1, 2, 256)
    scale = 0.125 / 20.0
    o, _ = oracle.fwd(q, k, v, causal=True, scale=scale)
    err = {}
    for name, signs in (("naive", None), ("rotated", 0x0F1E2D3C4B5A6978)):
        r = fp8.fwd_fp8(q, k, v, causal=True, scale=scale, signs=signs)
        err[name] = np.linalg.norm(r["O"] - o) / np.linalg.norm(o)
    assert err["rotated"] < err["naive"] / 1.5, err


def test_fwd_fp8_masks_exact_on_representable_inputs():
    # the masks of the exact forward carry over: on inputs the format holds
    # exactly, the FP8 model with a window, documents or a block mask is the
    # exact masked forward, and an emptied row has zero weights
    rng = np.random.default_rng(9)
    B, H, N = 1, 2, 300
    q = _representable(rng, (B, H, N, 64))
    k = _representable(rng, (B, H, N, 64))
    v = _representable(rng, (B, H, N, 64), per_col=True)
    starts = np.zeros((1, N), dtype=np.int64)      # documents [0,90) [90,200) [200,300)
    starts[0, 90:200] = 90
    starts[0, 200:] = 200
    bm = np.array([[[0, 0, 0], [1, 1, 0], [1, 0, 1]]], dtype=np.uint8)
    for kw in (dict(window=37), dict(docs=starts), dict(block_mask=bm)):
        r = fp8.fwd_fp8(q, k, v, causal=True, scale=0.125, **kw)
        o, lse = oracle.fwd(q, k, v, causal=True, scale=0.125, **kw)
        np.testing.assert_array_equal(r["O"], o)
        np.testing.assert_array_equal(r["LSE"], lse)
    assert np.all(np.isneginf(r["LSE"][..., :128]))
    assert np.all(r["W"][..., :128, :] == 0) and np.all(r["A"][..., :128] == 0)


def test_fp8_weights_against_brute_force():
    """W, U and A of fwd_fp8 against their definitions written as plain loops
    over (row, key, channel) on a tiny case (dequantised operands from the
    returned codes, probabilities from math.exp of the masked scores):
      W_id = sum_j P_ij |v_jd|,   U_id = max_j P_ij * sum_{j visible} |v_jd|,
      A_i  = max_{j visible} sum_d |q_id| |k_jd|."""
    import math
    rng = np.random.default_rng(10)
    B, H, N = 1, 1, 7
    q = rng.standard_normal((B, H, N, 64)) * 2
    k = rng.standard_normal((B, H, N, 64))
    v = rng.standard_normal((B, H, N, 64))
    for causal, kw in ((True, {}), (False, {}), (True, dict(window=3))):
        r = fp8.fwd_fp8(q, k, v, causal=causal, scale=0.2, signs=0xDEADBEEF, **kw)
        c = r["codes"]
        qh = fp8.dequantize_rows(c["q"], c["eq"])[0, 0]
        kh = fp8.dequantize_rows(c["k"], c["ek"])[0, 0]
        vh = fp8.dequantize_cols(c["v"], c["ev"])[0, 0]
        win = kw.get("window", 0)
        for i in range(N):
            vis = [j for j in range(N) if (not causal or (j <= i and (win == 0 or j > i - win)))]
            s = {j: 0.2 * sum(qh[i, t] * kh[j, t] for t in range(64)) for j in vis}
            mx = max(s.values())
            e = {j: math.exp(s[j] - mx) for j in vis}
            tot = sum(e.values())
            p = {j: e[j] / tot for j in vis}
            for dd in range(64):
                w = sum(p[j] * abs(vh[j, dd]) for j in vis)
                u = max(p.values()) * sum(abs(vh[j, dd]) for j in vis)
                assert abs(r["W"][0, 0, i, dd] - w) <= 1e-12 * max(w, 1e-300)
                assert abs(r["U"][0, 0, i, dd] - u) <= 1e-12 * max(u, 1e-300)
            a = max(sum(abs(qh[i, t]) * abs(kh[j, t]) for t in range(64)) for j in vis)
            assert abs(r["A"][0, 0, i] - a) <= 1e-12 * a
            o = [sum(p[j] * vh[j, dd] for j in vis) for dd in range(64)]
            np.testing.assert_allclose(r["O"][0, 0, i], o, rtol=0, atol=1e-12)
            assert abs(r["LSE"][0, 0, i] - (mx + math.log(tot))) <= 1e-12 * (1 + abs(mx))
