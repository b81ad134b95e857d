"""FP8 (E4M3) forward with optional incoherent processing, as a CPU model.

TEST INFRASTRUCTURE (see the oracle package header).

Source: the FlashAttention explainer page (marketmaker.cc,
flash-attention-trading-models), section "FA3: the Hopper mechanics", item 3
(FP8 with incoherent processing).  Naive FP8 attention suffers from outliers.
FA3 applies a random rotation to the vectors before quantising them block by
block, which spreads an outlier's magnitude over all coordinates.  The same
page's section on checking precision says to measure a low-precision path
against an fp64 reference on identical inputs.  ``fwd_fp8`` is that reference
for the FP8 path.

The page leaves the details open.  The readings taken here:
  * Format: OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals, largest finite 448, no infinities).  Rounding is to nearest,
    ties to even.
  * Rotation: R = diag(s) H / 8.  H is the 64 x 64 Sylvester Hadamard matrix,
    H[i][j] = (-1)^popcount(i & j), and s is a vector of random signs passed
    in as a 64-bit mask (bit i set: s_i = -1).  R is orthogonal, so
    (Q R)(K R)^T = Q K^T.  It is applied to the rows of Q and K only; the
    output is linear in V, so V is quantised as it is.
  * The rotated values are the exact products x R, formed here in fp64 as
    a plain matrix product with R written out from its definition (no fast
    transform).  A kernel that rotates in fp32 rounds them; the tests allow
    a code one step away exactly where the exact value lies within that
    rounding's bound of a rounding boundary (and an exponent one away where
    a block's largest magnitude lies that close to a power of two).
  * Blocks: Q and K get one scale per 64 consecutive rows of a head.  V gets
    one scale per column of a head.  P V is accumulated per output column
    over all keys, so a column scale costs one multiply at the end.  Scales
    are powers of two, 2^e with e = floor(log2 amax) - 7, which puts the
    block's largest magnitude in [128, 256).  Scaling by a power of two is
    exact, so a code depends only on the value it encodes.
  * The attention itself is computed exactly (fp64) on the dequantised
    operands.  A kernel also rounds the probabilities P to E4M3 before
    multiplying them by V.  That rounding happens against a running max, so
    it is bounded (``fwd_fp8`` returns the weight the bound needs) rather
    than reproduced.
"""
from __future__ import annotations

import numpy as np

from .attention import fwd as _fwd_exact
from .attention import _visible

E4M3_MAX = 448.0
ROW_BLOCK = 64


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte, as float64 (0x7F and 0xFF are NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    val = np.where(ef == 0, mf / 8.0 * 2.0 ** -6, (1.0 + mf / 8.0) * np.exp2(ef - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code of each value, rounded to nearest with ties to even.
    Magnitudes above 448 raise (the kernels scale every block below 256)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("e4m3_encode: magnitude above 448")
    # quantum of the binade holding a: 2^(e - 3) with e = max(floor(log2 a), -6)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # floor(log2) from a float log can be off by one near powers of two
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.maximum(e, -6.0)
    q = np.rint(a / np.exp2(e - 3))          # numpy rounds halves to even
    # q in [8, 16] for normals (16 carries into the next binade), [0, 8] at e = -6
    carry = q >= 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    normal = q >= 8
    ef = np.where(normal, e + 7, 0).astype(np.int64)
    mf = np.where(normal, q - 8, q).astype(np.int64)
    code = (ef << 3) | mf
    if np.any(code > 0x7E):
        raise ValueError("e4m3_encode: rounds beyond 448")
    # the sign bit is kept for values that round to zero, as the format has -0
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def sign_vector(signs: int) -> np.ndarray:
    """The 64 signs s_i = -1 where bit i of the mask is set, else +1."""
    return np.array([-1.0 if (int(signs) >> i) & 1 else 1.0 for i in range(64)])


def hadamard(n: int = 64) -> np.ndarray:
    """The n x n Sylvester Hadamard matrix, H[i][j] = (-1)^popcount(i & j)."""
    i = np.arange(n)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pop = np.zeros_like(bits)
    while bits.any():
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 1, -1.0, 1.0)


def rotation(signs: int) -> np.ndarray:
    """R = diag(s) H / 8 (64 x 64, orthogonal)."""
    return sign_vector(signs)[:, None] * hadamard(64) / 8.0


def rotate(x, signs: int) -> np.ndarray:
    """Rows of x times R in fp64: the signed sums of 64 bf16 or fp32 terms
    err by at most 64 * 2^-53 * sum_k |x_k| / 8, some 2^-23 of what one fp32
    rounding of the same sums may err, so these are the exact values for
    every purpose the codes serve."""
    return np.asarray(x, dtype=np.float64) @ rotation(signs)


def block_exponent(amax) -> np.ndarray:
    """e = floor(log2 amax) - 7 (amax > 0), 0 for amax = 0: the scale 2^e puts
    amax / 2^e in [128, 256)."""
    a = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(a)          # a = m 2^ex, m in [0.5, 1)
    return np.where(a > 0, ex - 1 - 7, 0).astype(np.int64)


def quantize_rows(X, rotate_signs=None):
    """Codes and block exponents of Q or K: X is (..., N, 64); each head's
    rows are optionally rotated, then split into blocks of 64 rows (the last
    may be short) with one exponent per block.  Returns (codes uint8
    (..., N, 64), exps int64 (..., ceil(N/64)))."""
    X = np.asarray(X)
    xr = rotate(X, rotate_signs) if rotate_signs is not None else X.astype(np.float64)
    N = xr.shape[-2]
    nb = (N + ROW_BLOCK - 1) // ROW_BLOCK
    codes = np.empty(xr.shape, dtype=np.uint8)
    exps = np.empty(xr.shape[:-2] + (nb,), dtype=np.int64)
    for b in range(nb):
        blk = xr[..., b * ROW_BLOCK:(b + 1) * ROW_BLOCK, :]
        e = block_exponent(np.abs(blk).max(axis=(-2, -1)))
        exps[..., b] = e
        codes[..., b * ROW_BLOCK:(b + 1) * ROW_BLOCK, :] = e4m3_encode(
            np.ldexp(blk, -e[..., None, None]))
    return codes, exps


def quantize_cols(X):
    """Codes and per-column exponents of V: X is (..., N, 64); each head's
    column gets one exponent from its largest magnitude over all N rows.
    Returns (codes uint8 (..., N, 64), exps int64 (..., 64))."""
    x32 = np.asarray(X).astype(np.float32)
    e = block_exponent(np.abs(x32).max(axis=-2))
    codes = e4m3_encode(np.ldexp(x32.astype(np.float64), -e[..., None, :]))
    return codes, e


def dequantize_rows(codes, exps):
    """Inverse of ``quantize_rows`` (without undoing the rotation)."""
    v = e4m3_decode(codes)
    e = np.repeat(np.asarray(exps), ROW_BLOCK, axis=-1)[..., :v.shape[-2]]
    return np.ldexp(v, e[..., None])


def dequantize_cols(codes, exps):
    return np.ldexp(e4m3_decode(codes), np.asarray(exps)[..., None, :])


def fwd_fp8(Q, K, V, causal=True, scale=None, signs=None, window=0, docs=None,
            block_mask=None):
    """FP8 forward model.  Q is (B, H, N, 64); K, V are (B, Hkv, N, 64) with
    H a multiple of Hkv.  ``signs`` is None for plain (naive) block
    quantisation, else the rotation's 64-bit sign mask.  window, docs and
    block_mask are the masks of the exact forward (attention.fwd); a row they
    leave empty has O = 0, LSE = -inf and zero weights.

    Returns a dict:
      O, LSE   exact attention on the dequantised operands (fp64);
      W        sum_j P_ij |V^_jd| per row and column, P the exact
               probabilities: rounding P to E4M3 (relative error <= 2^-4 in
               the normal range) adds at most 2^-4 W to O;
      U        max_j P_ij * sum_j |V^_jd| over the visible keys: the weight
               of the absolute error of probabilities rounded in the
               subnormal range (a kernel that quantises 256 P relative to a
               running max adds at most 2^-18 U to O there);
      A        max over visible keys j of sum_d |Q^_id| |K^_jd|: a sum of
               the 64 products with relative precision eps errs by at most
               eps A_i in S_ij, hence by c eps A_i in LSE_i and by a factor
               of at most 2 c eps A_i in P;
      codes    {"q", "k", "v"} uint8 and {"eq", "ek", "ev"} exponents.
    """
    Q, K, V = (np.asarray(x) for x in (Q, K, V))
    B, H, N, d = Q.shape
    Hkv = K.shape[1]
    g = H // Hkv
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    cq, eq = quantize_rows(Q, signs)
    ck, ek = quantize_rows(K, signs)
    cv, ev = quantize_cols(V)
    qh = dequantize_rows(cq, eq)
    kh = np.repeat(dequantize_rows(ck, ek), g, axis=1)
    vh = np.repeat(dequantize_cols(cv, ev), g, axis=1)
    O, LSE = _fwd_exact(qh, kh, vh, causal=causal, scale=c, window=window, docs=docs,
                        block_mask=block_mask)
    W = np.empty_like(O)
    U = np.empty_like(O)
    A = np.empty_like(LSE)
    idx = np.arange(N)
    for b in range(B):
        for h in range(H):
            vis = _visible(idx, N, causal, window, None if docs is None else np.asarray(docs)[b],
                           None if block_mask is None else np.asarray(block_mask)[b])
            s = np.where(vis, c * (qh[b, h] @ kh[b, h].T), -np.inf)
            live = np.isfinite(LSE[b, h])[:, None]
            p = np.where(vis & live, np.exp(s - np.where(live, LSE[b, h][:, None], 0.0)), 0.0)
            W[b, h] = p @ np.abs(vh[b, h])
            U[b, h] = p.max(axis=1)[:, None] * (np.where(vis, 1.0, 0.0) @ np.abs(vh[b, h]))
            sa = np.abs(qh[b, h]) @ np.abs(kh[b, h]).T
            A[b, h] = np.where(vis, sa, 0.0).max(axis=1)
    return {"O": O, "LSE": LSE, "W": W, "U": U, "A": A, "scale": c,
            "codes": {"q": cq, "k": ck, "v": cv, "eq": eq, "ek": ek, "ev": ev}}
