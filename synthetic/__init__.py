"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and casts them. It holds none of the
attention arithmetic, so both the HIP path (through the tests and the bench)
and the fp64 oracle can take their inputs from it without sharing any of the
method's code.

Recipe (one per workload, see ``WORKLOADS``):
  * generator: NumPy ``PCG64`` seeded with ``SeedSequence(seed)`` and spawned
    into eight independent streams in the fixed order
    ``[Q, K, V, dO, g_dQ, g_dK, g_dV, mu]``;
  * each tensor is drawn as fp64 standard normals in C order ``(B, H, N, d)``,
    multiplied by its scale, cast to fp32 and then, for bf16 workloads, cast to
    bf16 with round-to-nearest-even (torch's cast);
  * the large-key workload shifts every key by one shared vector ``mu`` of
    norm ``mean_norm`` and multiplies the queries by the power of two ``tau``.

The shapes follow the GPT-2-Small attention head (d = 64, H = 12) used for the
isolated-layer test on the FlashBoB page (rit.work, flashbob-second-order-attention,
section "Two scalar states replace quadratic tensors"); the large-key regime
follows the GProj page (rit.work, flashattention-bf16-gradient-gproj, section
"How a zero sum turns into a false gradient").
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np
import torch

STREAMS = ("q", "k", "v", "do", "g_dq", "g_dk", "g_dv", "mu")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "bf16" or "fp32"
    seed: int
    causal: bool = True
    qkv_std: float = 1.0  # std of Q, K, V draws
    do_std: float = 1.0   # std of dO
    cot_std: float = 1.0  # std of the BoB cotangents g_dQ, g_dK, g_dV
    # large-key regime: K = z + mu with |mu| = mean_norm, Q = tau * q
    mean_norm: float = 0.0
    tau: float = 1.0
    ops: Tuple[str, ...] = ("fwd", "bwd", "bob")

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads.  Seeds are 1000 + the workload's number.
WORKLOADS: Dict[int, Workload] = {
    1: Workload("causal-fp32-B1H2N128", 1, 2, 128, 64, "fp32", 1001,
                ops=("fwd", "bwd", "bob")),
    2: Workload("gpt2s-layer-B8H12N1024", 8, 12, 1024, 64, "bf16", 1002,
                qkv_std=0.5, do_std=1.0, ops=("fwd", "bwd")),
    # tau is a parameter: the value used by the tests is the smallest power of
    # two that makes most rows near one-hot, chosen by a script over the oracle
    # and stored with the golden fixtures.
    3: Workload("large-key-gproj-B1H12N16384", 1, 12, 16384, 64, "bf16", 1003,
                qkv_std=1.0, do_std=1.0, mean_norm=8.0, tau=1.0,
                ops=("fwd", "bwd")),
    4: Workload("bob-B4H12N4096", 4, 12, 4096, 64, "bf16", 1004,
                qkv_std=0.5, do_std=0.5, cot_std=1.0, ops=("fwd", "bwd", "bob")),
    5: Workload("bob-long-B1H12N262144", 1, 12, 262144, 64, "bf16", 1005,
                qkv_std=0.5, do_std=0.5, cot_std=1.0, ops=("fwd", "bob")),
}


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return {name: np.random.Generator(np.random.PCG64(child))
            for name, child in zip(STREAMS, ss.spawn(len(STREAMS)))}


def _cast(x64: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x64.astype(np.float32)))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)   # round-to-nearest-even
    return t


def _draw(rng, shape, std, dtype, shift=None, chunk_elems: int = 1 << 22):
    """std * N(0,1) (+ shift, a length-d vector) in C order, drawn in row
    chunks to bound the fp64 memory; chunking does not change the values."""
    B, H, N, d = shape
    out = torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    flat = out.view(B * H * N, d)
    rows = B * H * N
    step = max(1, chunk_elems // d)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = rng.standard_normal((r1 - r0, d))
        if std != 1.0:
            x *= std
        if shift is not None:
            x += shift
        flat[r0:r1] = _cast(x, dtype)
    return out


def make_inputs(w: Workload, which=("q", "k", "v", "do", "g_dq", "g_dk", "g_dv")
                ) -> Dict[str, torch.Tensor]:
    """Draw the requested tensors of workload ``w`` as CPU torch tensors of the
    workload dtype, shaped (B, H, N, d).  Every tensor comes from its own
    stream, so asking for a subset does not change the values drawn."""
    rs = _streams(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    out: Dict[str, torch.Tensor] = {}
    mu = None
    if w.mean_norm > 0.0:
        u = rs["mu"].standard_normal(w.d)
        mu = u * (w.mean_norm / np.linalg.norm(u))
    for name in which:
        if name in ("q", "k", "v"):
            std = w.qkv_std
        elif name == "do":
            std = w.do_std
        else:
            std = w.cot_std
        if name == "q":
            std = std * w.tau
        out[name] = _draw(rs[name], shape, std, w.dtype,
                          shift=mu if name == "k" else None)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a CPU or GPU tensor (bf16 and fp32 widen exactly)."""
    return t.detach().to("cpu", torch.float64).numpy()


def fp8_inputs(seed: int, B: int, H: int, Hkv: int, N: int, dtype: str = "bf16",
               std: float = 1.0, outlier_channels=(), outlier_mag: float = 1.0
               ) -> Dict[str, torch.Tensor]:
    """Q (B, H, N, 64), K and V (B, Hkv, N, 64) for the FP8 forward: std * N(0, 1)
    from the q, k, v streams of ``seed``; the head-dimension channels listed in
    ``outlier_channels`` of Q and K are multiplied by ``outlier_mag`` before the
    cast (a few large channels, the outlier pattern rotation is meant for)."""
    rs = _streams(seed)
    out = {}
    for name, heads in (("q", H), ("k", Hkv), ("v", Hkv)):
        x = rs[name].standard_normal((B, heads, N, 64)) * std
        if name != "v":
            for ch in outlier_channels:
                x[..., ch] *= outlier_mag
        out[name] = _cast(x, dtype)
    return out


def sign_mask(seed: int) -> int:
    """A random 64-bit sign mask (the rotation's random signs) from ``seed``."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return int(rng.integers(0, 2 ** 63)) * 2 + int(rng.integers(0, 2))


def rademacher(seed: int, shape, dtype: str = "fp32") -> torch.Tensor:
    """Independent random signs (+1 / -1) of the given shape from ``seed``: the
    probes of a Hutchinson estimate of a Hessian diagonal."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = np.where(rng.integers(0, 2, size=shape) == 1, 1.0, -1.0)
    return _cast(x, dtype)
