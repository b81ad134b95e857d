"""Exact causal multi-head softmax attention for MI355X (gfx950): forward,
backward with optional GProj, and backward-over-backward, as hand-written HIP
kernels behind the C ABI of libfbd.so (include/fbd.h).

    from fwd_bwd_double_amd import attn_fwd, attn_bwd, attn_bob, attn_hvp
    from fwd_bwd_double_amd import attn_fwd_fp8     # E4M3 forward, optional rotation
    from fwd_bwd_double_amd import attention        # torch op, differentiable twice

The functions take torch tensors shaped (B, H, N, 64) in bf16 or fp32 on the
GPU; torch provides device memory and the stream, the kernels do the work.
"""
from ._lib import (AttnError, attn_bob, attn_bob_noalloc, attn_bwd, attn_fwd,  # noqa: F401
                   attn_hvp, BOB_NOALLOC_MAX_ROWS,
                   bob_workspace_bytes, bwd_workspace_bytes, hvp_workspace_bytes, load,
                   bob_ex_workspace_bytes, bwd_ex_workspace_bytes,
                   LIB_PATH, attn_fwd_fp8, attn_fp8_quantize, attn_fwd_fp8_codes, fp8_parts,
                   fp8_workspace_bytes)
from .autograd import attention  # noqa: F401

__all__ = ["attn_fwd", "attn_bwd", "attn_bob", "attn_bob_noalloc", "BOB_NOALLOC_MAX_ROWS",
           "attn_hvp", "bwd_workspace_bytes",
           "bob_workspace_bytes", "hvp_workspace_bytes", "bwd_ex_workspace_bytes",
           "bob_ex_workspace_bytes", "AttnError", "load", "LIB_PATH",
           "attn_fwd_fp8", "attn_fp8_quantize", "attn_fwd_fp8_codes", "fp8_parts",
           "fp8_workspace_bytes", "attention"]
