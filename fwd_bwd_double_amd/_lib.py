"""ctypes binding of libfbd.so.

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity), their device pointers and torch's current HIP stream are handed to
the C ABI, and the status is turned into an exception.  Every step of the
computation runs in the library's HIP kernels; if the library is missing or
fails to load, every call raises -- there is no other implementation here.

torch is imported before the library is loaded so that the HIP runtime torch
already holds (same soname) is the one the library binds to.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfbd.so")

ATTN_BF16, ATTN_F32 = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported dtype or shape",
          3: "pointer not 16-byte aligned", 4: "workspace missing or too small",
          5: "HIP kernel launch failed"}


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        msg = f"{fn}: {STATUS.get(status, 'unknown status')} (status {status})"
        if status == 5:
            msg += f", hipError {hip_error}"
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run `python -m fwd_bwd_double_amd.build`)")
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
    i64, f32, vp, i32, sz = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.attn_fwd.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, i32, f32, vp, vp, vp]
    lib.attn_fwd.restype = i32
    lib.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, i32, f32, i32,
                             vp, vp, vp, vp, sz, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bob_workspace_bytes.argtypes = [i64, i64, i64]
    lib.attn_bob_workspace_bytes.restype = sz
    lib.attn_bob.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                             f32, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_bob.restype = i32
    lib.attn_bwd_passes.argtypes = [i32] + lib.attn_bwd.argtypes
    lib.attn_bwd_passes.restype = i32
    lib.attn_bob_passes.argtypes = [i32] + lib.attn_bob.argtypes
    lib.attn_bob_passes.restype = i32
    lib.attn_bob_noalloc.argtypes = lib.attn_bob.argtypes[:-3] + [vp]
    lib.attn_bob_noalloc.restype = i32
    for fn in (lib.attn_bwd_ex_workspace_bytes, lib.attn_bob_ex_workspace_bytes):
        fn.argtypes = [i64, i64, i64, i64]
        fn.restype = sz
    # extended forms: Hkv after H; the window, doc_start and block_mask after causal
    lib.attn_fwd_ex.argtypes = [i32, i64, i64, i64, i64, i64, vp, vp, vp, i32, i64, vp, vp, f32,
                                vp, vp, vp]
    lib.attn_fwd_ex.restype = i32
    a = lib.attn_bwd.argtypes
    lib.attn_bwd_ex.argtypes = a[:3] + [i64] + a[3:12] + [i64, vp, vp] + a[12:]
    lib.attn_bwd_ex.restype = i32
    a = lib.attn_bob.argtypes
    lib.attn_bob_ex.argtypes = a[:3] + [i64] + a[3:15] + [i64, vp, vp] + a[15:16] + [i32] + a[16:]
    lib.attn_bob_ex.restype = i32
    lib.attn_hvp_workspace_bytes.argtypes = [i64, i64, i64]
    lib.attn_hvp_workspace_bytes.restype = sz
    lib.attn_hvp.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32, f32, i32,
                             vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_hvp.restype = i32
    lib.attn_hvp_ex_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.attn_hvp_ex_workspace_bytes.restype = sz
    lib.attn_hvp_ex.argtypes = ([i32, i64, i64, i64, i64, i64] + [vp] * 7 + [i32, i64, vp, vp, f32, i32]
                                + [vp] * 10 + [sz, vp])
    lib.attn_hvp_ex.restype = i32
    # FP8 forward
    u64 = ctypes.c_uint64
    lib.attn_fp8_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.attn_fp8_workspace_bytes.restype = sz
    lib.attn_fp8_workspace_layout.argtypes = [i64, i64, i64, i64, ctypes.POINTER(sz)]
    lib.attn_fp8_workspace_layout.restype = i32
    lib.attn_fp8_quantize.argtypes = [i32, i64, i64, i64, i64, i64, vp, vp, vp, i32, u64, vp, sz,
                                      vp]
    lib.attn_fp8_quantize.restype = i32
    lib.attn_fwd_fp8.argtypes = [i32, i64, i64, i64, i64, i64, vp, sz, i32, i64, vp, vp, f32, vp,
                                 vp, vp]
    lib.attn_fwd_fp8.restype = i32
    lib.attn_status_str.argtypes = [i32]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = i32
    _lib = lib
    return lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; bf16 or fp32 only")


def _check(name: str, t: torch.Tensor, like: torch.Tensor, dtype=None, shape=None):
    """t is a dense tensor of the given dtype and shape (default: like's) on
    like's GPU.  The kernels read every tensor as a dense (.., N, d) array
    from its data pointer, so a strided view (a slice of a packed tensor, a
    permutation) is rejected, never reinterpreted."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != (like.dtype if dtype is None else dtype):
        raise TypeError(f"{name} has dtype {t.dtype}")
    if tuple(t.shape) != tuple(like.shape if shape is None else shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != like.device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU device of q ({like.device})")


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _raise(fn: str, st: int):
    if st != 0:
        raise AttnError(fn, st, load().attn_last_hip_error())


def _kv_heads(q: torch.Tensor, k: torch.Tensor) -> int:
    """Key/value heads of k: 1 <= Hkv <= H and H % Hkv == 0 (grouped-query
    attention when Hkv < H)."""
    if k.dim() != 4:
        raise ValueError("k must be shaped (B, Hkv, N, d)")
    H, Hkv = q.shape[1], k.shape[1]
    if Hkv < 1 or Hkv > H or H % Hkv:
        raise ValueError(f"k has {Hkv} heads; it must divide q's {H}")
    return Hkv


def _kv_shape(q: torch.Tensor, Hkv: int):
    B, _, N, d = q.shape
    return (B, Hkv, N, d)


def _bmask(q: torch.Tensor, block_mask) -> Optional[int]:
    """Device pointer of a (B, nb, nb) uint8 block mask (nb = ceil(N / 128)),
    or None."""
    if block_mask is None:
        return None
    B, _, N, _ = q.shape
    nb = (N + 127) // 128
    _check("block_mask", block_mask, q, torch.uint8, (B, nb, nb))
    return block_mask.data_ptr()


def _docs(q: torch.Tensor, doc_start) -> Optional[int]:
    """Device pointer of a (B, N) int32 doc_start tensor, or None."""
    if doc_start is None:
        return None
    B, _, N, _ = q.shape
    _check("doc_start", doc_start, q, torch.int32, (B, N))
    return doc_start.data_ptr()


def _scale(q: torch.Tensor, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)


def bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load().attn_bwd_workspace_bytes(B, H, N))


def bob_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load().attn_bob_workspace_bytes(B, H, N))


def bwd_ex_workspace_bytes(B: int, H: int, Hkv: int, N: int) -> int:
    return int(load().attn_bwd_ex_workspace_bytes(B, H, Hkv, N))


def bob_ex_workspace_bytes(B: int, H: int, Hkv: int, N: int) -> int:
    return int(load().attn_bob_ex_workspace_bytes(B, H, Hkv, N))


def hvp_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load().attn_hvp_workspace_bytes(B, H, N))


def attn_fwd(q, k, v, causal: bool = True, scale: Optional[float] = None,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             window: int = 0, doc_start: Optional[torch.Tensor] = None,
             block_mask: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O, LSE = attention(q, k, v); q shaped (B, H, N, d), k and v (B, Hkv, N, d)
    with H % Hkv == 0 (Hkv < H: grouped-query attention), bf16 or fp32.
    window > 0 (causal only): query i sees keys i - window < j <= i.
    doc_start (causal only): (B, N) int32 first position of each query's
    document (packed sequences; non-decreasing, doc_start[b, i] <= i).
    block_mask: (B, nb, nb) uint8, nb = ceil(N / 128); a zero hides the
    128 x 128 block (query block, key block) on top of the other masks."""
    lib = load()
    _check("q", q, q)
    Hkv = _kv_heads(q, k)
    for n, t in (("k", k), ("v", v)):
        _check(n, t, q, shape=_kv_shape(q, Hkv))
    B, H, N, d = q.shape
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32) if lse is None else lse
    _check("out", out, q)
    _check("lse", lse, q, torch.float32, (B, H, N))
    st = lib.attn_fwd_ex(_dt(q), B, H, Hkv, N, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                         1 if causal else 0, int(window), _docs(q, doc_start),
                         _bmask(q, block_mask), _scale(q, scale),
                         out.data_ptr(), lse.data_ptr(), _stream(q.device))
    _raise("attn_fwd", st)
    return out, lse


def attn_bwd(q, k, v, o, lse, do, causal: bool = True, scale: Optional[float] = None,
             gproj: bool = False, workspace: Optional[torch.Tensor] = None, outs=None,
             passes: int = 3, window: int = 0, doc_start: Optional[torch.Tensor] = None,
             block_mask: Optional[torch.Tensor] = None
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dQ, dK, dV of <dO, O>.  `workspace` (fp32, >= bwd_workspace_bytes) holds
    the row states D, r and -LSE*log2(e), each B*H*N floats, afterwards; when
    none is given, grouped-query heads get one of bwd_ex_workspace_bytes,
    which lets the column pass split each group over several workgroups.
    passes: 1 row pass, 2 column pass, 3 both."""
    lib = load()
    _check("q", q, q)
    Hkv = _kv_heads(q, k)
    kvs = _kv_shape(q, Hkv)
    for n, t in (("o", o), ("do", do)):
        _check(n, t, q)
    for n, t in (("k", k), ("v", v)):
        _check(n, t, q, shape=kvs)
    B, H, N, d = q.shape
    _check("lse", lse, q, torch.float32, (B, H, N))
    if outs is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    else:
        dq, dk, dv = outs
    _check("dq", dq, q)
    for n, t in (("dk", dk), ("dv", dv)):
        _check(n, t, q, shape=kvs)
    ext = Hkv != H or window != 0 or doc_start is not None or block_mask is not None
    if ext and passes != 3:
        raise ValueError("grouped-query or masked backward runs both passes (passes=3)")
    need = lib.attn_bwd_ex_workspace_bytes(B, H, Hkv, N)
    if workspace is None:
        workspace = torch.empty(need // 4, device=q.device, dtype=torch.float32)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            do.data_ptr())
    rest = (_scale(q, scale), 1 if gproj else 0, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            workspace.data_ptr(), ws_bytes, _stream(q.device))
    c = 1 if causal else 0
    if ext:
        st = lib.attn_bwd_ex(_dt(q), B, H, Hkv, N, d, *ptrs, c, int(window),
                             _docs(q, doc_start), _bmask(q, block_mask), *rest)
    else:
        st = lib.attn_bwd_passes(passes, _dt(q), B, H, N, d, *ptrs, c, *rest)
    _raise("attn_bwd", st)
    return dq, dk, dv


def attn_bob(q, k, v, o, lse, do, g_dq, g_dk, g_dv, causal: bool = True,
             scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None, outs=None,
             passes: int = 3, window: int = 0, doc_start: Optional[torch.Tensor] = None,
             block_mask: Optional[torch.Tensor] = None, gproj: bool = False
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """g_Q, g_K, g_V, g_dO: the VJP of (q, k, v, do) -> (dQ, dK, dV) with
    cotangents (g_dq, g_dk, g_dv).  `workspace` holds the row states D, alpha,
    beta, -LSE*log2(e) and -kappa = -(alpha*D + beta) afterwards; when none is
    given, grouped-query heads get one of bob_ex_workspace_bytes (split column
    pass).  `gproj` projects the residual row sums of g_Q's bf16 key weights
    and g_dO's value weights (attn_bob_ex)."""
    lib = load()
    _check("q", q, q)
    Hkv = _kv_heads(q, k)
    kvs = _kv_shape(q, Hkv)
    for n, t in (("o", o), ("do", do), ("g_dq", g_dq)):
        _check(n, t, q)
    for n, t in (("k", k), ("v", v), ("g_dk", g_dk), ("g_dv", g_dv)):
        _check(n, t, q, shape=kvs)
    B, H, N, d = q.shape
    _check("lse", lse, q, torch.float32, (B, H, N))
    if outs is None:
        gq, gk, gv, gdo = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(k),
                           torch.empty_like(q))
    else:
        gq, gk, gv, gdo = outs
    for n, t in (("g_q", gq), ("g_do", gdo)):
        _check(n, t, q)
    for n, t in (("g_k", gk), ("g_v", gv)):
        _check(n, t, q, shape=kvs)
    ext = (Hkv != H or window != 0 or doc_start is not None or block_mask is not None
           or bool(gproj))
    if ext and passes != 3:
        raise ValueError("grouped-query, masked or projected BoB runs both passes (passes=3)")
    need = lib.attn_bob_ex_workspace_bytes(B, H, Hkv, N)
    if workspace is None:
        workspace = torch.empty(need // 4, device=q.device, dtype=torch.float32)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            do.data_ptr(), g_dq.data_ptr(), g_dk.data_ptr(), g_dv.data_ptr())
    rest = (_scale(q, scale), gq.data_ptr(), gk.data_ptr(), gv.data_ptr(), gdo.data_ptr(),
            workspace.data_ptr(), ws_bytes, _stream(q.device))
    c = 1 if causal else 0
    if ext:
        st = lib.attn_bob_ex(_dt(q), B, H, Hkv, N, d, *ptrs, c, int(window),
                             _docs(q, doc_start), _bmask(q, block_mask), rest[0],
                             1 if gproj else 0, *rest[1:])
    else:
        st = lib.attn_bob_passes(passes, _dt(q), B, H, N, d, *ptrs, c, *rest)
    _raise("attn_bob", st)
    return gq, gk, gv, gdo


# Largest B * H * N attn_bob_noalloc accepts (its row states live in a
# library-owned device array of this many rows).
BOB_NOALLOC_MAX_ROWS = 3 << 20


def attn_bob_noalloc(q, k, v, o, lse, do, g_dq, g_dk, g_dv, causal: bool = True,
                     scale: Optional[float] = None, outs=None
                     ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """attn_bob without a workspace: the row states live in the library's
    own device array (multi-head only, B * H * N <= BOB_NOALLOC_MAX_ROWS).
    With `outs` given, the call allocates nothing.  Calls that overlap in
    time on one GPU share that array and race."""
    lib = load()
    _check("q", q, q)
    for n, t in (("k", k), ("v", v), ("o", o), ("do", do), ("g_dq", g_dq), ("g_dk", g_dk),
                 ("g_dv", g_dv)):
        _check(n, t, q)
    B, H, N, d = q.shape
    _check("lse", lse, q, torch.float32, (B, H, N))
    if outs is None:
        outs = tuple(torch.empty_like(q) for _ in range(4))
    for n, t in zip(("g_q", "g_k", "g_v", "g_do"), outs):
        _check(n, t, q)
    gq, gk, gv, gdo = outs
    st = lib.attn_bob_noalloc(_dt(q), B, H, N, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              o.data_ptr(), lse.data_ptr(), do.data_ptr(), g_dq.data_ptr(),
                              g_dk.data_ptr(), g_dv.data_ptr(), 1 if causal else 0,
                              _scale(q, scale), gq.data_ptr(), gk.data_ptr(), gv.data_ptr(),
                              gdo.data_ptr(), _stream(q.device))
    _raise("attn_bob_noalloc", st)
    return gq, gk, gv, gdo


def attn_hvp(q, k, v, do, v_q, v_k, v_v, causal: bool = True, scale: Optional[float] = None,
             gproj: bool = False, grad: bool = True, workspace: Optional[torch.Tensor] = None,
             window: int = 0, doc_start: Optional[torch.Tensor] = None,
             block_mask: Optional[torch.Tensor] = None):
    """Hessian-vector product of Phi(q, k, v) = <do, O(q, k, v)> (do fixed) with
    v = (v_q, v_k, v_v), in one library call (forward, optional backward, BoB).
    Returns a dict with O, LSE, Hv_q, Hv_k, Hv_v, Hv_do (the derivative of
    <v, grad Phi> with respect to do) and, when `grad`, dQ, dK, dV.  k, v, v_k
    and v_v may have fewer heads than q (grouped-query); window, doc_start and
    block_mask as in attn_fwd."""
    lib = load()
    _check("q", q, q)
    Hkv = _kv_heads(q, k)
    kvs = _kv_shape(q, Hkv)
    for n, t in (("do", do), ("v_q", v_q)):
        _check(n, t, q)
    for n, t in (("k", k), ("v", v), ("v_k", v_k), ("v_v", v_v)):
        _check(n, t, q, shape=kvs)
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    hq, hdo = torch.empty_like(q), torch.empty_like(q)
    hk, hv = torch.empty_like(k), torch.empty_like(k)
    dq = dk = dv = None
    if grad:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    need = lib.attn_hvp_ex_workspace_bytes(B, H, Hkv, N)
    if workspace is None:
        workspace = torch.empty(need // 4, device=q.device, dtype=torch.float32)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    ptr = (lambda t: None if t is None else t.data_ptr())
    st = lib.attn_hvp_ex(_dt(q), B, H, Hkv, N, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                      do.data_ptr(), v_q.data_ptr(), v_k.data_ptr(), v_v.data_ptr(),
                      1 if causal else 0, int(window), _docs(q, doc_start),
                      _bmask(q, block_mask), _scale(q, scale), 1 if gproj else 0,
                      o.data_ptr(), lse.data_ptr(), ptr(dq),
                      ptr(dk), ptr(dv), hq.data_ptr(), hk.data_ptr(), hv.data_ptr(),
                      hdo.data_ptr(), workspace.data_ptr(), ws_bytes, _stream(q.device))
    _raise("attn_hvp", st)
    out = {"O": o, "LSE": lse, "Hv_q": hq, "Hv_k": hk, "Hv_v": hv, "Hv_do": hdo}
    if grad:
        out.update(dQ=dq, dK=dk, dV=dv)
    return out


FP8_PARTS = ("q", "k", "vt", "eq", "ek", "ev", "vmax")


def fp8_workspace_bytes(B: int, H: int, Hkv: int, N: int) -> int:
    return int(load().attn_fp8_workspace_bytes(B, H, Hkv, N))


def fp8_parts(ws: torch.Tensor, B: int, H: int, Hkv: int, N: int) -> dict:
    """Views of the parts of an FP8 workspace (uint8 tensor): codes q (B, H, N,
    64), k (B, Hkv, N, 64), vt (B, Hkv, 64, NP) and int32 exponents eq (B, H,
    nb), ek (B, Hkv, nb), ev (B, Hkv, 64), nb = ceil(N / 64), NP = 64 nb."""
    lib = load()
    offs = (ctypes.c_size_t * len(FP8_PARTS))()
    _raise("attn_fp8_workspace_layout", lib.attn_fp8_workspace_layout(B, H, Hkv, N, offs))
    nb = (N + 63) // 64
    shapes = {"q": ((B, H, N, 64), torch.uint8), "k": ((B, Hkv, N, 64), torch.uint8),
              "vt": ((B, Hkv, 64, nb * 64), torch.uint8), "eq": ((B, H, nb), torch.int32),
              "ek": ((B, Hkv, nb), torch.int32), "ev": ((B, Hkv, 64), torch.int32)}
    out = {}
    for i, name in enumerate(FP8_PARTS[:-1]):
        shape, dt = shapes[name]
        n = math.prod(shape) * (4 if dt == torch.int32 else 1)
        out[name] = ws[offs[i]:offs[i] + n].view(dt).view(shape)
    return out


def attn_fp8_quantize(q, k, v, signs: Optional[int] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """E4M3 codes and power-of-two exponents of q, k (rotated by diag(s) H / 8
    when `signs`, a 64-bit sign mask, is given) and v, written into an FP8
    workspace (uint8 tensor, returned; see fp8_parts for its contents)."""
    lib = load()
    _check("q", q, q)
    Hkv = _kv_heads(q, k)
    for n, t in (("k", k), ("v", v)):
        _check(n, t, q, shape=_kv_shape(q, Hkv))
    B, H, N, d = q.shape
    need = fp8_workspace_bytes(B, H, Hkv, N)
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    if workspace.device != q.device or workspace.dtype != torch.uint8 or \
            workspace.numel() < need or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 GPU tensor of >= {need} bytes")
    rotate = signs is not None
    mask = (int(signs) & (2 ** 64 - 1)) if rotate else 0
    st = lib.attn_fp8_quantize(_dt(q), B, H, Hkv, N, d, q.data_ptr(), k.data_ptr(),
                               v.data_ptr(), 1 if rotate else 0, mask, workspace.data_ptr(),
                               workspace.numel(), _stream(q.device))
    _raise("attn_fp8_quantize", st)
    return workspace


def attn_fwd_fp8_codes(workspace: torch.Tensor, B: int, H: int, Hkv: int, N: int,
                       dtype=torch.bfloat16, causal: bool = True, scale: Optional[float] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       window: int = 0, doc_start: Optional[torch.Tensor] = None,
                       block_mask: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor]:
    """O (dtype), LSE (fp32) of the forward on the codes of an FP8 workspace;
    window, doc_start and block_mask as in attn_fwd."""
    lib = load()
    dev = workspace.device
    if dev.type != "cuda" or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    o = torch.empty((B, H, N, 64), device=dev, dtype=dtype) if out is None else out
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32) if lse is None else lse
    _check("out", o, o, dtype, (B, H, N, 64))
    _check("lse", lse, o, torch.float32, (B, H, N))
    c = 0.125 if scale is None else float(scale)
    st = lib.attn_fwd_fp8(_dt(o), B, H, Hkv, N, 64, workspace.data_ptr(), workspace.numel(),
                          1 if causal else 0, int(window), _docs(o, doc_start),
                          _bmask(o, block_mask), c, o.data_ptr(), lse.data_ptr(), _stream(dev))
    _raise("attn_fwd_fp8", st)
    return o, lse


def attn_fwd_fp8(q, k, v, causal: bool = True, scale: Optional[float] = None,
                 signs: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                 window: int = 0, doc_start: Optional[torch.Tensor] = None,
                 block_mask: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O, LSE of attention with both products in E4M3 (see attn_fp8_quantize
    for `signs`); shapes, dtypes and masks as attn_fwd."""
    ws = attn_fp8_quantize(q, k, v, signs, workspace)
    B, H, N, _ = q.shape
    return attn_fwd_fp8_codes(ws, B, H, k.shape[1], N, q.dtype, causal, _scale(q, scale),
                              window=window, doc_start=doc_start, block_mask=block_mask)
