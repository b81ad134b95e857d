"""The C ABI library: it loads, exports every function include/fbd.h declares,
and its host-side argument checks reject bad calls before any launch.
Runs without a GPU: no call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (the library binds to the HIP runtime torch loads)

import fwd_bwd_double_amd as fbd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fbd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fbd.load()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"attn_fwd", "attn_bwd", "attn_bob", "attn_bwd_workspace_bytes",
            "attn_bob_workspace_bytes", "attn_status_str", "attn_last_hip_error",
            "attn_fp8_quantize", "attn_fwd_fp8", "attn_fp8_workspace_bytes",
            "attn_fp8_workspace_layout"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_sizes(lib):
    assert fbd.bwd_workspace_bytes(2, 3, 5) == 3 * 2 * 3 * 5 * 4
    assert fbd.bob_workspace_bytes(2, 3, 5) == 5 * 2 * 3 * 5 * 4
    assert fbd.bwd_workspace_bytes(0, 3, 5) == 0


def test_split_column_pass_workspace_sizes(lib):
    # grouped-query heads: the column passes split a group into the fewest
    # slices (a divisor of H / Hkv) that give 1536 workgroups of 128 keys, or
    # into single heads when none does; the partial sums (two fp32 key-side
    # tensors per slice) follow the row states at a 256-byte boundary
    def split(base, B, Hkv, N, nsl):
        return (base + 255) // 256 * 256 + 2 * nsl * B * Hkv * N * 64 * 4
    for B, H, N in ((1, 12, 16384), (2, 4, 300)):   # multi-head: never split
        assert fbd.bwd_ex_workspace_bytes(B, H, H, N) == fbd.bwd_workspace_bytes(B, H, N)
        assert fbd.bob_ex_workspace_bytes(B, H, H, N) == fbd.bob_workspace_bytes(B, H, N)
    # 128 key blocks x 4 key heads = 512 workgroups: three slices of one head
    assert fbd.bwd_ex_workspace_bytes(1, 12, 4, 16384) == split(3 * 12 * 16384 * 4, 1, 4, 16384, 3)
    assert fbd.bob_ex_workspace_bytes(1, 12, 4, 16384) == split(5 * 12 * 16384 * 4, 1, 4, 16384, 3)
    # 2048 workgroups already: no split
    assert fbd.bwd_ex_workspace_bytes(4, 12, 4, 16384) == fbd.bwd_workspace_bytes(4, 12, 16384)
    # 400 key blocks x 2 key heads = 800: two slices of two heads reach 1600
    assert fbd.bwd_ex_workspace_bytes(1, 8, 2, 51200) == split(3 * 8 * 51200 * 4, 1, 2, 51200, 2)
    # 32 x 2 = 64: even single heads stay below 1536, so four slices
    assert fbd.bob_ex_workspace_bytes(1, 8, 2, 4096) == split(5 * 8 * 4096 * 4, 1, 2, 4096, 4)
    # a row-state size that is not a multiple of 256 bytes is rounded up
    assert fbd.bwd_ex_workspace_bytes(1, 3, 1, 5) == split(3 * 3 * 5 * 4, 1, 1, 5, 3)
    for bad in ((1, 12, 5, 64), (1, 12, 0, 64), (1, 4, 8, 64), (0, 4, 2, 64)):
        assert fbd.bwd_ex_workspace_bytes(*bad) == 0
        assert fbd.bob_ex_workspace_bytes(*bad) == 0


def test_status_strings(lib):
    for s in range(6):
        assert lib.attn_status_str(s)
    assert lib.attn_status_str(0) == b"ok"


FAKE = 1 << 20   # an aligned address that is never dereferenced: checks fail first


def fwd_call(lib, dt=0, B=1, H=1, N=8, d=64, ptrs=(FAKE, FAKE * 2, FAKE * 3), causal=1,
             scale=0.125, out=(FAKE * 4, FAKE * 5)):
    return lib.attn_fwd(dt, B, H, N, d, *ptrs, causal, scale, *out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=32), 2), (dict(d=128), 2), (dict(dt=7), 2), (dict(N=0), 1), (dict(B=-1), 1),
    (dict(H=0), 1), (dict(scale=0.0), 1), (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1), (dict(scale=-1.0), 1),
    (dict(ptrs=(0, FAKE * 2, FAKE * 3)), 1), (dict(out=(0, FAKE * 5)), 1),
    (dict(ptrs=(FAKE + 8, FAKE * 2, FAKE * 3)), 3),
    (dict(out=(FAKE * 2, FAKE * 5)), 1),           # output aliases an input
    (dict(N=1 << 30), 2),                          # N * 64 beyond 32-bit indexing
    (dict(N=1 << 25), 2),                          # head bytes beyond 32-bit buffer offsets
    (dict(dt=1, N=1 << 24), 2),
])
def test_fwd_rejects_bad_arguments_before_launch(lib, kw, status):
    assert fwd_call(lib, **kw) == status


def test_bwd_and_bob_reject_small_workspace(lib):
    p = [FAKE * (i + 1) for i in range(12)]
    need = fbd.bwd_workspace_bytes(1, 1, 8)
    st = lib.attn_bwd(0, 1, 1, 8, 64, *p[:5], p[5], 1, 0.125, 0, p[6], p[7], p[8], p[9],
                      need - 4, None)
    assert st == 4
    st = lib.attn_bwd(0, 1, 1, 8, 64, *p[:5], p[5], 1, 0.125, 0, p[6], p[7], p[8], None,
                      need, None)
    assert st == 4
    need = fbd.bob_workspace_bytes(1, 1, 8)
    st = lib.attn_bob(0, 1, 1, 8, 64, *p[:6], p[6], p[7], p[8], 1, 0.125, p[9], p[10], p[11],
                      FAKE * 20, FAKE * 30, need - 1, None)
    assert st == 4


def hvp_call(lib, grad=(FAKE * 11, FAKE * 12, FAKE * 13), ws_bytes=None, **kw):
    p = [FAKE * (i + 1) for i in range(9)]   # Q K V dO vQ vK vV O LSE
    out = [FAKE * (20 + i) for i in range(4)]
    need = fbd.hvp_workspace_bytes(1, 1, 8)
    return lib.attn_hvp(kw.get("dt", 0), 1, 1, 8, kw.get("d", 64), *p[:7], 1, 0.125, 0, p[7],
                        p[8], *grad, *out, FAKE * 40, need if ws_bytes is None else ws_bytes,
                        None)


def test_hvp_rejects_bad_arguments_before_launch(lib):
    # BoB's five row states and the backward's r: six fp32 values per row
    assert fbd.hvp_workspace_bytes(2, 3, 5) == 6 * 2 * 3 * 5 * 4
    assert fbd.bob_workspace_bytes(2, 3, 5) == 5 * 2 * 3 * 5 * 4
    assert hvp_call(lib, d=32) == 2
    assert hvp_call(lib, grad=(FAKE * 11, None, FAKE * 13)) == 1     # partial gradient set
    assert hvp_call(lib, ws_bytes=fbd.hvp_workspace_bytes(1, 1, 8) - 4) == 4
    assert hvp_call(lib, grad=(FAKE * 11, FAKE * 12, FAKE)) == 1     # dV aliases Q


def test_hvp_ex_rejects_bad_arguments_before_launch(lib):
    # Q K V dO vQ vK vV, then O LSE dQ dK dV HvQ HvK HvV HvdO, then ws
    p = [FAKE * (i + 1) for i in range(7)]
    out = [FAKE * (20 + i) for i in range(9)]
    def call(H=4, Hkv=2, causal=1, window=0, ds=None, bm=None, ws_bytes=None, d=64):
        need = fbd.load().attn_hvp_ex_workspace_bytes(1, H, max(Hkv, 1), 8)
        return lib.attn_hvp_ex(0, 1, H, Hkv, 8, d, *p, causal, window, ds, bm, 0.125, 0, *out,
                               FAKE * 40, need if ws_bytes is None else ws_bytes, None)
    # the split column passes' partial sums follow the row states, 256-byte
    # aligned, as in attn_bob_ex's workspace
    r256 = lambda x: (x + 255) // 256 * 256
    for B, H, Hkv, N in ((1, 4, 2, 8), (1, 8, 1, 4096), (3, 6, 2, 100)):
        parts = fbd.bob_ex_workspace_bytes(B, H, Hkv, N) - fbd.bob_workspace_bytes(B, H, N)
        want = fbd.hvp_workspace_bytes(B, H, N)
        if parts:
            parts = fbd.bob_ex_workspace_bytes(B, H, Hkv, N) - r256(fbd.bob_workspace_bytes(B, H, N))
            want = r256(want) + parts
        assert lib.attn_hvp_ex_workspace_bytes(B, H, Hkv, N) == want, (B, H, Hkv, N)
    assert lib.attn_hvp_ex_workspace_bytes(2, 3, 3, 5) == fbd.hvp_workspace_bytes(2, 3, 5)
    for H, Hkv in ((4, 3), (4, 0), (4, 8)):
        assert call(H=H, Hkv=Hkv) == 1
    assert call(d=32) == 2
    assert call(window=-1) == 1
    assert call(causal=0, window=4) == 2          # a window needs the causal mask
    assert call(causal=0, ds=FAKE * 50) == 2      # so do document masks
    assert call(ds=FAKE * 50 + 2) == 3            # doc_start must be 4-byte aligned
    assert call(ws_bytes=fbd.hvp_workspace_bytes(1, 4, 8) - 4) == 4


def test_extended_forms_reject_bad_heads_and_windows(lib):
    p = [FAKE * (i + 1) for i in range(3)]
    call = lambda H, Hkv, causal=1, window=0, ds=None, bm=None: lib.attn_fwd_ex(
        0, 1, H, Hkv, 8, 64, *p, causal, window, ds, bm, 0.125, FAKE * 4, FAKE * 5, None)
    for H, Hkv in ((4, 3), (4, 0), (4, 8), (4, -1)):
        assert call(H, Hkv) == 1
    assert call(4, 2, window=-1) == 1
    assert call(4, 2, causal=0, window=4) == 2     # a window needs the causal mask
    assert call(4, 2, causal=0, ds=FAKE * 7) == 2  # so do document masks
    assert call(4, 2, ds=FAKE * 7 + 2) == 3        # doc_start must be 4-byte aligned
    assert call(4, 2, ds=FAKE * 4) == 1            # and must not overlap an output
    assert call(4, 2, bm=FAKE * 5 + 1) == 1        # a block mask must not overlap an output


def test_fp8_workspace_layout(lib):
    B, H, Hkv, N = 2, 4, 2, 130
    offs = (ctypes.c_size_t * 7)()
    assert lib.attn_fp8_workspace_layout(B, H, Hkv, N, offs) == 0
    nb = 3
    sizes = [B * H * N * 64, B * Hkv * N * 64, B * Hkv * 64 * nb * 64, B * H * nb * 4,
             B * Hkv * nb * 4, B * Hkv * 64 * 4, B * Hkv * 64 * 4]
    for i in range(7):
        assert offs[i] % 256 == 0
        end = offs[i] + sizes[i]
        nxt = offs[i + 1] if i < 6 else fbd.fp8_workspace_bytes(B, H, Hkv, N)
        assert end <= nxt
    assert fbd.fp8_workspace_bytes(0, 1, 1, 8) == 0
    assert lib.attn_fp8_workspace_layout(1, 4, 3, 8, offs) == 1   # Hkv must divide H
    assert lib.attn_fp8_workspace_layout(1, 1, 1, 8, None) == 1


def test_fp8_rejects_bad_arguments_before_launch(lib):
    B, H, Hkv, N = 1, 2, 1, 64
    need = fbd.fp8_workspace_bytes(B, H, Hkv, N)
    q, k, v, ws, o, lse = (FAKE * (i + 1) for i in range(6))
    ws = FAKE * 64   # far from the inputs: no overlap
    assert lib.attn_fp8_quantize(0, B, H, Hkv, N, 64, q, k, v, 1, 5, ws, need - 1, None) == 4
    assert lib.attn_fp8_quantize(0, B, H, Hkv, N, 64, q, k, v, 1, 5, None, need, None) == 4
    assert lib.attn_fp8_quantize(0, B, H, 3, N, 64, q, k, v, 1, 5, ws, need, None) == 1
    assert lib.attn_fp8_quantize(0, B, H, Hkv, N, 32, q, k, v, 1, 5, ws, need, None) == 2
    assert lib.attn_fp8_quantize(0, B, H, Hkv, N, 64, 0, k, v, 1, 5, ws, need, None) == 1
    assert lib.attn_fp8_quantize(0, B, H, Hkv, N, 64, q + 8, k, v, 1, 5, ws, need, None) == 3
    # the workspace overlapping an input
    assert lib.attn_fp8_quantize(0, B, H, Hkv, N, 64, q, k, v, 1, 5, k, need, None) == 1
    f8 = lambda dt=0, nb=need, causal=1, win=0, ds=None, bm=None, sc=0.125, out=o: \
        lib.attn_fwd_fp8(dt, B, H, Hkv, N, 64, ws, nb, causal, win, ds, bm, sc, out, lse, None)
    assert f8(nb=need - 1) == 4
    assert f8(sc=0.0) == 1
    assert f8(out=ws) == 1                  # the output overlaps the workspace
    assert f8(dt=7) == 2
    assert f8(causal=0, win=4) == 2         # a window needs the causal mask
    assert f8(ds=FAKE * 7 + 2) == 3         # doc_start must be 4-byte aligned
    assert f8(bm=lse) == 1                  # a block mask must not overlap an output


@pytest.mark.parametrize("op", ["fwd", "bwd", "bob", "hvp"])
@pytest.mark.parametrize("view", ["slice", "permute"])
def test_binding_rejects_strided_q(op, view):
    # The kernels read q through its data pointer as a dense (B, H, N, d)
    # array.  A view with the right shape but other strides -- the first 64
    # channels of a packed (B, H, N, 192) tensor, or a (B, N, H, d) tensor
    # permuted to (B, H, N, d) -- must be rejected before anything is
    # allocated or launched.  CPU tensors suffice: the layout checks come
    # before the device check.
    B, H, N, d = 1, 2, 8, 64
    dense = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    if view == "slice":
        q = torch.zeros(B, H, N, 3 * d, dtype=torch.bfloat16)[..., :d]
    else:
        q = torch.zeros(B, N, H, d, dtype=torch.bfloat16).permute(0, 2, 1, 3)
    assert q.shape == dense.shape and not q.is_contiguous()
    lse = torch.zeros(B, H, N)
    t = dense
    with pytest.raises(ValueError, match="q must be contiguous"):
        if op == "fwd":
            fbd.attn_fwd(q, t, t)
        elif op == "bwd":
            fbd.attn_bwd(q, t, t, t, lse, t, outs=(t, t, t))
        elif op == "bob":
            fbd.attn_bob(q, t, t, t, lse, t, t, t, t, outs=(t, t, t, t))
        else:
            fbd.attn_hvp(q, t, t, t, t, t, t)


def test_bob_noalloc_rejects_bad_arguments_before_any_device_call(lib):
    # attn_bob_noalloc: the size limit of the library's row-state array, then
    # the caller's pointers, are checked before the device is queried
    p = [FAKE * (i + 1) for i in range(13)]

    def call(B=1, H=1, N=8, ptrs=None, dt=0):
        a = p if ptrs is None else ptrs
        return lib.attn_bob_noalloc(dt, B, H, N, 64, *a[:6], a[6], a[7], a[8], 1, 0.125,
                                    a[9], a[10], a[11], a[12], None)

    assert fbd.BOB_NOALLOC_MAX_ROWS == 3 << 20
    assert call(B=1, H=13, N=262144) == 4           # 13 * 262144 rows > 12 * 262144
    assert call(B=2, H=12, N=262144) == 4
    assert call(B=1, H=12, N=262145) == 4
    assert call(ptrs=[0] + p[1:]) == 1              # null input
    assert call(ptrs=p[:9] + [0] + p[10:]) == 1     # null output
    assert call(ptrs=[FAKE + 8] + p[1:]) == 3       # misaligned
    assert call(ptrs=p[:9] + [p[0]] + p[10:]) == 1  # output aliases an input
    assert call(dt=5) == 2
    assert call(N=0) == 1


def declared_parameter_counts():
    """Number of parameters of every function include/fbd.h declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(attn_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else len(params.split(","))
    return out


def test_binding_argument_counts_match_the_header(lib):
    # every function the binding gives a signature must take exactly the
    # header's number of parameters (a stale ctypes list would shift every
    # argument after the first difference)
    counts = declared_parameter_counts()
    checked = 0
    for name, n in counts.items():
        argtypes = getattr(getattr(lib, name), "argtypes", None)
        if argtypes is None:
            continue
        assert len(argtypes) == n, (name, len(argtypes), n)
        checked += 1
    assert checked >= 20, checked


def test_bob_ex_rejects_bad_arguments_before_launch(lib):
    # Q K V O LSE dO gdQ gdK gdV, then gQ gK gV gdO, then ws
    p = [FAKE * (i + 1) for i in range(9)]
    out = [FAKE * (20 + i) for i in range(4)]
    def call(H=4, Hkv=2, causal=1, window=0, gproj=1, d=64, ws_bytes=None):
        need = lib.attn_bob_ex_workspace_bytes(1, H, max(Hkv, 1), 8)
        return lib.attn_bob_ex(0, 1, H, Hkv, 8, d, *p, causal, window, None, None, 0.125, gproj,
                               *out, FAKE * 40, need if ws_bytes is None else ws_bytes, None)
    assert call(d=32) == 2
    assert call(H=4, Hkv=3) == 1
    assert call(causal=0, window=4) == 2
    assert call(ws_bytes=fbd.bob_workspace_bytes(1, 4, 8) - 4) == 4
