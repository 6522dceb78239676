"""The C-ABI library without a GPU: it loads, exports what include/abla.h declares,
and rejects bad arguments on the host before anything is enqueued."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_sparse_attention_21_amd", "libabla.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libabla.so not built")

FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first
FAKE2 = ctypes.c_void_p(0x90000000)


@pytest.fixture(scope="module")
def A():
    import block_sparse_attention_21_amd as A
    return A


def declared_functions():
    with open(os.path.join(ROOT, "include", "abla.h")) as f:
        src = f.read()
    decl = r"^\s*(?:abla_status|size_t|const char\s*\*|int32_t)\s+(abla_[a-z_]+)\s*\("
    return sorted(set(re.findall(decl, src, flags=re.MULTILINE)))


def test_exports_every_declared_symbol(A):
    names = declared_functions()
    assert len(names) == 11
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(A.EXPORTED)
    assert A.version() == 200
    assert A.status_str(0) == "ok" and A.status_str(99) == "unknown status"


def G(A, **kw):
    base = dict(B=1, H=2, T=3, Hs=16, Ws=24, d=128, P=8)
    base.update(kw)
    return A.Geometry(**base).c()


def reorder(A, g, dtype=1, inverse=0, layout=0, x=FAKE, y=FAKE2, pooled=None):
    return A._lib.abla_reorder(ctypes.byref(g), dtype, inverse, layout, x, y, pooled, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 1), (dict(H=-1), 1), (dict(T=0), 1), (dict(Hs=12), 1), (dict(Ws=20), 1), (dict(d=0), 1),
    (dict(P=4, Hs=16, Ws=24), 2), (dict(d=96), 2), (dict(d=256), 2), (dict(B=1 << 40), 2),
    (dict(T=1 << 16, Hs=1 << 8, Ws=1 << 8), 2),  # 2^32 tokens per head
])
def test_reorder_geometry_errors(A, kw, code):
    assert reorder(A, G(A, **kw)) == code


def test_reorder_argument_errors(A):
    g = G(A)
    assert reorder(A, g, dtype=7) == 1
    assert reorder(A, g, x=None) == 1
    assert reorder(A, g, y=None) == 1  # no output and nothing to pool
    P = ctypes.c_void_p(0x7000000)
    assert reorder(A, g, y=None, pooled=P, layout=1) == 1  # pooling only takes the token layout
    assert reorder(A, g, y=None, pooled=P, inverse=1) == 1
    assert reorder(A, g, y=None, pooled=ctypes.c_void_p(0x10000 + 64)) == 1  # pooled overlaps x
    assert reorder(A, g, y=FAKE) == 1  # x == y
    assert reorder(A, g, y=ctypes.c_void_p(0x10000 + 64)) == 1  # overlapping
    assert reorder(A, g, layout=5) == 1
    assert reorder(A, g, inverse=1, layout=1) == 1
    assert reorder(A, g, inverse=1, pooled=ctypes.c_void_p(0x7000000)) == 1
    assert reorder(A, g, inverse=2) == 1
    assert A._lib.abla_reorder(None, 1, 0, 0, FAKE, FAKE2, None, None) == 1


def qkv_call(A, g, dtype=1, q=ctypes.c_void_p(1 << 32), k=ctypes.c_void_p(2 << 32), v=ctypes.c_void_p(3 << 32),
             qbar=ctypes.c_void_p(4 << 32), kbar=ctypes.c_void_p(5 << 32), v_rt=ctypes.c_void_p(6 << 32)):
    return A._lib.abla_pool_qk_reorder_v(ctypes.byref(g), dtype, q, k, v, qbar, kbar, v_rt, None)


def test_pool_qk_reorder_v_errors(A):
    g = G(A)
    for n in ("q", "k", "v", "qbar", "kbar", "v_rt"):
        assert qkv_call(A, g, **{n: None}) == 1, n
    assert qkv_call(A, g, dtype=7) == 1
    assert qkv_call(A, g, v_rt=ctypes.c_void_p(1 << 32)) == 1  # v_rt aliases q
    assert qkv_call(A, g, qbar=ctypes.c_void_p((3 << 32) + 64)) == 1  # qbar inside v
    assert qkv_call(A, g, kbar=ctypes.c_void_p((4 << 32) + 8)) == 1  # kbar overlaps qbar
    assert qkv_call(A, g, v_rt=ctypes.c_void_p((5 << 32) + 8)) == 1  # v_rt overlaps kbar
    assert qkv_call(A, G(A, d=96)) == 2
    assert qkv_call(A, G(A, B=0)) == 1
    assert A._lib.abla_pool_qk_reorder_v(None, 1, FAKE, FAKE, FAKE, FAKE2, FAKE2, FAKE2, None) == 1
    # The pooling-only form (v = v_rt = NULL) checks the rest the same way.
    for n in ("q", "k", "qbar", "kbar"):
        assert qkv_call(A, g, v=None, v_rt=None, **{n: None}) == 1, n
    assert qkv_call(A, g, v=None, v_rt=None, kbar=ctypes.c_void_p((1 << 32) + 64)) == 1  # kbar inside q
    assert qkv_call(A, g, v=None, v_rt=None, dtype=7) == 1
    assert qkv_call(A, G(A, d=96), v=None, v_rt=None) == 2


def mask_call(A, g, p, ws=FAKE, ws_bytes=1 << 40, q=FAKE, k=FAKE, words=FAKE2, counts=FAKE2):
    return A._lib.abla_build_mask(ctypes.byref(g), ctypes.byref(p), q, k, words, counts, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=5), 1), (dict(cut=3), 1), (dict(thr=math.nan), 1), (dict(tau=math.nan), 1), (dict(pool_scale=-1.0), 1),
    (dict(pool_scale=math.nan), 1), (dict(pool_scale=math.inf), 1),
    (dict(sta=(2, 3, 3)), 1), (dict(sta=(3, 0, 3)), 1), (dict(sta=(-1, 3, 3)), 1), (dict(sta=(3, 3, 4)), 1),
    (dict(mode="static", gamma=-0.1), 1), (dict(mode="static", gamma=1.5), 1), (dict(mode="static", gamma=math.nan), 1),
    (dict(mode="static", lam=math.nan), 1), (dict(mode="static", lam=2.0), 1), (dict(mode="static", lam=-1e-9), 1),
])
def test_mask_param_errors(A, kw, code):
    p = A.MaskParams(**kw).c()
    assert mask_call(A, G(A), p) == code


def test_mask_pointer_workspace_and_size_errors(A):
    g, p = G(A), A.MaskParams().c()
    assert mask_call(A, g, p, q=None) == 1
    assert mask_call(A, g, p, counts=None) == 1
    assert mask_call(A, g, p, ws=None) == 3
    need = A.build_mask_workspace_bytes(A.Geometry(1, 2, 3, 16, 24, 128))
    assert need == 2 * 18 * 18 * 8
    assert mask_call(A, g, p, ws_bytes=need - 1) == 3
    big = G(A, T=4097, Hs=8, Ws=8)  # nb = 4097 > one LDS-resident row
    assert mask_call(A, big, p) == 2
    assert A._lib.abla_build_mask_workspace_bytes(ctypes.byref(G(A, d=96))) == 0
    # The static mode reads no pooled vectors and no workspace: with those NULL it gets as far
    # as the size check.
    st = A.MaskParams(mode="static").c()
    assert mask_call(A, big, st, q=None, k=None, ws=None, ws_bytes=0) == 2
    assert mask_call(A, g, st, q=None, counts=None, ws=None) == 1


def test_mask_output_overlaps(A):
    g, p = G(A), A.MaskParams().c()
    # distinct fake buffers 4 GiB apart; every call fails validation before any launch
    q, k, words, counts, lists, ws = (ctypes.c_void_p(i << 32) for i in range(1, 7))
    def call(**over):
        a = dict(q=q, k=k, words=words, counts=counts, lists=lists, ws=ws)
        a.update(over)
        return A._lib.abla_build_mask(ctypes.byref(g), ctypes.byref(p), a["q"], a["k"], a["words"], a["counts"],
                                      a["lists"], a["ws"], 1 << 40, None)
    assert call(counts=words) == 1
    assert call(lists=ctypes.c_void_p((2 << 32) + 8)) == 1  # lists overlaps kbar
    assert call(ws=ctypes.c_void_p((5 << 32) - 64)) == 1  # workspace runs into lists
    assert call(words=ctypes.c_void_p((1 << 32) + 128)) == 1  # mask words inside qbar


def attn_call(A, g, dtype=1, scale=0.0, q=FAKE, k=ctypes.c_void_p(0x20000), v=ctypes.c_void_p(0x30000),
              counts=FAKE, lists=FAKE, out=FAKE2, ws=FAKE, ws_bytes=1 << 40, flags=1):
    return A._lib.abla_sparse_attn_fwd(ctypes.byref(g), dtype, scale, q, k, v, counts, lists, out, flags, None, ws,
                                       ws_bytes, None)


def test_attention_errors(A):
    g = G(A)
    assert attn_call(A, g, dtype=3) == 1
    assert attn_call(A, g, q=None) == 1
    assert attn_call(A, g, lists=None) == 1
    assert attn_call(A, g, out=None) == 1
    assert attn_call(A, g, out=FAKE) == 1  # aliases q
    assert attn_call(A, g, scale=math.nan) == 1
    assert attn_call(A, g, scale=-0.5) == 1
    assert attn_call(A, g, ws=None) == 3
    assert attn_call(A, g, flags=8) == 1  # unknown layout flag
    assert attn_call(A, g, flags=-1) == 1
    assert attn_call(A, g, flags=7, ws=None) == 3  # the known flags pass the argument checks
    assert attn_call(A, g, ws_bytes=2 * 18 * 4 - 1) == 3
    assert attn_call(A, G(A, d=32)) == 2
    # lse and the workspace overlap neither each other nor an input or out
    far = dict(q=ctypes.c_void_p(1 << 32), k=ctypes.c_void_p(2 << 32), v=ctypes.c_void_p(3 << 32),
               counts=ctypes.c_void_p(4 << 32), lists=ctypes.c_void_p(5 << 32), out=ctypes.c_void_p(6 << 32),
               ws=ctypes.c_void_p(7 << 32))
    def fwd(lse, **over):
        a = dict(far)
        a.update(over)
        return A._lib.abla_sparse_attn_fwd(ctypes.byref(g), 1, 0.0, a["q"], a["k"], a["v"], a["counts"], a["lists"],
                                           a["out"], 1, lse, a["ws"], 1 << 40, None)
    assert fwd(ctypes.c_void_p((6 << 32) + 16)) == 1  # lse inside out
    assert fwd(ctypes.c_void_p(8 << 32), ws=ctypes.c_void_p((4 << 32) + 4)) == 1  # workspace on counts
    assert fwd(ctypes.c_void_p(8 << 32), ws=ctypes.c_void_p((8 << 32) + 4)) == 1  # workspace on lse
    assert A.sparse_attn_workspace_bytes(A.Geometry(1, 2, 3, 16, 24, 128)) == 2 * 18 * 4 + 256


def bwd_call(A, g, dtype=1, scale=0.0, ws_bytes=1 << 40, **over):
    # Fake device addresses 4 GiB apart (no two overlap); every call below fails validation first.
    names = ("q", "k", "v", "o", "dout", "lse", "words", "counts", "lists", "dq", "dk", "dv", "ws")
    p = {n: ctypes.c_void_p((i + 1) << 32) for i, n in enumerate(names)}
    p.update(over)
    return A._lib.abla_sparse_attn_bwd(ctypes.byref(g), dtype, scale, *[p[n] for n in names[:-1]], p["ws"],
                                       ws_bytes, None)


def test_backward_errors(A):
    g = G(A)
    for n in ("q", "k", "v", "o", "dout", "lse", "words", "counts", "lists", "dq", "dk", "dv"):
        assert bwd_call(A, g, **{n: None}) == 1, n
    assert bwd_call(A, g, dtype=3) == 1
    assert bwd_call(A, g, dtype=0, ws=None) == 3  # float32 passes the argument checks
    assert bwd_call(A, g, scale=math.nan) == 1
    assert bwd_call(A, g, scale=-1.0) == 1
    assert bwd_call(A, g, dk=ctypes.c_void_p(1 << 32)) == 1  # dk aliases q
    assert bwd_call(A, g, dv=ctypes.c_void_p(10 << 32)) == 1  # dv aliases dq
    assert bwd_call(A, g, ws=None) == 3
    assert bwd_call(A, g, ws=ctypes.c_void_p((7 << 32) + 64)) == 1  # workspace inside the mask words
    assert bwd_call(A, g, dq=ctypes.c_void_p(6 << 32)) == 1  # dq aliases lse
    assert bwd_call(A, g, dk=ctypes.c_void_p((9 << 32) - 64)) == 1  # dk runs into the lists
    need = A.sparse_attn_bwd_workspace_bytes(A.Geometry(1, 2, 3, 16, 24, 128))
    def al(n):
        return (n + 255) // 256 * 256

    # B*H = 2, N = 1152, nb = 18: D and L2 rows, column counts and visiting order, column lists
    assert need == 2 * al(2 * 1152 * 4) + 2 * al(2 * 18 * 4) + al(2 * 18 * 18 * 4)
    assert bwd_call(A, g, ws_bytes=need - 1) == 3
    assert bwd_call(A, G(A, d=32)) == 2


def test_binding_rejects_cpu_tensors(A):
    import torch
    geom = A.Geometry(1, 1, 1, 8, 8, 64)
    with pytest.raises(ValueError):
        A.reorder(torch.zeros(1, 1, 64, 64), geom)


# ---------------------------------------------------------------- 16-byte alignment
def _p(i, shift=0):
    return ctypes.c_void_p((i << 34) + shift)  # far apart: no two buffers overlap


def _entry_calls(A):
    """For every computing entry point: (number of pointer arguments, call(pointers)) such that
    distinct, aligned, non-overlapping fake buffers pass validation."""
    g = G(A)
    geom = A.Geometry(1, 2, 3, 16, 24, 128)
    p = A.MaskParams(mode="cdf", thr=0.5).c()
    L = A._lib
    ws_mask = A.build_mask_workspace_bytes(geom)
    ws_attn = A.sparse_attn_workspace_bytes(geom)
    ws_bwd = A.sparse_attn_bwd_workspace_bytes(geom)
    return {
        "abla_reorder": (3, lambda P: L.abla_reorder(ctypes.byref(g), 1, 0, 0, *P, None)),
        "abla_pool_qk_reorder_v": (6, lambda P: L.abla_pool_qk_reorder_v(ctypes.byref(g), 1, *P, None)),
        "abla_build_mask": (6, lambda P: L.abla_build_mask(ctypes.byref(g), ctypes.byref(p), *P, ws_mask, None)),
        "abla_sparse_attn_fwd": (8, lambda P: L.abla_sparse_attn_fwd(ctypes.byref(g), 1, 0.0, *P[:6], 3, *P[6:],
                                                                      ws_attn, None)),
        "abla_sparse_attn_fwd_noalloc": (7, lambda P: L.abla_sparse_attn_fwd_noalloc(ctypes.byref(g), 1, 0.0,
                                                                                      *P[:6], 3, P[6], None)),
        "abla_sparse_attn_bwd": (13, lambda P: L.abla_sparse_attn_bwd(ctypes.byref(g), 1, 0.0, *P, ws_bwd, None)),
    }


def test_misaligned_pointers_rejected(A):
    """Each device pointer of each computing entry point must be 16-byte aligned: shifting any one
    of them by 8 bytes (or 4) turns a call that passes validation into ABLA_ERR_INVALID. Host
    only: the unshifted calls fail at the launch (ABLA_ERR_HIP) because no device is visible,
    which shows that they passed every argument check."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check: the unshifted calls would launch on a visible device")
    for name, (n, call) in _entry_calls(A).items():
        assert call([_p(i + 1) for i in range(n)]) == 4, name
        for slot in range(n):
            for shift in (8, 4):
                assert call([_p(i + 1, shift if i == slot else 0) for i in range(n)]) == 1, (name, slot, shift)


def test_noalloc_forward_limits(A):
    """The allocation-free forward has the forward's argument checks and refuses, before touching
    any device, a geometry whose visiting order exceeds its 1 MiB built-in scratch."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check: a call that passed validation would launch on a visible device")
    L = A._lib

    def call(g, P=None, flags=3):
        P = P or [_p(i + 1) for i in range(7)]
        return L.abla_sparse_attn_fwd_noalloc(ctypes.byref(g), 1, 0.0, *P[:6], flags, P[6], None)

    big = G(A, H=256, T=21, Hs=48, Ws=80)  # 256 * 1260 query blocks: 1.29 MB of visiting order
    assert A.sparse_attn_workspace_bytes(A.Geometry(1, 256, 21, 48, 80, 128)) > (1 << 20)
    assert call(big) == 3
    fits = G(A, H=200, T=21, Hs=48, Ws=80)  # 252000 blocks: fits, fails only at the launch here
    assert call(fits) == 4
    g = G(A)
    assert call(g, flags=8) == 1
    assert call(g, P=[_p(1), None] + [_p(i + 1) for i in range(2, 7)]) == 1
    assert call(g, P=[_p(i + 1) for i in range(5)] + [_p(1), _p(7)]) == 1  # out is q
    assert L.abla_sparse_attn_fwd_noalloc(ctypes.byref(G(A, d=96)), 1, 0.0, *[_p(i + 1) for i in range(6)], 3,
                                          _p(7), None) == 2


def test_probe_library_exports():
    """The benchmark's matrix-core probe library exports what include/abla_probe.h declares and
    rejects bad arguments before launching."""
    path = os.path.join(ROOT, "block_sparse_attention_21_amd", "libabla_probe.so")
    with open(os.path.join(ROOT, "include", "abla_probe.h")) as f:
        names = sorted(set(re.findall(r"^\s*(?:int32_t|double)\s+(abla_[a-z_0-9]+)\s*\(", f.read(), re.MULTILINE)))
    assert names == ["abla_probe_mfma", "abla_probe_mfma_flops", "abla_probe_stream"]
    lib = ctypes.CDLL(path)
    for n in names:
        assert hasattr(lib, n), n
    lib.abla_probe_mfma.restype = ctypes.c_int32
    lib.abla_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.abla_probe_mfma_flops.restype = ctypes.c_double
    lib.abla_probe_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    assert lib.abla_probe_mfma(2, 1, 1, FAKE, None) == 1
    assert lib.abla_probe_mfma(0, 0, 1, FAKE, None) == 1
    assert lib.abla_probe_mfma(0, 1, 1, None, None) == 1
    assert lib.abla_probe_mfma_flops(0, 1, 1) == 2.0 * 32 * 32 * 16 * 16
    assert lib.abla_probe_mfma_flops(1, 2, 3) == 2.0 * 32 * 32 * 2 * 16 * 6
    lib.abla_probe_stream.restype = ctypes.c_int32
    lib.abla_probe_stream.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]
    assert lib.abla_probe_stream(0, None, FAKE2, 1 << 20, None) == 1
    assert lib.abla_probe_stream(1, FAKE, FAKE2, (1 << 20) + 16, None) == 1
    assert lib.abla_probe_stream(1, FAKE, FAKE2, 1 << 14, None) == 1
    assert lib.abla_probe_stream(2, FAKE, FAKE2, 1 << 20, None) == 1
    assert lib.abla_probe_stream(0, ctypes.c_void_p(0x10008), FAKE2, 1 << 20, None) == 1
