"""The allocation-free attention forward (abla_sparse_attn_fwd_noalloc) through the C-ABI,
against the workspace entry point (abla_sparse_attn_fwd) on the same mask: bit-identical
output and LSE, on calls in a row whose geometries shrink, in both dtypes and with V in both
layouts; the first case is also compared with the oracle."""
import math

import numpy as np
import pytest
import torch

from gen import make_random_qkv
from oracle import nabla_ref as R
from tests import parity as PT

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def A():
    import block_sparse_attention_21_amd as A
    assert torch.cuda.is_available(), "the gpu tests need a HIP device"
    return A


def _one_call(A, geo, d, dtype, fuse_v, seed):
    B, H, T, Hs, Ws = geo
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    q, k, v = make_random_qkv(B, H, T, Hs, Ws, d, dtype, seed=seed, device=DEV)
    k = (k.float() + 2.0 * q.float()).to(q.dtype)
    run = A.NablaAttention(geom, A.MaskParams(mode="cdf", thr=0.7), dtype=q.dtype, want_lse=True, fuse_v=fuse_v)
    run(q, k, v)  # mask, and the workspace entry point's output and LSE
    v_in = v if fuse_v else run.v_rt
    out = torch.full_like(run.out, math.nan)
    lse = torch.full_like(run.lse, math.nan)
    A.sparse_attn_fwd_noalloc(q, k, v_in, run.counts, run.lists, geom, out, qk_original_order=True,
                              v_original_order=fuse_v, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, run.out), (geo, d, dtype, fuse_v)
    assert torch.equal(lse, run.lse), (geo, d, dtype, fuse_v)
    return geom, og, q, k, v, run, out


def test_noalloc_matches_workspace_entry_point(A):
    """Calls in a row on one device: each one smaller than the previous (the shared scratch keeps
    the last call's contents and must not leak into the next)."""
    cases = [((1, 3, 6, 32, 48), 128, "bf16", False), ((1, 2, 3, 24, 88), 128, "bf16", False),
             ((1, 1, 3, 16, 24), 64, "bf16", True), ((1, 2, 4, 16, 16), 64, "f32", False),
             ((1, 1, 2, 16, 16), 128, "f32", False)]
    for n, (geo, d, dtype, fuse_v) in enumerate(cases):
        geom, og, q, k, v, run, out = _one_call(A, geo, d, dtype, fuse_v, seed=20 + n)
        if n == 0:
            op = R.MaskParams(mode="cdf", thr=0.7)
            ref = R.nabla_attention(q, k, v, og, op, block_mask=PT.gpu_mask(run.words, og))
            PT.compare_attention(out.float().cpu().numpy(), ref.O, dtype)


def test_noalloc_repeat_after_larger_call(A):
    """A large call (480p-like geometry, 12 heads) and then a one-block call: both equal the
    workspace entry point."""
    _one_call(A, (1, 12, 21, 32, 56), 128, "bf16", False, seed=31)
    _one_call(A, (1, 1, 1, 8, 8), 128, "bf16", False, seed=32)
