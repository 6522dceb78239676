"""Backward (dQ, dK, dV) of the block-sparse attention: HIP path vs the CPU oracle, through the C-ABI.

Two kinds of check, both under the gradient rule of tests/parity.py:
- kernel parity: the backward entry point is handed the oracle's forward output O (rounded
  to bf16, as the forward stores it) and log-sum-exp, and the oracle's backward takes D from
  that same O, so both sides see identical inputs; the mask is the GPU's own (checked
  against the oracle by the forward tests) or a random one built here;
- end to end: the GPU forward's O and lse feed the GPU backward, compared with the oracle's
  exact gradients.
Small geometries are compared in full; the 480p workload runs at full size, both ways, with
dQ checked on sampled query blocks and dK / dV on sampled key blocks (the oracle then
processes every query block that keeps the key block).

Inputs use Q.K scores of order one: when one key dominates every row, P is nearly one-hot,
dP - D cancels to a few ulps of dP and the gradients carry no accurate digits in any
precision that stores O in bf16, which tests nothing about the kernels.
"""
import math

import numpy as np
import pytest
import torch

from gen import WORKLOADS, make_dout, make_qkv, make_random_qkv
from oracle import nabla_ref as R
from tests import parity as PT

pytestmark = pytest.mark.gpu

DEV = "cuda"
NAMES = ("dq", "dk", "dv")


@pytest.fixture(scope="module")
def A():
    import block_sparse_attention_21_amd as A
    assert torch.cuda.is_available(), "the gpu tests need a HIP device"
    return A


def _head(x, b, h, og):
    """Fractal-order float64 copy of one (b, h) slice of an original-order [B,H,N,d] tensor."""
    gh = R.Geom(1, 1, og.T, og.Hs, og.Ws, og.d, og.P)
    return R.reorder(R.to64(x[b, h]), gh), gh


def _oracle_forward(q, k, v, gm, og, dtype=torch.bfloat16):
    """Oracle O (original order, rounded to `dtype`) and lse (fractal order, float32) on mask gm."""
    scale = 1.0 / math.sqrt(og.d)
    O = np.empty((og.B, og.H, og.N, og.d))
    lse = np.empty((og.B, og.H, og.N))
    for b in range(og.B):
        for h in range(og.H):
            Qr, gh = _head(q, b, h, og)
            Kr, _ = _head(k, b, h, og)
            Vr, _ = _head(v, b, h, og)
            Or, lse[b, h] = R.masked_attention_head(Qr, Kr, Vr, gm[b, h], gh, scale)
            O[b, h] = R.inverse_reorder(Or, gh)
    o = torch.from_numpy(O).to(dtype).to(DEV)
    return o, torch.from_numpy(lse.astype(np.float32)).to(DEV)


def _check_full(og, q, k, v, dout, gm, dq, dk, dv, tag, o_given=None, dtype="bf16"):
    """Every element of the three gradients against the oracle, head by head. With o_given
    the oracle takes D from that (bf16) forward output."""
    scale = 1.0 / math.sqrt(og.d)
    got = {n: [] for n in NAMES}
    ref = {n: [] for n in NAMES}
    for b in range(og.B):
        for h in range(og.H):
            Qr, gh = _head(q, b, h, og)
            Kr, _ = _head(k, b, h, og)
            Vr, _ = _head(v, b, h, og)
            dOr, _ = _head(dout, b, h, og)
            Og = None if o_given is None else _head(o_given, b, h, og)[0]
            rs = R.masked_attention_backward_head(Qr, Kr, Vr, dOr, gm[b, h], gh, scale, O=Og)
            for n, t, r in zip(NAMES, (dq, dk, dv), rs):
                got[n].append(_head(t, b, h, og)[0])
                ref[n].append(r)
    errs = {n: PT.grad_errors(np.stack(got[n]), np.stack(ref[n])) for n in NAMES}
    print(f"{tag}: " + ", ".join(f"{n} rel {r:.2e} max {m:.2e}" for n, (r, m) in errs.items()), flush=True)
    for n in NAMES:
        PT.compare_grad(np.stack(got[n]), np.stack(ref[n]), f"{tag} {n}", dtype)
    return errs


def _inputs(B, H, T, Hs, Ws, d, seed, mix=0.25):
    q, k, v = make_random_qkv(B, H, T, Hs, Ws, d, "bf16", seed=seed, device=DEV)
    # A little of Q in K gives the pooled scores some structure for the mask.
    k = (k.float() + mix * q.float()).to(q.dtype)
    dout = make_dout(B, H, T * Hs * Ws, d, seed=seed + 1, device=DEV)
    return q, k, v, dout


SMALL = [
    # (name, d, (B,H,T,Hs,Ws), MaskParams kwargs)
    ("ragged", 128, (1, 2, 3, 24, 88), dict(mode="cdf", thr=0.7)),  # nb = 99
    ("d64", 64, (2, 1, 4, 16, 40), dict(mode="cdf", thr=0.9)),
    ("dyn", 128, (1, 2, 3, 32, 32), dict(mode="dyn", tau=2.0)),
    ("no-sta", 128, (1, 1, 5, 16, 24), dict(mode="cdf", thr=0.6, sta=(0, 0, 0))),
    ("full", 128, (1, 1, 2, 16, 32), dict(mode="cdf", thr=1.0)),
    ("one-block", 128, (1, 2, 1, 8, 8), dict(mode="cdf", thr=0.5)),
    ("d64-nb300", 64, (1, 1, 3, 80, 80), dict(mode="cdf", thr=0.95)),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_kernel_parity(A, case):
    """The backward entry point on the oracle's O and lse, every element."""
    name, d, (B, H, T, Hs, Ws), pkw = case
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    q, k, v, dout = _inputs(B, H, T, Hs, Ws, d, seed=11)
    run = A.NablaAttention(geom, A.MaskParams(**pkw), dtype=torch.bfloat16, want_lse=True)
    run(q, k, v)
    torch.cuda.synchronize()
    gm = PT.gpu_mask(run.words, og)
    o, lse = _oracle_forward(q, k, v, gm, og)
    print(f"backward {name}: B{B} H{H} nb{geom.nb} d{d} kept {int(gm.sum())}", flush=True)
    dq, dk, dv = A.sparse_attn_bwd(q, k, v, o, dout, lse, run.words, run.counts, run.lists, geom)
    torch.cuda.synchronize()
    _check_full(og, q, k, v, dout, gm, dq, dk, dv, name, o_given=o)


@pytest.mark.parametrize("case", [SMALL[0], SMALL[1]], ids=[SMALL[0][0], SMALL[1][0]])
def test_backward_end_to_end(A, case):
    """GPU forward then GPU backward (NablaAttention.backward) against the exact oracle."""
    name, d, (B, H, T, Hs, Ws), pkw = case
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    q, k, v, dout = _inputs(B, H, T, Hs, Ws, d, seed=12)
    run = A.NablaAttention(geom, A.MaskParams(**pkw), dtype=torch.bfloat16, want_lse=True)
    run(q, k, v)
    dq, dk, dv = run.backward(q, k, v, dout)
    torch.cuda.synchronize()
    _check_full(og, q, k, v, dout, PT.gpu_mask(run.words, og), dq, dk, dv, f"e2e {name}")


def _random_mask_inputs(og, rng, p_keep=0.3):
    """A random block mask with an empty row, an empty column and a full row, as words / counts / lists."""
    M = rng.random((og.B, og.H, og.nb, og.nb)) < p_keep
    M[..., 0, :] = False   # query block 0 keeps nothing
    M[..., 2, :] = True    # query block 2 keeps everything but key block 1
    M[..., :, 1] = False   # no query block keeps key block 1
    words = torch.from_numpy(np.ascontiguousarray(R.pack_bits(M)).view(np.int32)).to(DEV)
    counts = torch.from_numpy(M.sum(-1).astype(np.int32)).to(DEV)
    lists = np.zeros((og.B, og.H, og.nb, og.nb), dtype=np.int32)
    for idx in np.ndindex(M.shape[:-1]):
        nz = np.nonzero(M[idx])[0]
        lists[idx][: len(nz)] = nz
    return M, words, counts, torch.from_numpy(lists).to(DEV)


@pytest.mark.parametrize("d", [128, 64])
def test_backward_random_mask(A, d):
    """Masks not made by the mask builder: an empty row, an empty column, a full row."""
    B, H, T, Hs, Ws = 1, 2, 2, 24, 40
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    M, words, counts, lists = _random_mask_inputs(og, np.random.default_rng(d))
    q, k, v, dout = _inputs(B, H, T, Hs, Ws, d, seed=21, mix=0.0)
    o, lse = _oracle_forward(q, k, v, M, og)
    print(f"backward random mask d{d}: nb{geom.nb} kept {int(M.sum())}", flush=True)
    dq, dk, dv = A.sparse_attn_bwd(q, k, v, o, dout, lse, words, counts, lists, geom)
    torch.cuda.synchronize()
    _check_full(og, q, k, v, dout, M, dq, dk, dv, f"random-d{d}", o_given=o)
    # Rows of the empty query block get dQ = 0 exactly; keys of the empty column get dK = dV = 0.
    inv = torch.from_numpy(np.argsort(R.fractal_positions(og))).to(DEV)
    assert torch.count_nonzero(dq[:, :, inv[:64]]) == 0
    assert torch.count_nonzero(dk[:, :, inv[64:128]]) == 0
    assert torch.count_nonzero(dv[:, :, inv[64:128]]) == 0


def test_backward_empty_mask_gives_zero(A):
    geom, og = PT.geoms(1, 2, 2, 16, 16, 128)
    q, k, v, dout = _inputs(1, 2, 2, 16, 16, 128, seed=5)
    run = A.NablaAttention(geom, A.MaskParams(mode="cdf", thr=0.0, sta=(0, 0, 0)), want_lse=True)
    run(q, k, v)
    dq, dk, dv = run.backward(q, k, v, dout)
    torch.cuda.synchronize()
    assert int(run.counts.sum()) == 0
    for t in (dq, dk, dv):
        assert torch.count_nonzero(t) == 0


def test_backward_deterministic_and_reusable_workspace(A):
    """Two calls with the same workspace give bit-identical gradients (no atomics in the path)."""
    geom, og = PT.geoms(1, 2, 3, 24, 40, 128)
    q, k, v, dout = _inputs(1, 2, 3, 24, 40, 128, seed=6)
    run = A.NablaAttention(geom, A.MaskParams(mode="cdf", thr=0.8), want_lse=True)
    run(q, k, v)
    ws = torch.empty(A.sparse_attn_bwd_workspace_bytes(geom), dtype=torch.uint8, device=DEV)
    a = [t.clone() for t in run.backward(q, k, v, dout, workspace=ws)]
    b = run.backward(q, k, v, dout, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def _sampled(og, run, heads, n_rand_q=2, kcols=("max", "min", "rand")):
    """Sampled blocks per head: (head, query blocks, key blocks, rows whose O / lse decide them).
    Query blocks: the longest row plus random ones; key blocks: the longest / shortest column
    and a random one, as asked."""
    gm = PT.gpu_mask(run.words, og)
    rng = np.random.default_rng(1)
    picks = []
    for h in heads:
        m = gm[0, h]
        qblocks = sorted(set([int(m.sum(1).argmax())] + rng.integers(0, og.nb, n_rand_q).tolist()))
        col = m.sum(0)
        pick = {"max": int(col.argmax()), "min": int(col.argmin()), "rand": int(rng.integers(0, og.nb))}
        kblocks = sorted(set(pick[c] for c in kcols))
        need = sorted(set(qblocks).union(*[np.nonzero(m[:, j])[0].tolist() for j in kblocks]))
        picks.append((h, qblocks, kblocks, need))
    return gm, picks


def _compare_sampled(og, q, k, v, dout, gm, picks, dq, dk, dv, tag, o_given=None, dtype="bf16"):
    scale = 1.0 / math.sqrt(og.d)
    inv = np.argsort(R.fractal_positions(og))
    got = {n: [] for n in NAMES}
    ref = {n: [] for n in NAMES}
    for h, qblocks, kblocks, _ in picks:
        Qr, gh = _head(q, 0, h, og)
        Kr, _ = _head(k, 0, h, og)
        Vr, _ = _head(v, 0, h, og)
        dOr, _ = _head(dout, 0, h, og)
        Og = None if o_given is None else _head(o_given, 0, h, og)[0]
        m = gm[0, h]
        rows = PT.sample_rows(og, qblocks)
        rq, _, _ = R.masked_attention_backward_head(Qr, Kr, Vr, dOr, m, gh, scale, rows=rows, O=Og)
        got["dq"].append(dq[0, h, torch.from_numpy(inv[rows]).to(DEV)].float().cpu().numpy())
        ref["dq"].append(rq)
        for j in kblocks:
            keeps = np.nonzero(m[:, j])[0]
            print(f"  oracle backward, head {h}, key block {j}: {len(keeps)} query blocks keep it", flush=True)
            krows = PT.sample_rows(og, [j])
            qrows = PT.sample_rows(og, keeps) if len(keeps) else np.zeros(0, dtype=np.int64)
            _, rk, rv = R.masked_attention_backward_head(Qr, Kr, Vr, dOr, m, gh, scale, rows=qrows, O=Og)
            sel = torch.from_numpy(inv[krows]).to(DEV)
            got["dk"].append(dk[0, h, sel].float().cpu().numpy())
            got["dv"].append(dv[0, h, sel].float().cpu().numpy())
            ref["dk"].append(rk[krows])
            ref["dv"].append(rv[krows])
    errs = {n: PT.grad_errors(np.concatenate(got[n]), np.concatenate(ref[n])) for n in NAMES}
    print(f"{tag}: " + ", ".join(f"{n} rel {r:.2e} max {m:.2e}" for n, (r, m) in errs.items()), flush=True)
    for n in NAMES:
        PT.compare_grad(np.concatenate(got[n]), np.concatenate(ref[n]), f"{tag} {n}", dtype)


def _setup(A, name, **over):
    w = WORKLOADS[name].with_(**over) if over else WORKLOADS[name]
    geom, og = PT.geoms(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    q, k, v = make_qkv(w, device=DEV)
    dout = make_dout(w.B, w.H, geom.N, w.d, seed=7, device=DEV)
    run = A.NablaAttention(geom, A.MaskParams(mode=w.mode, thr=w.thr, tau=w.tau, sta=tuple(w.sta), gamma=w.gamma,
                                              lam=w.lam), want_lse=True)
    run(q, k, v)
    torch.cuda.synchronize()
    return w, geom, og, q, k, v, dout, run


def _kernel_parity_sampled(A, tag, name, heads, n_rand_q=2, kcols=("max", "min", "rand"), **over):
    """The backward entry point handed the oracle's O (bf16) and lse on every row that the
    sampled outputs depend on (the sampled query blocks and every query block keeping a
    sampled key block). The remaining rows get O = 0 and an lse of float32 max, which makes
    their P zero; they only feed outputs that are not compared."""
    w, geom, og, q, k, v, dout, run = _setup(A, name, **over)
    gm, picks = _sampled(og, run, heads(og), n_rand_q, kcols)
    scale = 1.0 / math.sqrt(og.d)
    inv = np.argsort(R.fractal_positions(og))
    O = np.zeros((og.B, og.H, og.N, og.d))
    lse = np.full((og.B, og.H, og.N), np.finfo(np.float32).max)
    for h, _, _, need in picks:
        Qr, gh = _head(q, 0, h, og)
        Kr, _ = _head(k, 0, h, og)
        Vr, _ = _head(v, 0, h, og)
        rows = PT.sample_rows(og, need)
        print(f"  oracle forward, head {h}: {len(need)} query blocks", flush=True)
        Or, lr = R.masked_attention_head(Qr, Kr, Vr, gm[0, h], gh, scale, rows=rows)
        O[0, h, inv[rows]] = Or
        lse[0, h, rows] = lr
    o = torch.from_numpy(O).to(torch.bfloat16).to(DEV)
    lse_t = torch.from_numpy(lse.astype(np.float32)).to(DEV)
    print(f"backward {tag} full size, oracle O / lse on {sum(len(p[3]) for p in picks)} query blocks", flush=True)
    dq, dk, dv = A.sparse_attn_bwd(q, k, v, o, dout, lse_t, run.words, run.counts, run.lists, geom)
    torch.cuda.synchronize()
    _compare_sampled(og, q, k, v, dout, gm, picks, dq, dk, dv, f"{tag} kernel", o_given=o)


def test_backward_480p_kernel_parity_sampled(A):
    """Full-size 480p (12 heads, nb = 588), two heads, longest / shortest / random columns."""
    _kernel_parity_sampled(A, "480p", "480p", lambda og: (0, og.H - 1))


def test_backward_720p_kernel_parity_sampled(A):
    """Full-size 720p (40 heads, nb = 1260): dQ on sampled query blocks of two heads, dK / dV on
    each head's shortest column (the longest would take the oracle minutes)."""
    _kernel_parity_sampled(A, "720p", "720p", lambda og: (0, og.H - 1), n_rand_q=1, kcols=("min",))


def test_backward_maximum_blocks_per_row(A):
    """nb = 4096 key blocks (16 frames of 128 x 128 tokens, one head, d = 64): column lists of
    the largest size; dQ on two query blocks, dK / dV on the shortest column. A tight dynamic
    threshold (tau = 0.5) keeps the columns short enough for the oracle."""
    _kernel_parity_sampled(A, "max-nb", "480p", lambda og: (0,), n_rand_q=1, kcols=("min",),
                           H=1, T=16, Hs=128, Ws=128, d=64, mode="dyn", tau=0.5)


def test_backward_480p_end_to_end_sampled(A):
    """Full-size 480p, GPU forward then GPU backward, against the exact oracle gradients."""
    w, geom, og, q, k, v, dout, run = _setup(A, "480p")
    gm, picks = _sampled(og, run, (0, og.H - 1))
    print("backward 480p full size, end to end", flush=True)
    dq, dk, dv = run.backward(q, k, v, dout)
    torch.cuda.synchronize()
    _compare_sampled(og, q, k, v, dout, gm, picks, dq, dk, dv, "480p e2e")


def test_autograd_function_matches_entry_points(A):
    """nabla_attention under torch.autograd gives the forward output and, from backward(), the
    gradients of the explicit entry-point calls, bit for bit."""
    B, H, T, Hs, Ws, d = 1, 2, 3, 24, 40, 128
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    q, k, v, dout = _inputs(B, H, T, Hs, Ws, d, seed=31)
    prm = A.MaskParams(mode="cdf", thr=0.8)
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = A.nabla_attention(qa, ka, va, geom, prm)
    out.backward(dout)
    run = A.NablaAttention(geom, prm, want_lse=True)
    run(q, k, v)
    dq, dk, dv = run.backward(q, k, v, dout)
    torch.cuda.synchronize()
    assert torch.equal(out.detach().view(torch.int16), run.out.view(torch.int16))
    for got, want in ((qa.grad, dq), (ka.grad, dk), (va.grad, dv)):
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("d,geo", [(64, (1, 2, 8, 16, 16)), (128, (1, 1, 3, 16, 24)), (64, (2, 1, 3, 24, 40))])
def test_backward_f32_kernel_parity(A, d, geo):
    """float32 backward on the oracle's O (float32) and lse, every element."""
    B, H, T, Hs, Ws = geo
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    q, k, v = make_random_qkv(B, H, T, Hs, Ws, d, "f32", seed=41, device=DEV)
    k = k + 0.25 * q
    dout = make_dout(B, H, geom.N, d, seed=42, device=DEV).float()
    run = A.NablaAttention(geom, A.MaskParams(mode="cdf", thr=0.8), dtype=torch.float32, want_lse=True)
    run(q, k, v)
    torch.cuda.synchronize()
    gm = PT.gpu_mask(run.words, og)
    o, lse = _oracle_forward(q, k, v, gm, og, dtype=torch.float32)
    print(f"backward f32 d{d} nb{geom.nb}", flush=True)
    dq, dk, dv = A.sparse_attn_bwd(q, k, v, o, dout, lse, run.words, run.counts, run.lists, geom)
    torch.cuda.synchronize()
    _check_full(og, q, k, v, dout, gm, dq, dk, dv, f"f32-d{d}", o_given=o, dtype="f32")


def test_backward_tiny_workload_end_to_end(A):
    """The tiny workload (float32, d = 64) through the autograd function, against the exact oracle."""
    w = WORKLOADS["tiny"]
    geom, og = PT.geoms(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    q, k, v = make_qkv(w, device=DEV)
    dout = make_dout(w.B, w.H, geom.N, w.d, seed=43, device=DEV).float()
    prm = A.MaskParams(mode=w.mode, thr=w.thr, tau=w.tau, sta=tuple(w.sta))
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = A.nabla_attention(qa, ka, va, geom, prm)
    out.backward(dout)
    torch.cuda.synchronize()
    run = A.NablaAttention(geom, prm, dtype=torch.float32)
    run(q, k, v)
    torch.cuda.synchronize()
    _check_full(og, q, k, v, dout, PT.gpu_mask(run.words, og), qa.grad, ka.grad, va.grad, "tiny e2e", dtype="f32")


MANY = [
    # (name, dtype, d, (B, H, T, Hs, Ws), MaskParams kwargs)
    ("4100-heads-long-lists", "bf16", 64, (1, 4100, 4, 40, 40), dict(mode="dyn", tau=1e9)),  # keep all, nb = 100
    ("65600-heads-one-block", "bf16", 64, (1, 65600, 1, 8, 8), dict(mode="cdf", thr=0.5)),
    ("4100-heads-f32", "f32", 64, (1, 4100, 4, 8, 8), dict(mode="cdf", thr=0.9)),
]


@pytest.mark.parametrize("case", MANY, ids=[c[0] for c in MANY])
def test_many_heads_end_to_end(A, case):
    """More (b, h) than the visiting-order kernels have workgroups (4096: each then takes several
    heads; 4100 heads of 100 blocks put the bf16 forward in its longest-first mode, the float32
    forward orders its rows the same way) and 65,600 one-block heads for the column lists' grid.
    Forward output and LSE of whole heads, and the gradients of the GPU's own forward on sampled
    blocks, against the oracle on the first head, the heads either side of 4096 and the last."""
    name, dtype, d, geo, pkw = case
    B, H, T, Hs, Ws = geo
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    q, k, v = make_random_qkv(B, H, T, Hs, Ws, d, dtype, seed=51, device=DEV)
    k = (k.float() + 0.25 * q.float()).to(q.dtype)
    dout = make_dout(B, H, geom.N, d, seed=52, device=DEV).to(q.dtype)
    run = A.NablaAttention(geom, A.MaskParams(**pkw), dtype=q.dtype, want_lse=True)
    run(q, k, v)
    dq, dk, dv = run.backward(q, k, v, dout)
    torch.cuda.synchronize()
    heads = sorted({0, 4095, 4096, H - 1} & set(range(H)))
    gm = PT.gpu_mask(run.words, og)
    scale = 1.0 / math.sqrt(og.d)
    for h in heads:
        Qr, gh = _head(q, 0, h, og)
        Kr, _ = _head(k, 0, h, og)
        Vr, _ = _head(v, 0, h, og)
        Or, lse = R.masked_attention_head(Qr, Kr, Vr, gm[0, h], gh, scale)
        PT.compare_attention(run.out[0, h].float().cpu().numpy(), R.inverse_reorder(Or, gh), dtype)
        got = run.lse[0, h].cpu().numpy()
        assert np.array_equal(np.isneginf(got), np.isneginf(lse))
        fin = np.isfinite(lse)
        np.testing.assert_allclose(got[fin], lse[fin], rtol=0, atol=2e-3 if dtype == "bf16" else 1e-4)
    _, picks = _sampled(og, run, heads, n_rand_q=1, kcols=("min",))
    _compare_sampled(og, q, k, v, dout, gm, picks, dq, dk, dv, f"{name} e2e", dtype=dtype)
