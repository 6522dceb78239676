"""HIP path vs the CPU oracle, through the C-ABI (via the ctypes binding).

Small geometries are compared element by element; the five workloads run at
their full sizes with the masks compared in full and the attention compared on
sampled query blocks (every row of each sampled block), including each head's
longest and shortest row.
"""
import math

import numpy as np
import pytest
import torch

from gen import WORKLOADS, make_qkv, make_random_qkv
from oracle import nabla_ref as R
from tests import parity as PT

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def A():
    import block_sparse_attention_21_amd as A
    assert torch.cuda.is_available(), "the gpu tests need a HIP device"
    return A


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def _pooled_oracle(x: torch.Tensor, og: R.Geom) -> np.ndarray:
    """Oracle block means, one head at a time (keeps host memory small at the big sizes)."""
    out = np.empty((og.B, og.H, og.nb, og.d))
    for h in range(og.H):
        gh = R.Geom(og.B, 1, og.T, og.Hs, og.Ws, og.d, og.P)
        out[:, h:h + 1] = R.block_means(R.reorder(R.to64(x[:, h:h + 1]), gh), gh)
    return out


# ---------------------------------------------------------------- reorder + pool
@pytest.mark.parametrize("dtype,d,geo", [
    ("f32", 64, (1, 2, 8, 16, 16)), ("bf16", 128, (1, 3, 3, 24, 40)), ("bf16", 64, (2, 1, 2, 16, 8)),
    ("f32", 128, (1, 1, 5, 8, 24)), ("bf16", 128, (1, 1, 1, 8, 8)),
])
def test_reorder_and_pool(A, dtype, d, geo):
    B, H, T, Hs, Ws = geo
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    x = make_random_qkv(B, H, T, Hs, Ws, d, dtype, seed=3, device=DEV)[0]
    y, pooled = A.reorder(x, geom, want_pooled=True)
    yt = A.reorder(x, geom, layout="block_t")
    back = A.reorder(y, geom, inverse=True)
    torch.cuda.synchronize()
    xb = _bits(x)
    ref = R.reorder(xb, og)
    assert np.array_equal(_bits(y), ref)
    ref_t = ref.reshape(B, H, og.nb, 64, d).transpose(0, 1, 2, 4, 3)
    assert np.array_equal(_bits(yt), ref_t)
    assert np.array_equal(_bits(back), xb)
    pref = R.block_means(R.reorder(R.to64(x), og), og)
    np.testing.assert_allclose(pooled.cpu().numpy(), pref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("dtype,d,geo", [
    ("f32", 64, (1, 2, 8, 16, 16)), ("bf16", 128, (1, 3, 3, 24, 40)), ("bf16", 64, (2, 1, 2, 16, 8)),
    ("f32", 128, (1, 1, 5, 8, 24)), ("bf16", 128, (1, 1, 1, 8, 8)),
])
def test_pool_qk_reorder_v(A, dtype, d, geo):
    """The one-launch first step: Q and K block means and V's channel-major fractal blocks equal
    the oracle's (V bit-exact, means to float64 rounding) and, bit for bit, the three separate
    abla_reorder passes."""
    B, H, T, Hs, Ws = geo
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    q, k, v = make_random_qkv(B, H, T, Hs, Ws, d, dtype, seed=4, device=DEV)
    qbar, kbar, v_rt = A.pool_qk_reorder_v(q, k, v, geom)
    sq = A.reorder(q, geom, pool_only=True)
    sk = A.reorder(k, geom, pool_only=True)
    sv = A.reorder(v, geom, layout="block_t")
    pq, pk, none = A.pool_qk_reorder_v(q, k, None, geom)  # the pooling-only form
    torch.cuda.synchronize()
    assert torch.equal(qbar, sq) and torch.equal(kbar, sk)
    assert none is None and torch.equal(pq, sq) and torch.equal(pk, sk)
    assert np.array_equal(_bits(v_rt), _bits(sv))
    ref_t = R.reorder(_bits(v), og).reshape(B, H, og.nb, 64, d).transpose(0, 1, 2, 4, 3)
    assert np.array_equal(_bits(v_rt), ref_t)
    for got, x in ((qbar, q), (kbar, k)):
        np.testing.assert_allclose(got.cpu().numpy(), R.block_means(R.reorder(R.to64(x), og), og),
                                   rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- small end-to-end, every element
SMALL = [
    # (name, dtype, d, (B,H,T,Hs,Ws), MaskParams kwargs)
    ("tiny-like", "f32", 64, (1, 2, 8, 16, 16), dict(mode="cdf", thr=0.8)),
    ("ragged-bf16", "bf16", 128, (1, 2, 3, 24, 88), dict(mode="cdf", thr=0.7)),  # nb = 99
    ("d64-bf16", "bf16", 64, (2, 1, 4, 16, 40), dict(mode="cdf", thr=0.9)),
    ("dyn-bf16", "bf16", 128, (1, 2, 3, 32, 32), dict(mode="dyn", tau=2.0)),
    ("no-sta", "bf16", 128, (1, 1, 5, 16, 24), dict(mode="cdf", thr=0.6, sta=(0, 0, 0))),
    ("full", "bf16", 128, (1, 1, 2, 16, 32), dict(mode="cdf", thr=1.0)),
    ("f32-d128", "f32", 128, (1, 1, 3, 16, 16), dict(mode="cdf", thr=0.5, sta=(1, 3, 3))),
    ("one-block", "bf16", 128, (1, 2, 1, 8, 8), dict(mode="cdf", thr=0.5)),
    ("nb-300", "bf16", 64, (1, 1, 3, 80, 80), dict(mode="cdf", thr=0.95)),  # 2 keys/thread in the select
    ("nb-600", "bf16", 64, (1, 1, 6, 80, 80), dict(mode="cdf", thr=0.95, sta=(0, 0, 0))),
    ("static", "bf16", 128, (1, 2, 5, 24, 40), dict(mode="static", gamma=0.5, lam=0.1)),
    ("static-f32-no-sta", "f32", 64, (1, 1, 6, 16, 24), dict(mode="static", gamma=0.3, lam=0.0, sta=(0, 0, 0))),
    ("static-gamma1", "bf16", 64, (1, 1, 3, 16, 16), dict(mode="static", gamma=1.0, lam=0.0)),
]


def _run_small(A, dtype, d, geo, pkw, qk_scale=1.0, seed=5):
    B, H, T, Hs, Ws = geo
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    prm = A.MaskParams(**pkw)
    q, k, v = make_random_qkv(B, H, T, Hs, Ws, d, dtype, seed=seed, device=DEV, scale=qk_scale)
    # Give the pooled keys some structure so the CDF cut is not trivial.
    k = (k.float() + 2.0 * q.float()).to(q.dtype)
    # The V path is fixed (channel-major V pass for bf16) so that these cases keep covering it;
    # the original-order V read and the choice between the two have tests of their own.
    run = A.NablaAttention(geom, prm, dtype=q.dtype, want_lse=True, fuse_v=dtype == "f32")
    run(q, k, v)
    torch.cuda.synchronize()
    return geom, og, prm, q, k, v, run


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_end_to_end(A, case):
    name, dtype, d, geo, pkw = case
    geom, og, prm, q, k, v, run = _run_small(A, dtype, d, geo, pkw)
    op = PT.oracle_params(prm)
    res = R.nabla_attention(q, k, v, og, op)
    rep = PT.check_mask(run.words, run.counts, run.lists, res.mask, op, og)
    gm = PT.gpu_mask(run.words, og)
    ref = R.nabla_attention(q, k, v, og, op, block_mask=gm)
    out = run.out.float().cpu().numpy()
    max_abs, rel = PT.compare_attention(out, ref.O, dtype)
    lse = run.lse.cpu().numpy()
    fin = np.isfinite(ref.lse_r)
    assert np.array_equal(np.isfinite(lse), fin)
    np.testing.assert_allclose(lse[fin], ref.lse_r[fin], rtol=0, atol=1e-4 if dtype == "f32" else 2e-3)
    print(f"{name}: kept {rep.kept}/{rep.total}, band diffs {rep.exempt_diff}, max|dO| {max_abs:.2e}, rel {rel:.2e}")


# ---------------------------------------------------------------- running maximum across tiles
def _ramp_qkv(order, d, fuse_seed=11):
    """Q and K whose scores grow (or fall, or jump) by about 6 nats from one key block to the
    next in the walk order: every key of block j is a_j * u plus noise and every query c * u plus
    noise, with a_j from `order`; V i.i.d. normal. bf16, B = 1, H = 2, 2 x 32 x 32 tokens."""
    B, H, T, Hs, Ws = 1, 2, 2, 32, 32
    g = torch.Generator().manual_seed(fuse_seed)
    N = T * Hs * Ws
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hs), np.arange(Ws), indexing="ij")
    blk = ((t * (Hs // 8) + y // 8) * (Ws // 8) + x // 8).reshape(-1)  # key block of each token
    a = torch.tensor(np.asarray(order, dtype=np.float64)[blk], dtype=torch.float32)
    u = torch.randn((H, 1, d), generator=g)
    c = 6.0 * math.sqrt(d) / (u * u).sum(-1, keepdim=True)  # c * |u|^2 / sqrt(d) = 6 nats per unit of a_j
    q = (c * u + 0.3 * torch.randn((H, N, d), generator=g)).unsqueeze(0)
    k = (a[None, :, None] * u + 0.3 * torch.randn((H, N, d), generator=g)).unsqueeze(0)
    v = torch.randn((B, H, N, d), generator=g)
    return (B, H, T, Hs, Ws), q.to(torch.bfloat16).to(DEV), k.to(torch.bfloat16).to(DEV), v.to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("fuse_v", [False, True], ids=["v-blocks", "v-original"])
@pytest.mark.parametrize("shape", ["rising", "falling", "jumping"])
def test_running_maximum_across_tiles(A, shape, fuse_v):
    """Probabilities are formed against the running maximum of the earlier tiles and the row is
    rebased when a tile's probabilities exceed it: with scores rising ~6 nats per key block
    every tile rebases, falling only the first does, jumping mixes both; the row maxima reach
    ~190 nats, so any missed rebase overflows. Every element against the oracle (full mask)."""
    nb = 32
    order = {"rising": np.arange(1, nb + 1), "falling": np.arange(nb, 0, -1),
             "jumping": (np.arange(nb) * 7) % nb + 1}[shape]
    for d in (64, 128):
        geo, q, k, v = _ramp_qkv(order, d)
        geom, og = PT.geoms(*geo, d)
        prm = A.MaskParams(mode="cdf", thr=1.0)
        run = A.NablaAttention(geom, prm, dtype=q.dtype, want_lse=True, fuse_v=fuse_v)
        run(q, k, v)
        torch.cuda.synchronize()
        assert int(run.counts.min()) == nb
        op = PT.oracle_params(prm)
        ref = R.nabla_attention(q, k, v, og, op, block_mask=PT.gpu_mask(run.words, og))
        assert np.isfinite(ref.lse_r).all() and ref.lse_r.max() > 150.0
        max_abs, rel = PT.compare_attention(run.out.float().cpu().numpy(), ref.O, "bf16")
        lse = run.lse.cpu().numpy()
        np.testing.assert_allclose(lse, ref.lse_r, rtol=0, atol=2e-3)
        print(f"{shape} d={d} fuse_v={fuse_v}: max|dO| {max_abs:.2e} rel {rel:.2e}, max lse {lse.max():.1f}")


def test_empty_rows_give_zero(A):
    geom, og, prm, q, k, v, run = _run_small(A, "bf16", 128, (1, 2, 2, 16, 16), dict(mode="cdf", thr=0.0,
                                                                                     sta=(0, 0, 0)))
    assert int(run.counts.sum()) == 0
    assert int(run.words.abs().sum()) == 0
    assert torch.count_nonzero(run.out) == 0
    assert torch.isneginf(run.lse).all()


def test_dyn_tau_zero_keeps_argmax(A):
    geom, og, prm, q, k, v, run = _run_small(A, "bf16", 128, (1, 1, 3, 16, 24), dict(mode="dyn", tau=0.0,
                                                                                     sta=(0, 0, 0)))
    op = PT.oracle_params(prm)
    res = R.nabla_attention(q, k, v, og, op)
    PT.check_mask(run.words, run.counts, run.lists, res.mask, op, og)
    assert (run.counts >= 1).all()


def test_fractal_order_output_and_determinism(A):
    geom, og, prm, q, k, v, run = _run_small(A, "bf16", 128, (1, 2, 3, 16, 24), dict(mode="cdf", thr=0.8))
    out1 = run.out.clone()
    run(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out1, run.out)
    o_r = A.sparse_attn_fwd(q, k, run.v_rt, run.counts, run.lists, geom, out_original_order=False,
                            qk_original_order=True)
    back = A.reorder(o_r, geom, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back, out1)


@pytest.mark.parametrize("dtype,d,geo", [
    ("bf16", 128, (1, 2, 3, 24, 88)), ("bf16", 64, (2, 1, 4, 16, 40)), ("f32", 64, (1, 2, 4, 16, 16)),
    ("bf16", 128, (1, 1, 2, 8, 8)), ("bf16", 64, (1, 1, 5, 8, 136)),
])
def test_fused_and_unfused_paths_agree(A, dtype, d, geo):
    """Q and K read in the original order (the default path: pooling only, no reordered copies),
    and V as well (its V^T operand through LDS transpose loads), give bit-identically the output
    and LSE of the path that reads fractal-order copies; the pooling-only pass writes the same
    block means as the reorder + pool pass."""
    B, H, T, Hs, Ws = geo
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    q, k, v = make_random_qkv(B, H, T, Hs, Ws, d, dtype, seed=9, device=DEV)
    k = (k.float() + 2.0 * q.float()).to(q.dtype)
    prm = A.MaskParams(mode="cdf", thr=0.7)
    fused = A.NablaAttention(geom, prm, dtype=q.dtype, want_lse=True, fuse_v=dtype == "f32")
    plain = A.NablaAttention(geom, prm, dtype=q.dtype, want_lse=True, fused=False)
    all_orig = A.NablaAttention(geom, prm, dtype=q.dtype, want_lse=True, fuse_v=True)
    fused(q, k, v)
    plain(q, k, v)
    all_orig(q, k, v)
    torch.cuda.synchronize()
    assert fused.q_r is None and plain.q_r is not None and all_orig.v_rt is None
    assert torch.equal(fused.qbar, plain.qbar) and torch.equal(fused.kbar, plain.kbar)
    assert torch.equal(fused.words, plain.words)
    for run in (fused, all_orig):
        assert np.array_equal(_bits(run.out), _bits(plain.out))
        assert torch.equal(run.lse, plain.lse)


def test_graph_replay_matches_eager(A):
    """The whole step captured into a HIP graph: each replay, on new inputs copied in by eager
    work with synchronizations in between, gives bit-identically what an eager run gives."""
    geo, d = (1, 2, 6, 32, 48), 128
    B, H, T, Hs, Ws = geo
    geom, _ = PT.geoms(B, H, T, Hs, Ws, d)
    prm = A.MaskParams(mode="cdf", thr=0.8, sta=(3, 3, 3))
    inputs = []
    for seed in (11, 12, 13):
        q, k, v = make_random_qkv(B, H, T, Hs, Ws, d, "bf16", seed=seed, device=DEV)
        inputs.append((q, (k.float() + 2.0 * q.float()).to(q.dtype), v))
    qb, kb, vb = (x.clone() for x in inputs[0])
    run = A.NablaAttention(geom, prm, dtype=torch.bfloat16, want_lse=True)
    graph = run.capture(qb, kb, vb)
    torch.cuda.synchronize()
    ref = A.NablaAttention(geom, prm, dtype=torch.bfloat16, want_lse=True)
    for rep, (q, k, v) in enumerate(inputs + inputs[:1]):
        qb.copy_(q)
        kb.copy_(k)
        vb.copy_(v)
        graph.replay()
        ref(q, k, v)
        torch.cuda.synchronize()
        for name in ("out", "lse", "words", "counts"):
            assert torch.equal(getattr(run, name), getattr(ref, name)), (rep, name)
        valid = torch.arange(geom.nb, device=DEV)[None, None, None, :] < ref.counts[..., None]
        assert torch.equal(run.lists[valid], ref.lists[valid]), rep


def test_binding_errors_on_device(A):
    geom = A.Geometry(1, 1, 1, 8, 8, 128)
    x = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(A.AblaError) as e:
        A.build_mask(torch.zeros(1, 1, 1, 128, device=DEV, dtype=torch.float64),
                     torch.zeros(1, 1, 1, 128, device=DEV, dtype=torch.float64), geom,
                     A.MaskParams(thr=math.nan))
    assert e.value.code == A.ERR_INVALID
    with pytest.raises(ValueError):
        A.reorder(x[..., :64], geom)


def test_overlapping_buffers_rejected_on_device(A):
    # Real device buffers with an empty mask (a launch would only write zeros), aliased so that
    # the entry points must refuse them before launching.
    geom = A.Geometry(1, 1, 1, 8, 8, 128)
    q, k, v = (torch.randn(1, 1, 64, 128, device=DEV).to(torch.bfloat16) for _ in range(3))
    v_rt = torch.zeros(1, 1, 1, 128, 64, dtype=torch.bfloat16, device=DEV)
    counts = torch.zeros(1, 1, 1, dtype=torch.int32, device=DEV)
    lists = torch.zeros(1, 1, 1, 1, dtype=torch.int32, device=DEV)
    words = torch.zeros(1, 1, 1, 1, dtype=torch.int32, device=DEV)
    buf = torch.zeros(1024, dtype=torch.float32, device=DEV)
    lse = buf[:64].view(1, 1, 64)
    with pytest.raises(A.AblaError) as e:  # the workspace (large enough) holds lse
        A.sparse_attn_fwd(q, k, v_rt, counts, lists, geom, qk_original_order=True, lse=lse,
                          workspace=buf.view(torch.uint8))
    assert e.value.code == A.ERR_INVALID
    o = torch.zeros_like(q)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    with pytest.raises(A.AblaError) as e:  # the workspace is dq's memory
        A.sparse_attn_bwd(q, k, v, o, o, lse, words, counts, lists, geom, dq=dq, dk=dk, dv=dv,
                          workspace=dq.view(torch.uint8).flatten())
    assert e.value.code == A.ERR_INVALID
    torch.cuda.synchronize()


# ---------------------------------------------------------------- the five workloads at full size
def _workload(A, name, fuse_v=None, **over):
    """Run one workload at full size. The output and LSE buffers are filled with NaN first, so
    a row the kernels never write is seen by _check_written."""
    w = WORKLOADS[name].with_(**over) if over else WORKLOADS[name]
    geom, og = PT.geoms(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    prm = A.MaskParams(mode=w.mode, thr=w.thr, tau=w.tau, sta=tuple(w.sta), gamma=w.gamma, lam=w.lam)
    q, k, v = make_qkv(w, device=DEV)
    if fuse_v is None:  # the channel-major V pass for bf16 unless a test asks for the other path
        fuse_v = w.dtype == "f32"
    run = A.NablaAttention(geom, prm, dtype=q.dtype, want_lse=True, fuse_v=fuse_v)
    run.out.fill_(math.nan)
    run.lse.fill_(math.nan)
    run(q, k, v)
    torch.cuda.synchronize()
    return w, geom, og, prm, q, k, v, run


def _check_written(run, og):
    """Every output element is written and finite; the LSE is finite exactly on the rows whose
    block keeps something and -inf on the others."""
    assert bool(torch.isfinite(run.out).all()), "output rows left unwritten or not finite"
    live = (run.counts > 0).repeat_interleave(og.bs, dim=-1)
    assert bool(torch.isfinite(run.lse[live]).all())
    assert bool(torch.isneginf(run.lse[~live]).all())


def _check_workload_mask(A, w, og, prm, q, k, run):
    qbar = _pooled_oracle(q, og)
    kbar = qbar if torch.equal(q, k) else _pooled_oracle(k, og)
    op = PT.oracle_params(prm)
    mres = R.build_block_mask(qbar, kbar, og, op)
    rep = PT.check_mask(run.words, run.counts, run.lists, mres, op, og)
    return mres, rep


def _head_arrays(og, q, k, v, h):
    gh = R.Geom(1, 1, og.T, og.Hs, og.Ws, og.d, og.P)
    Qr = R.reorder(R.to64(q[0, h]), gh)
    Kr = Qr if torch.equal(q[0, h], k[0, h]) else R.reorder(R.to64(k[0, h]), gh)
    Vr = R.reorder(R.to64(v[0, h]), gh)
    return gh, Qr, Kr, Vr


def _keep_per_head(run, og):
    return [round(float(x), 5) for x in (run.counts.double().sum(-1) / (og.nb * og.nb)).flatten().tolist()]


def _check_blocks(og, q, k, v, run, picks, dtype, lse_err=None):
    """Attention of the chosen query blocks ({head: [blocks]}) against the oracle on the GPU's
    own mask (only the kept key blocks, masked_attention_blocks); output in the original order,
    LSE in fractal order."""
    gm = PT.gpu_mask(run.words, og)
    inv = np.argsort(R.fractal_positions(og))  # fractal position -> original token
    scale = 1.0 / math.sqrt(og.d)
    gpu_all, ref_all = [], []
    for h, blocks in sorted(picks.items()):
        gh, Qr, Kr, Vr = _head_arrays(og, q, k, v, h)
        O_ref, lse_ref = R.masked_attention_blocks(Qr, Kr, Vr, gm[0, h], gh, scale, blocks)
        rows = PT.sample_rows(og, blocks)
        O_gpu = run.out[0, h, torch.from_numpy(inv[rows]).to(DEV)].float().cpu().numpy()
        lse_gpu = run.lse[0, h, torch.from_numpy(rows).to(DEV)].cpu().numpy()
        assert np.array_equal(np.isneginf(lse_gpu), np.isneginf(lse_ref))
        fin = np.isfinite(lse_ref)
        np.testing.assert_allclose(lse_gpu[fin], lse_ref[fin], rtol=0, atol=2e-3 if dtype == "bf16" else 1e-4)
        if lse_err is not None and fin.any():
            lse_err.append(float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()))
        gpu_all.append(O_gpu)
        ref_all.append(O_ref)
    return PT.compare_attention(np.concatenate(gpu_all), np.concatenate(ref_all), dtype)


def _sampled_picks(og, run, n_rand=3, seed=0):
    """Heads 0 and H-1 plus two random ones; in each, the longest and the shortest row and
    random blocks."""
    counts = run.counts.cpu().numpy()
    rng = np.random.default_rng(seed)
    heads = sorted(set([0, og.H - 1] + rng.integers(0, og.H, 2).tolist()))
    return {h: sorted(set([int(counts[0, h].argmax()), int(counts[0, h].argmin())]
                          + rng.integers(0, og.nb, n_rand).tolist())) for h in heads}


def _frame_picks(og, run, all_heads, seed=1):
    """One query block in every frame: in every head (all_heads), or in head f % H for frame f;
    plus each head's longest row."""
    F = og.nbh * og.nbw
    rng = np.random.default_rng(seed)
    counts = run.counts.cpu().numpy()
    picks = {}
    for f in range(og.T):
        for h in (range(og.H) if all_heads else [f % og.H]):
            picks.setdefault(h, set()).add(f * F + int(rng.integers(0, F)))
    for h in picks:
        picks[h].add(int(counts[0, h].argmax()))
    return {h: sorted(b) for h, b in picks.items()}


def test_workload_tiny(A):
    w, geom, og, prm, q, k, v, run = _workload(A, "tiny")
    _check_written(run, og)
    op = PT.oracle_params(prm)
    res = R.nabla_attention(q, k, v, og, op)
    rep = PT.check_mask(run.words, run.counts, run.lists, res.mask, op, og)
    assert rep.diff == 0
    ref = R.nabla_attention(q, k, v, og, op, block_mask=PT.gpu_mask(run.words, og))
    max_abs, rel = PT.compare_attention(run.out.cpu().numpy(), ref.O, "f32")
    lse_err = float(np.abs(run.lse.cpu().numpy() - ref.lse_r).max())
    PT.record(workload="tiny", dtype="f32", keep=rep.kept / rep.total, keep_per_head=_keep_per_head(run, og),
              mask_bits=rep.total, mask_diff=rep.diff, band_blocks=rep.band, band_diff=rep.exempt_diff,
              rows_compared=og.B * og.H * og.N, max_abs=max_abs, rel_l2=rel, lse_max_abs=lse_err)
    print(f"tiny: keep {rep.kept / rep.total:.4f}, max|dO| {max_abs:.2e}")


@pytest.mark.parametrize("name", ["480p", "480p-dyn", "480p-static", "720p", "long"])
def test_workload_full_size(A, name):
    """Full mask comparison; zero differences inside the band at 480p and 480p-dyn (and none
    possible for the static mask). Attention: the 480p family on every row of the last head
    plus sampled blocks of heads 0 and H-1 and two random heads; 720p one block per frame in
    every head; the long clip one block per frame (frame f in head f mod H)."""
    w, geom, og, prm, q, k, v, run = _workload(A, name)
    _check_written(run, og)
    mres, rep = _check_workload_mask(A, w, og, prm, q, k, run)
    if name.startswith("480p"):
        assert rep.diff == 0, f"{rep.diff} mask bits differ (all inside the band)"
        picks = _sampled_picks(og, run)
        picks[og.H - 1] = list(range(og.nb))
    else:
        picks = _frame_picks(og, run, all_heads=(name == "720p"))
    lse_err = []
    max_abs, rel = _check_blocks(og, q, k, v, run, picks, w.dtype, lse_err)
    n_rows = sum(len(b) for b in picks.values()) * og.bs
    PT.record(workload=name, dtype=w.dtype, keep=rep.kept / rep.total, keep_per_head=_keep_per_head(run, og),
              mask_bits=rep.total, mask_diff=rep.diff, band_blocks=rep.band, band_diff=rep.exempt_diff,
              rows_compared=n_rows, max_abs=max_abs, rel_l2=rel, lse_max_abs=max(lse_err))
    print(f"{name}: keep {rep.kept / rep.total:.4f}, band diffs {rep.exempt_diff}, {n_rows} rows compared, "
          f"max|dO| {max_abs:.2e}, rel {rel:.2e}")


def test_workload_480p_v_original_order(A):
    """The attention reading V in the original token order (its V^T operand through LDS
    transpose loads, no reordered copy) against the oracle: every row of head H-1 and sampled
    blocks of the other heads."""
    w, geom, og, prm, q, k, v, run = _workload(A, "480p", fuse_v=True)
    assert run.v_rt is None
    _check_written(run, og)
    picks = _sampled_picks(og, run, seed=3)
    picks[og.H - 1] = list(range(og.nb))
    max_abs, rel = _check_blocks(og, q, k, v, run, picks, w.dtype)
    print(f"480p V original order: max|dO| {max_abs:.2e}, rel {rel:.2e}")


def test_maximum_blocks_per_row(A):
    """The largest supported row: nb = 4096 key blocks (16 frames of 128 x 128 tokens, one head,
    d = 64), the limit of the LDS-resident mask row and of the attention's 12-bit schedule."""
    w, geom, og, prm, q, k, v, run = _workload(A, "480p", H=1, T=16, Hs=128, Ws=128, d=64)
    assert geom.nb == 4096
    _check_written(run, og)
    mres, rep = _check_workload_mask(A, w, og, prm, q, k, run)
    picks = _sampled_picks(og, run)
    picks[0] = sorted(set(picks[0]) | set(_frame_picks(og, run, all_heads=True)[0]))
    max_abs, rel = _check_blocks(og, q, k, v, run, picks, w.dtype)
    print(f"max-nb: keep {rep.kept / rep.total:.4f}, band diffs {rep.exempt_diff}, "
          f"max|dO| {max_abs:.2e}, rel {rel:.2e}")


# ---------------------------------------------------------------- the sparse regime, every element
SPARSE = [
    # (name, workload overrides): the video recipe at reduced size, keep 5-10 %
    ("video-cdf", dict(H=2, T=12, Hs=32, Ws=64, mode="cdf", thr=0.7)),
    ("video-dyn-tau2", dict(H=2, T=12, Hs=32, Ws=64, mode="dyn", tau=2.0)),
    ("video-cdf-no-sta", dict(H=2, T=16, Hs=32, Ws=56, mode="cdf", thr=0.7, sta=(0, 0, 0))),
    ("video-dyn-odd-T", dict(H=2, T=11, Hs=40, Ws=64, mode="dyn", tau=3.0)),
    # head dim 64 (its own kernel instances): keep about 7 % and 11 %, the second with an odd T
    ("video-d64-dyn", dict(H=2, T=12, Hs=32, Ws=64, d=64, mode="dyn", tau=2.0)),
    ("video-d64-cdf-odd-T", dict(H=2, T=13, Hs=32, Ws=64, d=64, mode="cdf", thr=0.5)),
]


@pytest.mark.parametrize("fuse_v", [False, True], ids=["v-blocks", "v-original"])
@pytest.mark.parametrize("case", SPARSE, ids=[c[0] for c in SPARSE])
def test_sparse_regime_every_element(A, case, fuse_v):
    """Content-adaptive masks that keep 5-10 % of the blocks (the dynamic threshold dropping most
    of every row): mask bits equal, and every output and LSE element compared."""
    name, over = case
    w, geom, og, prm, q, k, v, run = _workload(A, "480p", fuse_v=fuse_v, **over)
    _check_written(run, og)
    mres, rep = _check_workload_mask(A, w, og, prm, q, k, run)
    assert rep.diff == 0
    assert rep.kept < 0.15 * rep.total
    max_abs, rel = _check_blocks(og, q, k, v, run, {h: list(range(og.nb)) for h in range(og.H)}, w.dtype)
    print(f"{name} {'v-original' if fuse_v else ''}: keep {rep.kept / rep.total:.4f}, "
          f"max|dO| {max_abs:.2e}, rel {rel:.2e}")


@pytest.mark.parametrize("case", [c for c in SMALL if c[1] == "bf16"][:6], ids=lambda c: c[0])
def test_small_v_original_order(A, case):
    """The original-order V path against the oracle on the small geometries."""
    name, dtype, d, geo, pkw = case
    B, H, T, Hs, Ws = geo
    geom, og = PT.geoms(B, H, T, Hs, Ws, d)
    prm = A.MaskParams(**pkw)
    q, k, v = make_random_qkv(B, H, T, Hs, Ws, d, dtype, seed=5, device=DEV)
    k = (k.float() + 2.0 * q.float()).to(q.dtype)
    run = A.NablaAttention(geom, prm, dtype=q.dtype, want_lse=True, fuse_v=True)
    run(q, k, v)
    torch.cuda.synchronize()
    op = PT.oracle_params(prm)
    ref = R.nabla_attention(q, k, v, og, op, block_mask=PT.gpu_mask(run.words, og))
    PT.compare_attention(run.out.float().cpu().numpy(), ref.O, dtype)


# ---------------------------------------------------------------- ties and near-ties at the CDF cut
def _mask_from_pooled(A, qbar, kbar, geom, og, thr, cut):
    prm = A.MaskParams(mode="cdf", thr=thr, sta=(0, 0, 0), cut=cut)
    words, counts, lists = A.build_mask(torch.from_numpy(qbar).to(DEV), torch.from_numpy(kbar).to(DEV), geom, prm)
    torch.cuda.synchronize()
    op = PT.oracle_params(prm)
    mres = R.build_block_mask(qbar, kbar, og, op)
    return PT.check_mask(words, counts, lists, mres, op, og), PT.gpu_mask(words, og), mres


@pytest.mark.parametrize("cut", ["radix", "bitonic"])
def test_near_tie_at_the_cut_ranked_by_value(A, cut):
    """Two pooled keys that differ only in their low bits: block 40's probability exceeds block
    10's by about 3e-14 relative (below 2^-40, so a ranking on probabilities truncated to 40
    mantissa bits could see a tie), and they are the row's two largest. A threshold of half the top probability keeps only the top rank: block 40
    by value, although the lower index 10 wins an index tie-break. Far outside the band."""
    geom, og = PT.geoms(1, 1, 1, 64, 64, 128)
    rng = np.random.default_rng(7)
    qv = rng.standard_normal(128)
    qbar = np.broadcast_to(qv, (1, 1, og.nb, 128)).copy()
    kbar = 0.2 * rng.standard_normal((1, 1, og.nb, 128))
    u = qv / (qv @ qv)
    kbar[0, 0, 10] += 3.0 * math.sqrt(128) * u  # the row maximum
    kbar[0, 0, 40] = kbar[0, 0, 10] + 3e-14 * math.sqrt(128) * u
    res = R.build_block_mask(qbar, kbar, og, R.MaskParams(mode="cdf", thr=0.5, sta=(0, 0, 0)))
    p = res.Pm[0, 0, 0]
    assert p[40] > p[10] and (p[40] - p[10]) / p[10] < 2.0 ** -40
    assert p.argsort()[-3] not in (10, 40) and p[10] > 1.5 * np.sort(p)[-3]
    rep, gm, mres = _mask_from_pooled(A, qbar, kbar, geom, og, float(p[10]) / 2, cut)
    assert rep.diff == 0
    assert gm[0, 0, :, 40].all() and not gm[0, 0, :, 10].any()
    rep, gm, _ = _mask_from_pooled(A, qbar, kbar, geom, og, float(p[40]) + float(p[10]) / 2, cut)
    assert rep.diff == 0 and gm[0, 0, :, 10].all() and gm[0, 0, :, 40].all()


@pytest.mark.parametrize("cut", ["radix", "bitonic"])
def test_tie_class_split_by_the_cut(A, cut):
    """Exact ties across the cut: three identical pooled keys (blocks 5, 17, 33) are the row's
    largest; a threshold of 1.5 times their probability keeps two of them, the lower indices 5 and
    17. And uniform rows (every pooled key equal, nb = 588 and 300): ceil(thr * nb) blocks, the
    lowest indices, with equality cases left to the band."""
    geom, og = PT.geoms(1, 2, 1, 64, 64, 128)
    rng = np.random.default_rng(8)
    qbar = np.broadcast_to(rng.standard_normal(128), (1, 2, og.nb, 128)).copy()
    kbar = 0.1 * rng.standard_normal((1, 2, og.nb, 128))
    top = kbar[0, 0, 5] + 0.4 * qbar[0, 0, 0]
    for j in (5, 17, 33):
        kbar[0, :, j] = top
    res = R.build_block_mask(qbar, kbar, og, R.MaskParams(mode="cdf", thr=0.5, sta=(0, 0, 0)))
    ptop = float(res.Pm[0, 0, 0, 5])
    assert ptop == res.Pm[0, 0, 0].max() and res.Pm[0, 0, 0, 17] == ptop == res.Pm[0, 0, 0, 33]
    rep, gm, _ = _mask_from_pooled(A, qbar, kbar, geom, og, 1.5 * ptop, cut)
    assert rep.diff == 0
    assert gm[0, 0, :, 5].all() and gm[0, 0, :, 17].all() and not gm[0, 0, :, 33].any()
    for (T, Hs, Ws), thr in (((21, 32, 56), 0.7), ((3, 80, 80), 0.5), ((3, 80, 80), 0.31)):
        geom, og = PT.geoms(1, 1, T, Hs, Ws, 64)
        qbar = rng.standard_normal((1, 1, og.nb, 64))
        kbar = np.broadcast_to(rng.standard_normal(64), (1, 1, og.nb, 64)).copy()
        rep, gm, _ = _mask_from_pooled(A, qbar, kbar, geom, og, thr, cut)
        x = thr * og.nb
        # thr * nb an integer n: the n-th block sits on the threshold (C_excl = thr, in the band)
        allowed = {round(x), round(x) + 1} if abs(x - round(x)) < 1e-9 else {math.ceil(x)}
        got = gm[0, 0].sum(-1)
        assert set(np.unique(got).tolist()) <= allowed, (og.nb, thr, np.unique(got))
        assert gm[0, 0, :, : min(allowed)].all()


@pytest.mark.parametrize("name,over", [
    ("720p", {}), ("long", dict(gamma=0.7, lam=0.02)), ("480p", dict(H=1, T=16, Hs=128, Ws=128, d=64)),
])
def test_static_masks_bit_exact(A, name, over):
    """The Static-Ratio mask has no floating-point decision near a threshold: bit-exact against
    the oracle at full size (720p, the long clip, and nb = 4096), identical for every head."""
    w = WORKLOADS[name].with_(mode="static", **over)
    geom, og = PT.geoms(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    prm = A.MaskParams(mode="static", sta=tuple(w.sta), gamma=w.gamma, lam=w.lam)
    # The static mode reads no pooled vectors: zeros stand in for them.
    qbar = torch.zeros((w.B, w.H, geom.nb, w.d), dtype=torch.float64, device=DEV)
    words, counts, lists = A.build_mask(qbar, qbar, geom, prm)
    torch.cuda.synchronize()
    op = PT.oracle_params(prm)
    gh = R.Geom(1, 1, og.T, og.Hs, og.Ws, og.d, og.P)
    mres = R.build_block_mask(np.zeros((1, 1, og.nb, 1)), np.zeros((1, 1, og.nb, 1)), gh, op)
    gm = PT.gpu_mask(words, og)
    assert np.array_equal(gm, np.broadcast_to(mres.mask[0, 0], gm.shape))
    c = counts.cpu().numpy()
    assert np.array_equal(c, gm.sum(-1))
    L = lists[0, 0].cpu().numpy()
    for i in range(0, og.nb, max(1, og.nb // 64)):
        assert np.array_equal(L[i][: c[0, 0, i]], np.nonzero(gm[0, 0, i])[0])
    print(f"static {name} {over}: nb {og.nb}, keep {gm.mean():.4f}")


@pytest.mark.parametrize("tau", [2.0, 8.0])
def test_dyn_tau_sweep_masks(A, tau):
    w, geom, og, prm, q, k, v, run = _workload(A, "480p-dyn", tau=tau)
    mres, rep = _check_workload_mask(A, w, og, prm, q, k, run)
    PT.record(workload=f"480p-dyn tau={tau}", dtype=w.dtype, keep=rep.kept / rep.total,
              keep_per_head=_keep_per_head(run, og), mask_bits=rep.total, mask_diff=rep.diff, band_blocks=rep.band,
              band_diff=rep.exempt_diff)
    print(f"480p-dyn tau={tau}: keep {rep.kept / rep.total:.4f}, band diffs {rep.exempt_diff}")


# ---------------------------------------------------------------- the two CDF-cut algorithms agree
@pytest.mark.parametrize("name", ["tiny", "480p", "720p", "long"])
def test_cut_algorithms_agree(A, name):
    """Radix select and the bitonic sort find the same last kept rank: identical bits, counts, lists."""
    import dataclasses
    w = WORKLOADS[name]
    geom, og = PT.geoms(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    q, k, _ = make_qkv(w, device=DEV)
    qr, qbar = A.reorder(q, geom, want_pooled=True)
    kr, kbar = A.reorder(k, geom, want_pooled=True)
    out = {}
    for thr in (w.thr, 0.5, 0.999):
        for cut in ("radix", "bitonic"):
            prm = A.MaskParams(mode="cdf", thr=thr, sta=tuple(w.sta), cut=cut)
            out[cut] = A.build_mask(qbar, kbar, geom, prm)
        torch.cuda.synchronize()
        assert torch.equal(out["radix"][0], out["bitonic"][0])
        assert torch.equal(out["radix"][1], out["bitonic"][1])
        c = out["radix"][1]
        L1, L2 = out["radix"][2], out["bitonic"][2]
        ar = torch.arange(geom.nb, device=DEV)
        valid = ar[None, None, None, :] < c[..., None]
        assert torch.equal(torch.where(valid, L1, 0), torch.where(valid, L2, 0))


def test_cut_algorithms_agree_small(A):
    for geo, thr in [((1, 2, 3, 24, 88), 0.7), ((1, 1, 1, 8, 8), 0.5), ((1, 1, 6, 80, 80), 0.95),
                     ((1, 2, 2, 16, 16), 1e-9), ((1, 1, 5, 16, 24), 0.999999)]:
        B, H, T, Hs, Ws = geo
        geom, og = PT.geoms(B, H, T, Hs, Ws, 128)
        q, k, _ = make_random_qkv(B, H, T, Hs, Ws, 128, "bf16", seed=11, device=DEV)
        _, qbar = A.reorder(q, geom, want_pooled=True)
        _, kbar = A.reorder((k.float() + q.float()).to(q.dtype), geom, want_pooled=True)
        res = [A.build_mask(qbar, kbar, geom, A.MaskParams(mode="cdf", thr=thr, sta=(0, 0, 0), cut=c))
               for c in ("radix", "bitonic")]
        torch.cuda.synchronize()
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1]), geo


# ---------------------------------------------------------------- one mask at two workgroup sizes
def _masks_equal(a, b, nb):
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    valid = torch.arange(nb, device=DEV)[None, None, None, :] < a[1][..., None]
    assert torch.equal(torch.where(valid, a[2], 0), torch.where(valid, b[2], 0))


@pytest.mark.parametrize("name", ["480p", "480p-dyn", "480p-static", "720p"])
def test_select_widths_agree(A, name):
    """The row selection on its default width (one wave per row at 480p, two at 720p) and on four
    waves per row ('radix-wide') gives the same bits, counts and lists in every mode: a race in
    the row's LDS steps would show as a difference between the two partitions."""
    import dataclasses
    w = WORKLOADS[name]
    geom, og = PT.geoms(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    q, k, _ = make_qkv(w, device=DEV)
    _, qbar = A.reorder(q, geom, want_pooled=True)
    _, kbar = A.reorder(k, geom, want_pooled=True)
    base = A.MaskParams(mode=w.mode, thr=w.thr, tau=w.tau, sta=tuple(w.sta), gamma=w.gamma, lam=w.lam)
    res = [A.build_mask(qbar, kbar, geom, dataclasses.replace(base, cut=c)) for c in ("radix", "radix-wide")]
    torch.cuda.synchronize()
    _masks_equal(res[0], res[1], geom.nb)


def test_select_widths_agree_small(A):
    """Rows of at most 256 blocks (64 threads by default) against four waves, in the three modes."""
    for geo in [(1, 2, 3, 24, 88), (1, 1, 1, 8, 8), (1, 2, 2, 16, 16), (1, 1, 5, 16, 24)]:
        B, H, T, Hs, Ws = geo
        geom, og = PT.geoms(B, H, T, Hs, Ws, 128)
        q, k, _ = make_random_qkv(B, H, T, Hs, Ws, 128, "bf16", seed=12, device=DEV)
        _, qbar = A.reorder(q, geom, want_pooled=True)
        _, kbar = A.reorder((k.float() + q.float()).to(q.dtype), geom, want_pooled=True)
        for prm in (dict(mode="cdf", thr=0.7), dict(mode="dyn", tau=2.0), dict(mode="static", gamma=0.5, lam=0.05)):
            res = [A.build_mask(qbar, kbar, geom, A.MaskParams(sta=(3, 3, 3), cut=c, **prm))
                   for c in ("radix", "radix-wide")]
            torch.cuda.synchronize()
            _masks_equal(res[0], res[1], geom.nb)


# ---------------------------------------------------------------- more rows than one launch holds
@pytest.mark.parametrize("prm", [dict(mode="cdf", thr=0.5, cut="radix"), dict(mode="cdf", thr=0.5, cut="radix-wide"),
                                 dict(mode="dyn", tau=0.25)])
def test_mask_launches_split_over_many_rows(A, prm):
    """2^22 + 5 heads of two blocks: the score tiles and the mask rows run in several launches of
    at most 2^22 workgroups. Block 0 has pooled key +e0 and block 1 -e0, and each query row is
    +-2 e0 with a sign pattern over the rows, so its pooled logits are +-0.25 and -+0.25 and it
    keeps exactly its larger block (CDF thr 0.5: that block holds 62% of the mass; DYN: the other
    is 0.5 below the maximum). Outputs are pre-filled so an unwritten row shows."""
    H = (1 << 22) + 5
    geom = A.Geometry(B=1, H=H, T=2, Hs=8, Ws=8, d=64)
    assert geom.nb == 2
    row = torch.arange(H * 2, device=DEV).view(1, H, 2)
    sign = torch.where(row % 3 == 0, 1.0, -1.0).to(torch.float64)
    qbar = torch.zeros(1, H, 2, 64, dtype=torch.float64, device=DEV)
    qbar[..., 0] = 2.0 * sign
    kbar = torch.zeros_like(qbar)
    kbar[:, :, 0, 0] = 1.0
    kbar[:, :, 1, 0] = -1.0
    words = torch.full((1, H, 2, 1), -1, dtype=torch.int32, device=DEV)
    counts = torch.full((1, H, 2), -1, dtype=torch.int32, device=DEV)
    lists = torch.full((1, H, 2, 2), -1, dtype=torch.int32, device=DEV)
    A.build_mask(qbar, kbar, geom, A.MaskParams(sta=(0, 0, 0), **prm), words=words, counts=counts, lists=lists)
    torch.cuda.synchronize()
    kept = torch.where(sign > 0, 0, 1).to(torch.int32)
    assert bool((counts == 1).all())
    assert torch.equal(words[..., 0], torch.bitwise_left_shift(torch.ones_like(kept), kept))
    assert torch.equal(lists[..., 0], kept)


def _head_pattern(H, dtype):
    """x[0, h, n, c] = ((3n + 5c) mod 23) - 11 + (h mod 7): small integers, exact in bf16, built
    without a full-size integer temporary. Returns (x, pattern[64, 64], offsets[H])."""
    n = torch.arange(64, device=DEV)
    pat = ((3 * n[:, None] + 5 * n[None, :]) % 23 - 11).to(dtype)
    off = (torch.arange(H, device=DEV) % 7).to(dtype)
    x = torch.empty(1, H, 64, 64, dtype=dtype, device=DEV)
    torch.add(pat[None, None], off[None, :, None, None], out=x)
    return x, pat, off


def test_first_step_launches_split_over_many_blocks(A):
    """1,398,110 heads of one 8x8 patch in one frame (3*B*H*nb just above 2^22 workgroups, so the
    first step runs in two launches). With one block per head the fractal order is the original
    order: the V block must be the head's tile transposed (channel-major) and the pooled means the
    column means, exactly."""
    H = 1_398_110
    geom = A.Geometry(B=1, H=H, T=1, Hs=8, Ws=8, d=64)
    assert 3 * H * geom.nb > (1 << 22)
    q, pat, off = _head_pattern(H, torch.bfloat16)
    k = q.neg()
    qbar = torch.full((1, H, 1, 64), math.nan, dtype=torch.float64, device=DEV)
    kbar = torch.full_like(qbar, math.nan)
    v_rt = torch.zeros(1, H, 1, 64, 64, dtype=torch.bfloat16, device=DEV)
    A.pool_qk_reorder_v(q, k, q, geom, qbar=qbar, kbar=kbar, v_rt=v_rt)
    torch.cuda.synchronize()
    mean = pat.double().mean(dim=0)[None, :] + off.double()[:, None]  # [H, 64]
    assert torch.equal(qbar.view(H, 64), mean)
    assert torch.equal(kbar.view(H, 64), -mean)
    for h0 in range(0, H, 1 << 18):
        h1 = min(H, h0 + (1 << 18))
        assert torch.equal(v_rt[0, h0:h1, 0], q[0, h0:h1].transpose(1, 2))


def test_pooling_only_first_step_split_over_many_blocks(A):
    """The pooling-only form of the first step (v = v_rt = NULL) over 2^21 + 3 one-block heads:
    2*B*H*nb just above 2^22 workgroups, two launches; the means exactly."""
    H = (1 << 21) + 3
    geom = A.Geometry(B=1, H=H, T=1, Hs=8, Ws=8, d=64)
    assert 2 * H * geom.nb > (1 << 22)
    q, pat, off = _head_pattern(H, torch.bfloat16)
    k = q.neg()
    qbar = torch.full((1, H, 1, 64), math.nan, dtype=torch.float64, device=DEV)
    kbar = torch.full_like(qbar, math.nan)
    _, _, none = A.pool_qk_reorder_v(q, k, None, geom, qbar=qbar, kbar=kbar)
    torch.cuda.synchronize()
    mean = pat.double().mean(dim=0)[None, :] + off.double()[:, None]
    assert none is None
    assert torch.equal(qbar.view(H, 64), mean)
    assert torch.equal(kbar.view(H, 64), -mean)


def test_reorder_launches_split_over_many_blocks(A):
    """2^22 + 3 heads of one block: the reorder grid runs in two launches. Forward into the
    channel-major layout with pooling (the transposed tile and the column means), then the inverse
    of the token layout (the identity for one block per head)."""
    H = (1 << 22) + 3
    geom = A.Geometry(B=1, H=H, T=1, Hs=8, Ws=8, d=64)
    x, pat, off = _head_pattern(H, torch.bfloat16)
    y = torch.zeros(1, H, 1, 64, 64, dtype=torch.bfloat16, device=DEV)
    pooled = torch.full((1, H, 1, 64), math.nan, dtype=torch.float64, device=DEV)
    A.reorder(x, geom, layout="block_t", out=y, pooled=pooled)
    torch.cuda.synchronize()
    assert torch.equal(pooled.view(H, 64), pat.double().mean(dim=0)[None, :] + off.double()[:, None])
    for h0 in range(0, H, 1 << 19):
        h1 = min(H, h0 + (1 << 19))
        assert torch.equal(y[0, h0:h1, 0], x[0, h0:h1].transpose(1, 2))
    del pooled
    z = y.view(1, H, 64, 64)
    z.zero_()
    A.reorder(x, geom, inverse=True, out=z)
    torch.cuda.synchronize()
    for h0 in range(0, H, 1 << 19):
        h1 = min(H, h0 + (1 << 19))
        assert torch.equal(z[0, h0:h1], x[0, h0:h1])


# ---------------------------------------------------------------- the default V path
@pytest.mark.parametrize("over,short", [(dict(mode="dyn", tau=2.0), True), (dict(mode="cdf", thr=1.0), False)],
                         ids=["short-lists", "long-lists"])
def test_default_v_path_follows_the_mask(A, over, short):
    """fuse_v=None (bf16) picks the original-order V read when the first mask's mean kept count
    per row is at most FUSE_V_MAX_MEAN_COUNT, the channel-major V pass otherwise; either way the
    outputs equal both explicit paths bit for bit, on the first call and on the next. Inputs:
    the video recipe at 12 x 32 x 64 tokens (384 blocks), two heads."""
    w = WORKLOADS["480p"].with_(H=2, T=12, Hs=32, Ws=64, **over)
    geom, og = PT.geoms(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    q, k, v = make_qkv(w, device=DEV)
    p = A.MaskParams(mode=w.mode, thr=w.thr, tau=w.tau, sta=tuple(w.sta))
    auto = A.NablaAttention(geom, p, want_lse=True)
    fixed = {fv: A.NablaAttention(geom, p, want_lse=True, fuse_v=fv) for fv in (False, True)}
    for call in range(2):
        auto(q, k, v)
        for run in fixed.values():
            run(q, k, v)
        torch.cuda.synchronize()
        mean = float(auto.counts.sum()) / (w.B * w.H * geom.nb)
        assert (mean <= A.FUSE_V_MAX_MEAN_COUNT) == short, mean
        assert auto.fuse_v == short and (auto.v_rt is None) == short
        for run in fixed.values():
            assert torch.equal(auto.out, run.out) and torch.equal(auto.lse, run.lse), call
