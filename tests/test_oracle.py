"""Pins for the CPU oracle: each checks it against something other than itself.

Kinds of pin used here: brute force written from 3D token coordinates in the
original order (no fractal permutation involved), exhaustive subset search,
closed forms, library routines (torch scaled_dot_product_attention, scipy
softmax) and the hand-worked examples in tests/golden/. The mutation test at
the bottom plants plausible mistakes in the oracle and checks that some pin
fails for each one.
"""
import dataclasses
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from oracle import nabla_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _coords(g):
    t, y, x = np.meshgrid(np.arange(g.T), np.arange(g.Hs), np.arange(g.Ws), indexing="ij")
    return t.reshape(-1), y.reshape(-1), x.reshape(-1)


def _attention_original_order(Q, K, V, allowed, scale):
    """Brute force in the original token order, one query at a time."""
    N = Q.shape[0]
    O = np.zeros_like(V)
    for n in range(N):
        a = allowed(n)
        if not a.any():
            continue
        s = scale * (K[a] @ Q[n])
        w = np.exp(s - s.max())
        O[n] = (w / w.sum()) @ V[a]
    return O


# ---------------------------------------------------------------- P1
def test_p1_full_threshold_is_full_attention():
    """thr = 1 keeps every block, so the path must equal plain softmax(QK^T/sqrt(d))V."""
    g = R.Geom(B=1, H=2, T=3, Hs=16, Ws=24, d=16)
    Q, K, V = (_rand((g.B, g.H, g.N, g.d), s) for s in (1, 2, 3))
    for sta in [(0, 0, 0), (3, 3, 3)]:
        res = R.nabla_attention(Q, K, V, g, R.MaskParams(mode="cdf", thr=1.0, sta=sta))
        assert res.mask.mask.all()
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V)).numpy()
        np.testing.assert_allclose(res.O, ref, rtol=1e-12, atol=1e-12)
        # LSE against the library log-sum-exp of the full score rows (fractal order).
        Qr, Kr = R.reorder(Q, g), R.reorder(K, g)
        lse = scipy.special.logsumexp(Qr @ np.swapaxes(Kr, -1, -2) / math.sqrt(g.d), axis=-1)
        np.testing.assert_allclose(res.lse_r, lse, rtol=1e-12)


# ---------------------------------------------------------------- P2
@pytest.mark.parametrize("window", [(3, 3, 3), (1, 3, 5), (3, 1, 1), (5, 5, 5)])
def test_p2_pure_sta_equals_bruteforce_window(window):
    """thr = 0 leaves only STA: token (t,y,x) sees (t',y',x') iff every patch offset is within the window."""
    g = R.Geom(B=1, H=1, T=4, Hs=16, Ws=24, d=8)
    Q, K, V = (_rand((g.N, g.d), s) for s in (4, 5, 6))
    res = R.nabla_attention(Q[None, None], K[None, None], V[None, None], g,
                            R.MaskParams(mode="cdf", thr=0.0, sta=window))
    t, y, x = _coords(g)
    r = [(w - 1) // 2 for w in window]

    def allowed(n):
        return ((np.abs(t - t[n]) <= r[0]) & (np.abs(y // g.P - y[n] // g.P) <= r[1])
                & (np.abs(x // g.P - x[n] // g.P) <= r[2]))

    ref = _attention_original_order(Q, K, V, allowed, 1 / math.sqrt(g.d))
    np.testing.assert_allclose(res.O[0, 0], ref, rtol=1e-11, atol=1e-12)


def test_p2_random_block_mask_bruteforce():
    """An arbitrary (asymmetric) block mask, expanded by coordinates in the original order."""
    g = R.Geom(B=1, H=1, T=3, Hs=16, Ws=16, d=8)
    Q, K, V = (_rand((g.N, g.d), s) for s in (7, 8, 9))
    rng = np.random.default_rng(10)
    M = rng.random((g.nb, g.nb)) < 0.35
    M[3] = False  # one empty row
    t, y, x = _coords(g)
    blk = (t * g.nbh + y // g.P) * g.nbw + x // g.P  # block numbering convention (frame, patch row, patch col)
    ref = _attention_original_order(Q, K, V, lambda n: M[blk[n], blk], 1 / math.sqrt(g.d))
    Qr, Kr, Vr = (R.reorder(a, g) for a in (Q, K, V))
    Or, lse = R.masked_attention_head(Qr, Kr, Vr, M, g, 1 / math.sqrt(g.d))
    np.testing.assert_allclose(R.inverse_reorder(Or, g), ref, rtol=1e-11, atol=1e-12)
    assert np.isneginf(lse[3 * g.bs:4 * g.bs]).all() and np.isfinite(np.delete(lse, np.s_[3 * g.bs:4 * g.bs])).all()


# ---------------------------------------------------------------- P3
def _min_prefix_bruteforce(p_frac, thr_frac):
    """Smallest subset size whose exact mass reaches thr, and all subsets of that size that do."""
    n = len(p_frac)
    for size in range(n + 1):
        hits = [set(c) for c in itertools.combinations(range(n), size) if sum(p_frac[i] for i in c) >= thr_frac]
        if hits:
            return size, hits
    return None, []


@pytest.mark.parametrize("seed", range(40))
def test_p3_minimal_prefix_bruteforce(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    ints = rng.integers(1, 50, size=n)
    if seed % 3 == 0 and n > 2:
        ints[rng.integers(n)] = ints[0]  # force ties
    tot = int(ints.sum())
    p_frac = [Fraction(int(v), tot) for v in ints]
    p = np.array([float(f) for f in p_frac])
    for thr_num in range(1, 2 * tot, 3):
        thr_frac = Fraction(2 * thr_num + 1, 4 * tot)  # never equal to a subset mass
        if thr_frac >= 1:
            break
        keep, _ = R.cdf_select_row(p, float(thr_frac))
        size, hits = _min_prefix_bruteforce(p_frac, thr_frac)
        kept = set(np.nonzero(keep)[0].tolist())
        assert len(kept) == size and kept in hits
        # Among equal probabilities, lower indices are kept first.
        for i, j in itertools.combinations(range(n), 2):
            if p_frac[i] == p_frac[j] and j in kept:
                assert i in kept
        if kept and len(kept) < n:
            assert min(p[list(kept)]) >= max(np.delete(p, list(kept)))


def test_p3_invariants_on_generated_rows():
    from gen import WORKLOADS, make_qkv
    w = WORKLOADS["tiny"]
    g = R.Geom(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    Q, K, V = make_qkv(w)
    Qr, Kr = R.reorder(R.to64(Q), g), R.reorder(R.to64(K), g)
    res = R.build_block_mask(R.block_means(Qr, g), R.block_means(Kr, g), g,
                             R.MaskParams(mode="cdf", thr=w.thr, sta=(0, 0, 0)))
    for idx in np.ndindex(res.sel.shape[:-1]):
        p, k = res.Pm[idx], res.sel[idx]
        assert p[k].sum() >= w.thr
        assert p[k].sum() - p[k].min() < w.thr
        if (~k).any():
            assert p[k].min() >= p[~k].max()


# ---------------------------------------------------------------- P4
@pytest.mark.parametrize("T,Hs,Ws,thr,expect", [(21, 32, 56, 0.7, 412), (5, 24, 24, 0.5, 23), (1, 8, 8, 0.3, 1)])
def test_p4_uniform_rows_keep_lowest_indices(T, Hs, Ws, thr, expect):
    """All pooled keys equal -> P = 1/nb -> exactly ceil(thr*nb) blocks, the lowest indices."""
    g = R.Geom(B=1, H=1, T=T, Hs=Hs, Ws=Ws, d=4)
    assert math.ceil(thr * g.nb) == expect
    Q = _rand((1, 1, g.N, g.d), 11)
    K = np.ones((1, 1, g.N, g.d)) * 0.5
    res = R.build_block_mask(R.block_means(R.reorder(Q, g), g), R.block_means(R.reorder(K, g), g), g,
                             R.MaskParams(mode="cdf", thr=thr, sta=(0, 0, 0)))
    expected = np.zeros(g.nb, dtype=bool)
    expected[:expect] = True
    assert (res.mask[0, 0] == expected[None, :]).all()


def test_dominant_block_row_softmax():
    """One pooled key dominates every row -> only that block survives a modest threshold.

    Rows, not columns, are normalised: with every row dominated by block 0, a
    column-wise softmax would spread block 0's mass over all rows.
    """
    g = R.Geom(B=1, H=1, T=2, Hs=16, Ws=16, d=4)
    qbar = np.ones((1, 1, g.nb, g.d))
    kbar = np.zeros((1, 1, g.nb, g.d))
    kbar[0, 0, 0] = 10.0
    res = R.build_block_mask(qbar, kbar, g, R.MaskParams(mode="cdf", thr=0.9, sta=(0, 0, 0)))
    S = 0.5 * qbar[0, 0] @ kbar[0, 0].T
    np.testing.assert_allclose(res.Pm[0, 0], scipy.special.softmax(S, axis=-1), rtol=1e-13)
    assert res.Pm[0, 0, 0, 0] > 0.9
    assert (res.mask[0, 0, :, 0]).all() and res.mask[0, 0].sum() == g.nb


def test_identical_pooled_keys_tie_exactly():
    """Blocks with equal pooled keys have equal probabilities (then the lower index ranks first)."""
    rng = np.random.default_rng(21)
    nb, d = 700, 128
    kbar = rng.standard_normal((nb, d))
    dup_src = rng.choice(nb, 40, replace=False)
    dup_dst = rng.choice(np.setdiff1d(np.arange(nb), dup_src), 40, replace=False)
    kbar[dup_dst] = kbar[dup_src]
    qbar = rng.standard_normal((nb, d))
    S = R.pooled_logits(qbar[None], kbar[None], 0.1)[0]
    assert np.array_equal(S[:, dup_dst], S[:, dup_src])
    np.testing.assert_allclose(S, 0.1 * qbar @ kbar.T, rtol=1e-12, atol=1e-12)
    g = R.Geom(B=1, H=1, T=7, Hs=80, Ws=80, d=d)
    assert g.nb == nb
    res = R.build_block_mask(qbar[None, None], kbar[None, None], g, R.MaskParams(mode="cdf", thr=0.5, sta=(0, 0, 0)))
    for a, b in zip(dup_src, dup_dst):
        lo, hi = min(a, b), max(a, b)
        assert res.Pm[0, 0, :, a].tolist() == res.Pm[0, 0, :, b].tolist()
        assert not (res.sel[0, 0, :, hi] & ~res.sel[0, 0, :, lo]).any()


# ---------------------------------------------------------------- P5
def test_p5_nesting_and_limits():
    from gen import WORKLOADS, make_qkv
    w = WORKLOADS["tiny"]
    g = R.Geom(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    Q, K, _ = make_qkv(w)
    qbar = R.block_means(R.reorder(R.to64(Q), g), g)
    kbar = R.block_means(R.reorder(R.to64(K), g), g)
    prev = None
    for thr in [0.0, 0.1, 0.3, 0.5, 0.8, 0.95, 0.999, 1.0]:
        m = R.build_block_mask(qbar, kbar, g, R.MaskParams(mode="cdf", thr=thr, sta=(0, 0, 0))).mask
        if prev is not None:
            assert (prev <= m).all()
        prev = m
    assert prev.all()
    prev = None
    for tau in [0.0, 0.5, 1.0, 2.0, 4.0, 8.0, 1e9]:
        res = R.build_block_mask(qbar, kbar, g, R.MaskParams(mode="dyn", tau=tau, sta=(0, 0, 0)))
        if prev is not None:
            assert (prev <= res.mask).all()
        if tau == 0.0:
            assert (res.mask == (res.S == res.S.max(axis=-1, keepdims=True))).all()
        prev = res.mask
    assert prev.all()


# ---------------------------------------------------------------- P6
def test_p6_reorder_is_blockwise_bijection():
    g = R.Geom(B=2, H=3, T=3, Hs=16, Ws=24, d=5)
    X = _rand((g.B, g.H, g.N, g.d), 12)
    Xr = R.reorder(X, g)
    assert np.array_equal(R.inverse_reorder(Xr, g), X)
    pos = R.fractal_positions(g)
    assert np.array_equal(np.sort(pos), np.arange(g.N))
    # Block i of the reordered sequence holds exactly the tokens of patch coords(i).
    t, y, x = _coords(g)
    c = R.block_coords(g)
    for i in range(g.nb):
        members = np.nonzero(pos // g.bs == i)[0]
        want = np.nonzero((t == c[i, 0]) & (y // g.P == c[i, 1]) & (x // g.P == c[i, 2]))[0]
        assert np.array_equal(np.sort(members), want)
    # Time order is kept: every token of frame t comes before every token of frame t+1.
    assert (np.diff(pos[np.argsort(pos)] // (g.N // g.T)) >= 0).all()
    assert (pos // (g.N // g.T) == t).all()
    # Pooled means: sum over blocks times block size equals the sum over tokens.
    qbar = R.block_means(Xr, g)
    np.testing.assert_allclose(qbar.sum(axis=-2) * g.bs, X.sum(axis=-2), rtol=1e-12)
    np.testing.assert_allclose(qbar[0, 0, 2], X[0, 0][(t == c[2, 0]) & (y // g.P == c[2, 1]) & (x // g.P == c[2, 2])].mean(0))


# ---------------------------------------------------------------- P7
def test_p7_attention_identities():
    g = R.Geom(B=1, H=1, T=2, Hs=16, Ws=16, d=8)
    rng = np.random.default_rng(13)
    M = rng.random((g.nb, g.nb)) < 0.3
    M[np.arange(g.nb), np.arange(g.nb)] = True
    Qr, Kr = _rand((g.N, g.d), 14), _rand((g.N, g.d), 15)
    Vc = np.full((g.N, g.d), 0.75)
    O, _ = R.masked_attention_head(Qr, Kr, Vc, M, g, 0.3)
    np.testing.assert_allclose(O, 0.75, rtol=1e-13)
    Vr = _rand((g.N, g.d), 16)
    O, _ = R.masked_attention_head(np.zeros_like(Qr), Kr, Vr, M, g, 0.3)
    allowed = R.expand_to_tokens(M, g)
    mean = (allowed @ Vr) / allowed.sum(1, keepdims=True)
    np.testing.assert_allclose(O, mean, rtol=1e-11, atol=1e-13)
    onehot = np.eye(g.N)[:, : g.N]
    O, _ = R.masked_attention_head(Qr, Kr, onehot, M, g, 0.3)
    np.testing.assert_allclose(O.sum(1), 1.0, rtol=1e-12)
    assert (O[~allowed] == 0).all()


# ---------------------------------------------------------------- P9
def test_p9_dyn_vs_probability_ratio():
    from gen import WORKLOADS, make_qkv
    w = WORKLOADS["tiny"]
    g = R.Geom(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    Q, K, _ = make_qkv(w)
    qbar = R.block_means(R.reorder(R.to64(Q), g), g)
    kbar = R.block_means(R.reorder(R.to64(K), g), g)
    for tau in [0.05, 0.2, 1.0]:
        res = R.build_block_mask(qbar, kbar, g, R.MaskParams(mode="dyn", tau=tau, sta=(0, 0, 0)))
        ratio = res.Pm / res.Pm.max(axis=-1, keepdims=True)
        assert (ratio[res.mask] >= math.exp(-tau) * (1 - 1e-12)).all()
        assert (ratio[~res.mask] < math.exp(-tau) * (1 + 1e-12)).all()


# ---------------------------------------------------------------- golden rows and packing
def test_golden_cdf_rows():
    with open(os.path.join(GOLDEN, "cdf_examples.json")) as f:
        rows = json.load(f)["rows"]
    for r in rows:
        p = np.array(r["p"])
        keep, _ = R.cdf_select_row(p, r["thr"])
        assert np.nonzero(keep)[0].tolist() == r["kept"], r
        if 0 < r["thr"] < 1:
            # The page's literal wording: ascending order, cumulative probability > 1 - thr.
            asc = np.lexsort((-np.arange(len(p)), p))
            cum = np.cumsum(p[asc])
            lit = np.zeros(len(p), bool)
            lit[asc] = cum > 1 - r["thr"] + 1e-12
            assert np.nonzero(lit)[0].tolist() == r["kept"], r


def test_pack_bits_layout():
    m = np.zeros((2, 70), dtype=bool)
    m[0, [0, 5, 31, 32, 69]] = True
    m[1, 33] = True
    w = R.pack_bits(m)
    assert w.shape == (2, 3) and w.dtype == np.uint32
    assert w[0].tolist() == [1 | 32 | (1 << 31), 1, 1 << 5]
    assert w[1].tolist() == [0, 2, 0]
    assert np.array_equal(R.unpack_bits(w, 70), m)
    counts, lists = R.kept_lists(m)
    assert counts.tolist() == [5, 1]
    assert lists[0, :5].tolist() == [0, 5, 31, 32, 69] and (lists[0, 5:] == -1).all()


def test_sta_counts_closed_form():
    """Blocks kept by STA alone: product over axes of the truncated window lengths."""
    g = R.Geom(B=1, H=1, T=21, Hs=32, Ws=56, d=4)
    sta = R.sta_block_mask(g, (3, 3, 3))
    c = R.block_coords(g)

    def span(v, n):
        return min(v + 1, n - 1) - max(v - 1, 0) + 1

    want = np.array([span(a, g.T) * span(b, g.nbh) * span(e, g.nbw) for a, b, e in c])
    assert np.array_equal(sta.sum(1), want)
    assert abs(sta.mean() - 0.0335) < 5e-4
    assert (sta == sta.T).all() and sta.diagonal().all()


# ---------------------------------------------------------------- backward (gradients)
def _bwd_case(seed=0):
    g = R.Geom(1, 1, 2, 16, 16, 8, 8)
    rng = np.random.default_rng(seed)
    Q, K, V, G = (rng.standard_normal((g.N, g.d)) for _ in range(4))
    M = rng.random((g.nb, g.nb)) < 0.5
    M[0] = False  # an empty row
    M[1] = True   # a full row
    return g, Q, K, V, G, M, 1.0 / math.sqrt(g.d)


def test_p10_backward_finite_differences():
    """Central differences of L = sum(O * G) match the closed-form gradients (dO = G)."""
    g, Q, K, V, G, M, sc = _bwd_case()
    dQ, dK, dV = R.masked_attention_backward_head(Q, K, V, G, M, g, sc)
    rng = np.random.default_rng(1)

    def loss(Qx, Kx, Vx):
        O, _ = _ORIG['masked_attention_head'](Qx, Kx, Vx, M, g, sc)
        return float(np.sum(O * G))

    h = 1e-6
    for which, grad in ((0, dQ), (1, dK), (2, dV)):
        for _ in range(8):
            i, c = int(rng.integers(g.N)), int(rng.integers(g.d))
            args_p, args_m = [Q.copy(), K.copy(), V.copy()], [Q.copy(), K.copy(), V.copy()]
            args_p[which][i, c] += h
            args_m[which][i, c] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[i, c]) < 1e-6 * max(1.0, abs(fd)), (which, i, c, fd, grad[i, c])


def test_p11_backward_full_mask_matches_autograd():
    """With every block allowed the gradients are those of dense softmax attention (torch autograd, float64)."""
    g, Q, K, V, G, _, sc = _bwd_case(2)
    M = np.ones((g.nb, g.nb), dtype=bool)
    dQ, dK, dV = R.masked_attention_backward_head(Q, K, V, G, M, g, sc)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    o = torch.softmax(sc * q @ k.T, dim=-1) @ v
    (o * torch.tensor(G)).sum().backward()
    np.testing.assert_allclose(dQ, q.grad.numpy(), atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(dK, k.grad.numpy(), atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(dV, v.grad.numpy(), atol=1e-12, rtol=1e-10)


def test_p12_backward_invariants():
    """Sum over keys of dK is zero (each row of dS sums to zero); sum over keys of dV equals the
    sum of dO over rows that see any key (each live row of P sums to one); rows with nothing
    allowed get dQ = 0."""
    g, Q, K, V, G, M, sc = _bwd_case(3)
    dQ, dK, dV = R.masked_attention_backward_head(Q, K, V, G, M, g, sc)
    live = M.any(axis=1)[np.arange(g.N) // g.bs]
    assert np.abs(dK.sum(axis=0)).max() < 1e-12
    np.testing.assert_allclose(dV.sum(axis=0), G[live].sum(axis=0), atol=1e-12)
    assert not live[:g.bs].any() and np.all(dQ[:g.bs] == 0)
    assert np.abs(dQ[live]).max() > 0


def test_p13_backward_row_subsets():
    """Restricted to a set of query rows, dQ equals the full result on those rows, and dK / dV
    equal it on every key block whose column (the query blocks keeping it) lies inside the set."""
    g, Q, K, V, G, M, sc = _bwd_case(4)
    dQ, dK, dV = R.masked_attention_backward_head(Q, K, V, G, M, g, sc)
    j = 2
    qblocks = np.nonzero(M[:, j])[0]
    rows = np.concatenate([np.arange(b * g.bs, (b + 1) * g.bs) for b in qblocks])
    sQ, sK, sV = R.masked_attention_backward_head(Q, K, V, G, M, g, sc, rows=rows, chunk=48)
    np.testing.assert_allclose(sQ, dQ[rows], atol=1e-13)
    kr = slice(j * g.bs, (j + 1) * g.bs)
    np.testing.assert_allclose(sK[kr], dK[kr], atol=1e-13)
    np.testing.assert_allclose(sV[kr], dV[kr], atol=1e-13)
    # Leaving out one query block that keeps j changes block j's gradients.
    tQ, tK, tV = R.masked_attention_backward_head(Q, K, V, G, M, g, sc, rows=rows[g.bs:])
    assert np.abs(tV[kr] - dV[kr]).max() > 1e-6


def test_p14_backward_given_output():
    """Handing the backward the exact O changes nothing; a perturbed O' moves only D:
    dV is unchanged and dQ changes by -scale * <dO_i, O'_i - O_i> (P K)_i."""
    g, Q, K, V, G, M, sc = _bwd_case(5)
    dQ, dK, dV = R.masked_attention_backward_head(Q, K, V, G, M, g, sc)
    O, _ = _ORIG['masked_attention_head'](Q, K, V, M, g, sc)
    eQ, eK, eV = R.masked_attention_backward_head(Q, K, V, G, M, g, sc, O=O)
    for a, b in ((eQ, dQ), (eK, dK), (eV, dV)):
        np.testing.assert_allclose(a, b, atol=1e-13)
    delta = 1e-3 * np.random.default_rng(6).standard_normal(O.shape)
    pQ, pK, pV = R.masked_attention_backward_head(Q, K, V, G, M, g, sc, O=O + delta)
    np.testing.assert_allclose(pV, dV, atol=1e-13)
    key_block = np.arange(g.N) // g.bs
    allowed = M[key_block[:, None], key_block[None, :]]
    S = np.where(allowed, sc * Q @ K.T, -np.inf)
    P = np.zeros_like(S)
    live = allowed.any(axis=1)
    E = np.exp(S[live] - S[live].max(axis=1, keepdims=True))
    P[live] = E / E.sum(axis=1, keepdims=True)
    dD = np.sum(G * delta, axis=1)
    np.testing.assert_allclose(pQ - dQ, -sc * dD[:, None] * (P @ K), atol=1e-12)
    assert np.abs(pK - dK).max() > 1e-6


# ---------------------------------------------------------------- Static-Ratio mode
def test_p15_static_counts_hand_values():
    """k(dt) written out by hand for 28 blocks per frame (4 x 7), gamma 1/2, lambda 0.05:
    28, 28/2 = 14, 28/4 = 7, ceil(28/8 = 3.5) = 4, ceil(1.75) = 2, then the floor
    ceil(28 * 0.05 = 1.4) = 2; and the limits gamma = 1 (all), gamma = lambda = 0 (own frame)."""
    g = R.Geom(1, 1, 8, 32, 56, 64, 8)
    assert R.static_ratio_counts(g, 0.5, 0.05).tolist() == [28, 14, 7, 4, 2, 2, 2, 2]
    assert R.static_ratio_counts(g, 0.5, 0.0).tolist() == [28, 14, 7, 4, 2, 1, 1, 1]
    assert R.static_ratio_counts(g, 1.0, 0.0).tolist() == [28] * 8
    assert R.static_ratio_counts(g, 0.0, 0.0).tolist() == [28] + [0] * 7
    assert R.static_ratio_counts(g, 0.0, 1.0).tolist() == [28] * 8


def _nearest_bruteforce(g, i, frame, k):
    """The k positions of `frame` nearest to block i's position, by explicit pairwise comparison."""
    ti, rem = divmod(i, g.nbh * g.nbw)
    hi, wi = divmod(rem, g.nbw)
    cand = []
    for p in range(g.nbh * g.nbw):
        hp, wp = divmod(p, g.nbw)
        cand.append(((hp - hi) * (hp - hi) + (wp - wi) * (wp - wi), p))
    chosen = []
    for _ in range(k):  # selection by repeated minimum
        best = min(c for c in cand if c not in chosen)
        chosen.append(best)
    return {frame * g.nbh * g.nbw + p for _, p in chosen}


def test_p16_static_mask_bruteforce():
    """Every row keeps, in every key frame, exactly the k(|dt|) nearest positions."""
    g = R.Geom(1, 1, 5, 40, 24, 64, 8)  # 5 x 3 blocks per frame, 5 frames
    for gamma, lam in ((0.5, 0.1), (0.7, 0.0), (0.3, 0.3)):
        m = R.static_ratio_block_mask(g, gamma, lam)
        k = R.static_ratio_counts(g, gamma, lam)
        F = g.nbh * g.nbw
        for i in range(g.nb):
            for f in range(g.T):
                want = _nearest_bruteforce(g, i, f, int(k[abs(i // F - f)]))
                got = {j for j in range(f * F, (f + 1) * F) if m[i, j]}
                assert got == want, (gamma, lam, i, f)


def test_p17_static_special_cases():
    """gamma = 1 keeps everything; gamma = lambda = 0 keeps exactly the own frame; the mode
    ignores the pooled vectors and ORs the STA window."""
    g = R.Geom(1, 2, 4, 16, 24, 64, 8)
    assert R.static_ratio_block_mask(g, 1.0, 0.0).all()
    own = R.block_coords(g)[:, 0]
    assert np.array_equal(R.static_ratio_block_mask(g, 0.0, 0.0), own[:, None] == own[None, :])
    rng = np.random.default_rng(0)
    a = R.build_block_mask(rng.standard_normal((1, 2, g.nb, 64)), rng.standard_normal((1, 2, g.nb, 64)), g,
                           R.MaskParams(mode="static", gamma=0.4, lam=0.0, sta=(3, 3, 3)))
    b = R.build_block_mask(np.zeros((1, 2, g.nb, 64)), np.ones((1, 2, g.nb, 64)), g,
                           R.MaskParams(mode="static", gamma=0.4, lam=0.0, sta=(3, 3, 3)))
    assert np.array_equal(a.mask, b.mask)
    expect = R.static_ratio_block_mask(g, 0.4, 0.0) | R.sta_block_mask(g, (3, 3, 3))
    assert np.array_equal(a.mask[0, 1], expect)


# ---------------------------------------------------------------- kept blocks only
def test_gathered_attention_equals_masked_rows():
    """masked_attention_blocks (only the kept key blocks' tokens) equals the dense masked rows of
    masked_attention_head, on random masks with an empty row, a full row and single blocks."""
    g = R.Geom(B=1, H=1, T=3, Hs=16, Ws=24, d=16)
    Q, K, V = (_rand((g.N, g.d), s) for s in (21, 22, 23))
    rng = np.random.default_rng(5)
    m = rng.random((g.nb, g.nb)) < 0.3
    m[0] = False
    m[1] = True
    m[2] = False
    m[2, g.nb - 1] = True
    blocks = [0, 1, 2, 7, g.nb - 1, 4]
    O, lse = R.masked_attention_blocks(Q, K, V, m, g, 0.3, blocks)
    rows = np.concatenate([np.arange(b * g.bs, (b + 1) * g.bs) for b in blocks])
    O_ref, lse_ref = R.masked_attention_head(Q, K, V, m, g, 0.3, rows=rows)
    np.testing.assert_allclose(O, O_ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=1e-12, atol=1e-12)
    assert not O[: g.bs].any()


# ---------------------------------------------------------------- the parity band
# Mask comparison rule: a block whose decision sits within 1e-5 of its threshold may differ
# between two correct implementations (CDF: |C_excl - thr|; dynamic: |S - (max S - tau)|);
# sliding-tile blocks are always kept and never exempt. exemption_sets computes that set.
def _one_row(mode, thr_or_tau, p=None, s=None, sta=()):
    """MaskResult of one row ([1, 1, 1, n]) from given probabilities (CDF) or logits (dynamic),
    selected by the oracle's own row functions; sta lists the row's sliding-tile blocks."""
    n = len(p if p is not None else s)
    sta_row = np.zeros((1, n), dtype=bool)
    sta_row[0, list(sta)] = True
    if mode == "cdf":
        p = np.asarray(p, np.float64)
        sel, cex = R.cdf_select_row(p, thr_or_tau)
        res = R.MaskResult(S=np.log(p)[None, None, None], Pm=p[None, None, None], sel=sel[None, None, None],
                           sta=sta_row, mask=(sel | sta_row[0])[None, None, None], c_excl=cex[None, None, None])
        return res, R.MaskParams(mode="cdf", thr=thr_or_tau, sta=(1, 1, 1))
    s = np.asarray(s, np.float64)
    sel = R.dyn_select_row(s, thr_or_tau)
    e = np.exp(s - s.max())
    res = R.MaskResult(S=s[None, None, None], Pm=(e / e.sum())[None, None, None], sel=sel[None, None, None],
                       sta=sta_row, mask=(sel | sta_row[0])[None, None, None], c_excl=None)
    return res, R.MaskParams(mode="dyn", tau=thr_or_tau, sta=(1, 1, 1))


def test_band_golden_rows():
    """Hand-worked rows (tests/golden/band_examples.json): the exempt blocks and the kept set."""
    with open(os.path.join(GOLDEN, "band_examples.json")) as f:
        gold = json.load(f)
    band = gold["band"]
    for mode, key, par in (("cdf", "p", "thr"), ("dyn", "s", "tau")):
        for r in gold[mode]:
            kw = {key: r[key]}
            res, prm = _one_row(mode, r[par], sta=r["sta"], **kw)
            ex = R.exemption_sets(res, prm, band)[0, 0, 0]
            assert np.nonzero(ex)[0].tolist() == r["exempt"], r
            assert np.nonzero(res.mask[0, 0, 0])[0].tolist() == sorted(set(r["kept"]) | set(r["sta"])), r


def test_band_golden_rows_through_the_mask_builder():
    """The same rows through build_block_mask: d = 1, pool_scale 1, every pooled query 1 and
    pooled key j = log p_j (CDF) or s_j (dynamic), so row i's logits are the given row; one
    frame of n patches with a 1 x 1 x 1 window makes block i the only sliding-tile block of
    row i."""
    with open(os.path.join(GOLDEN, "band_examples.json")) as f:
        gold = json.load(f)
    for mode, key, par in (("cdf", "p", "thr"), ("dyn", "s", "tau")):
        for r in gold[mode]:
            if r["sta"]:  # rows with their own window list repeat a row without one
                continue
            vals = np.asarray(r[key], np.float64)
            n = len(vals)
            g = R.Geom(1, 1, 1, 8, 8 * n, 1, 8)
            kbar = (np.log(vals) if mode == "cdf" else vals).reshape(1, 1, n, 1)
            prm = R.MaskParams(mode=mode, thr=r[par] if mode == "cdf" else 0.9, tau=r[par] if mode == "dyn" else 4.0,
                               pool_scale=1.0, sta=(1, 1, 1))
            res = R.build_block_mask(np.ones((1, 1, n, 1)), kbar, g, prm)
            ex = R.exemption_sets(res, prm, gold["band"])
            for i in range(n):
                assert np.nonzero(ex[0, 0, i])[0].tolist() == [j for j in r["exempt"] if j != i], (r, i)
                assert np.nonzero(res.mask[0, 0, i])[0].tolist() == sorted(set(r["kept"]) | {i}), (r, i)


@pytest.mark.parametrize("seed", range(10))
def test_band_bruteforce_rows(seed):
    """Random rows with ties: C_excl summed in exact rationals straight from its definition (the
    mass of every block with a larger probability, or an equal one and a lower index), the
    thresholds placed inside, on and just outside the band around each block, and the exempt
    set compared with |C_excl - thr| <= 1e-5 minus the sliding-tile blocks. The dynamic mode the
    same way on the logits."""
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(2, 13))
    ints = rng.integers(1, 40, size=n)
    if seed % 2 and n > 2:
        ints[rng.integers(1, n)] = ints[0]
    tot = int(ints.sum())
    pf = [Fraction(int(v), tot) for v in ints]
    p = np.array([float(f) for f in pf])
    C = [sum((pf[k] for k in range(n) if pf[k] > pf[j] or (pf[k] == pf[j] and k < j)), Fraction(0))
         for j in range(n)]
    sta = [j for j in range(n) if rng.random() < 0.25]
    band = Fraction(1e-5)
    offsets = (0.0, 4e-6, -7e-6, 9.9e-6, -9.9e-6, 1.05e-5, -1.2e-5, 3e-5)
    for js in range(n):
        for off in offsets:
            thr = float(C[js]) + off
            if not 0.0 < thr < 1.0:
                continue
            res, prm = _one_row("cdf", thr, p=p, sta=sta)
            np.testing.assert_allclose(res.c_excl[0, 0, 0], [float(c) for c in C], rtol=0, atol=1e-15)
            want = [j for j in range(n) if abs(C[j] - Fraction(thr)) <= band and j not in sta]
            assert np.nonzero(R.exemption_sets(res, prm)[0, 0, 0])[0].tolist() == want, (js, off)
    s = np.round(rng.standard_normal(n) * 3, 3)
    for js in range(n):
        for off in offsets:
            tau = float(s.max() - s[js]) - off  # edge = s[js] + off
            if tau < 0:
                continue
            res, prm = _one_row("dyn", tau, s=s, sta=sta)
            edge = Fraction(float(s.max())) - Fraction(tau)
            want = [j for j in range(n) if abs(Fraction(float(s[j])) - edge) <= band and j not in sta]
            assert np.nonzero(R.exemption_sets(res, prm)[0, 0, 0])[0].tolist() == want, (js, off)


# ---------------------------------------------------------------- planted mistakes
PINS = [
    test_p1_full_threshold_is_full_attention,
    lambda: test_p2_pure_sta_equals_bruteforce_window((3, 3, 3)),
    lambda: test_p2_pure_sta_equals_bruteforce_window((1, 3, 5)),
    test_p2_random_block_mask_bruteforce,
    lambda: [test_p3_minimal_prefix_bruteforce(s) for s in (0, 1, 3, 6)],
    test_p3_invariants_on_generated_rows,
    lambda: test_p4_uniform_rows_keep_lowest_indices(21, 32, 56, 0.7, 412),
    test_dominant_block_row_softmax,
    test_p5_nesting_and_limits,
    test_p6_reorder_is_blockwise_bijection,
    test_p7_attention_identities,
    test_p9_dyn_vs_probability_ratio,
    test_golden_cdf_rows,
    test_pack_bits_layout,
    test_sta_counts_closed_form,
    test_p10_backward_finite_differences,
    test_p11_backward_full_mask_matches_autograd,
    test_p12_backward_invariants,
    test_p13_backward_row_subsets,
    test_p14_backward_given_output,
    test_p15_static_counts_hand_values,
    test_p16_static_mask_bruteforce,
    test_p17_static_special_cases,
    test_gathered_attention_equals_masked_rows,
    test_band_golden_rows,
    test_band_golden_rows_through_the_mask_builder,
    lambda: [test_band_bruteforce_rows(s) for s in (0, 1, 2)],
]


_ORIG = {n: getattr(R, n) for n in ("cdf_select_row", "sta_block_mask", "masked_attention_head", "reorder",
                                    "masked_attention_backward_head", "static_ratio_counts", "exemption_sets",
                                    "masked_attention_blocks")}


def _m_sort_ascending(p):
    return np.lexsort((np.arange(p.shape[-1]), p))


def _m_tie_high_first(p):
    return np.lexsort((-np.arange(p.shape[-1]), -p))


def _m_cdf_inclusive(p, thr):
    order = R.rank_order(p)
    c = np.empty(len(p))
    c[order] = np.cumsum(p[order])
    return (c < thr) | (thr >= 1), c


def _m_cdf_le(p, thr):
    keep, c = _ORIG['cdf_select_row'](p, thr)
    return (c <= thr) | (thr >= 1), c


def _m_positions_patch_transposed(g):
    t, y, x = np.meshgrid(np.arange(g.T), np.arange(g.Hs), np.arange(g.Ws), indexing="ij")
    block = (t * g.nbw + x // g.P) * g.nbh + y // g.P
    return (block * g.bs + (y % g.P) * g.P + x % g.P).reshape(-1)


def _m_positions_time_inner(g):
    t, y, x = np.meshgrid(np.arange(g.T), np.arange(g.Hs), np.arange(g.Ws), indexing="ij")
    block = ((y // g.P) * g.nbw + x // g.P) * g.T + t
    return (block * g.bs + (y % g.P) * g.P + x % g.P).reshape(-1)


def _m_sta_wide(g, window):
    return _ORIG['sta_block_mask'](g, tuple(w + 2 if w else 0 for w in window))


def _m_block_sums(Xr, g):
    Xr = np.asarray(Xr, np.float64)
    return Xr.reshape(Xr.shape[:-2] + (g.nb, g.bs, Xr.shape[-1])).sum(axis=-2)


def _m_softmax_cols(S):
    m = S.max(axis=-2, keepdims=True)
    e = np.exp(S - m)
    return e / e.sum(axis=-2, keepdims=True)


def _m_dyn_strict(s, tau):
    return s > s.max() - tau


def _m_dyn_from_min(s, tau):
    return s <= s.min() + tau


def _m_pack_msb(mask):
    nb = mask.shape[-1]
    out = np.zeros(mask.shape[:-1] + ((nb + 31) // 32,), dtype=np.uint64)
    for j in range(nb):
        out[..., j // 32] |= mask[..., j].astype(np.uint64) << np.uint64(31 - j % 32)
    return out.astype(np.uint32)


def _m_attn_transposed(Qr, Kr, Vr, block_mask, g, scale, rows=None, chunk=256):
    return _ORIG['masked_attention_head'](Qr, Kr, Vr, block_mask.T, g, scale, rows, chunk)


def _m_attn_no_scale(Qr, Kr, Vr, block_mask, g, scale, rows=None, chunk=256):
    return _ORIG['masked_attention_head'](Qr, Kr, Vr, block_mask, g, 1.0, rows, chunk)


def _m_inverse_as_forward(Xr, g):
    return _ORIG['reorder'](Xr, g)


def _bwd_flawed(flaw):
    """The backward of the oracle rewritten with one planted flaw."""
    def f(Qr, Kr, Vr, dOr, block_mask, g, scale, rows=None, O=None, chunk=256):
        bm = block_mask.T if flaw == "mask transposed" else block_mask
        key_block = np.arange(g.N) // g.bs
        r = np.arange(g.N) if rows is None else np.asarray(rows)
        dK, dV = np.zeros_like(Kr), np.zeros_like(Vr)
        allowed = bm[(r // g.bs)[:, None], key_block[None, :]]
        sc = np.where(allowed, scale * (Qr[r] @ Kr.T), -np.inf)
        mx = sc.max(axis=1)
        live = np.isfinite(mx)
        P = np.zeros_like(sc)
        e = np.exp(sc[live] - mx[live, None])
        P[live] = e / e.sum(axis=1, keepdims=True)
        dP = dOr[r] @ Vr.T
        Orow = P @ Vr if (O is None or flaw == "ignores O") else O[r]
        D = np.sum(dOr[r] * Orow, axis=1)
        dS = P * dP if flaw == "no D" else P * (dP - D[:, None])
        dQ = scale * (dS @ Kr)
        dK = (1.0 if flaw == "dK unscaled" else scale) * (dS.T @ Qr[r])
        dV = dS.T @ dOr[r] if flaw == "dV from dS" else P.T @ dOr[r]
        return dQ, dK, dV
    return f


def _m_static_chebyshev(g):
    F = g.nbh * g.nbw
    hp, wp = np.divmod(np.arange(F), g.nbw)
    rank = np.empty((F, F), dtype=np.int64)
    for p in range(F):
        d = np.maximum(np.abs(hp - hp[p]), np.abs(wp - wp[p]))
        rank[p, np.lexsort((np.arange(F), d))] = np.arange(F)
    return rank


def _m_static_tie_high(g):
    F = g.nbh * g.nbw
    hp, wp = np.divmod(np.arange(F), g.nbw)
    rank = np.empty((F, F), dtype=np.int64)
    for p in range(F):
        d2 = (hp - hp[p]) ** 2 + (wp - wp[p]) ** 2
        rank[p, np.lexsort((-np.arange(F), d2))] = np.arange(F)
    return rank


def _m_static_no_floor(g, gamma, lam):
    return _ORIG['static_ratio_counts'](g, gamma, 0.0)


def _m_static_decay_from_one(g, gamma, lam):
    c = _ORIG['static_ratio_counts'](g, gamma, lam)
    return np.concatenate([c[1:], c[-1:]])


def _m_gathered_transposed(Qr, Kr, Vr, block_mask, g, scale, blocks):
    return _ORIG['masked_attention_blocks'](Qr, Kr, Vr, block_mask.T, g, scale, blocks)


def _m_band_wide(res, prm, band=1e-5):
    return _ORIG['exemption_sets'](res, prm, 1e-3)


def _m_band_keeps_sta(res, prm, band=1e-5):
    return _ORIG['exemption_sets'](res, prm, band) | (_ORIG['exemption_sets'](
        dataclasses.replace(res, sta=np.zeros_like(res.sta)), prm, band))


def _m_band_dyn_on_probs(res, prm, band=1e-5):
    if prm.mode != "dyn":
        return _ORIG['exemption_sets'](res, prm, band)
    edge = res.Pm.max(axis=-1, keepdims=True) * math.exp(-prm.tau)
    return (np.abs(res.Pm - edge) <= band) & ~res.sta


def _m_band_inclusive_mass(res, prm, band=1e-5):
    if prm.mode != "cdf" or not 0 < prm.thr < 1:
        return _ORIG['exemption_sets'](res, prm, band)
    return (np.abs(res.c_excl + res.Pm - prm.thr) <= band) & ~res.sta


MUTATIONS = {
    "rank ascending": ("rank_order", _m_sort_ascending),
    "ties high index first": ("rank_order", _m_tie_high_first),
    "cdf inclusive mass": ("cdf_select_row", _m_cdf_inclusive),
    "cdf <= instead of <": ("cdf_select_row", _m_cdf_le),
    "patch rows/cols swapped in reorder": ("fractal_positions", _m_positions_patch_transposed),
    "time not outermost": ("fractal_positions", _m_positions_time_inner),
    "sta window too wide": ("sta_block_mask", _m_sta_wide),
    "pool sums not means": ("block_means", _m_block_sums),
    "column softmax": ("softmax_rows", _m_softmax_cols),
    "dyn strict": ("dyn_select_row", _m_dyn_strict),
    "dyn from row min": ("dyn_select_row", _m_dyn_from_min),
    "pack msb first": ("pack_bits", _m_pack_msb),
    "mask transposed in attention": ("masked_attention_head", _m_attn_transposed),
    "attention scale dropped": ("masked_attention_head", _m_attn_no_scale),
    "inverse reorder = forward": ("inverse_reorder", _m_inverse_as_forward),
    "backward without D": ("masked_attention_backward_head", _bwd_flawed("no D")),
    "backward mask transposed": ("masked_attention_backward_head", _bwd_flawed("mask transposed")),
    "backward dK unscaled": ("masked_attention_backward_head", _bwd_flawed("dK unscaled")),
    "backward dV from dS": ("masked_attention_backward_head", _bwd_flawed("dV from dS")),
    "backward ignores the given O": ("masked_attention_backward_head", _bwd_flawed("ignores O")),
    "static Chebyshev distance": ("static_ratio_ranks", _m_static_chebyshev),
    "static ties high index first": ("static_ratio_ranks", _m_static_tie_high),
    "static floor ignored": ("static_ratio_counts", _m_static_no_floor),
    "static decay one frame early": ("static_ratio_counts", _m_static_decay_from_one),
    "gathered attention with the mask transposed": ("masked_attention_blocks", _m_gathered_transposed),
    "band 1e-3 instead of 1e-5": ("exemption_sets", _m_band_wide),
    "band exempts sliding-tile blocks": ("exemption_sets", _m_band_keeps_sta),
    "dynamic band on probabilities": ("exemption_sets", _m_band_dyn_on_probs),
    "band on the inclusive mass": ("exemption_sets", _m_band_inclusive_mass),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    orig = getattr(R, attr)
    monkeypatch.setattr(R, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin)
    monkeypatch.setattr(R, attr, orig)
    assert failed, f"no pin detects the planted mistake: {name}"
