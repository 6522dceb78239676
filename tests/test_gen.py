"""The synthetic workloads: reproducible and with the statistics their recipe states."""
import hashlib

import numpy as np
import torch

from gen import WORKLOADS, make_qkv, make_random_qkv


def _digest(ts):
    h = hashlib.sha256()
    for t in ts:
        h.update(t.float().numpy().tobytes())
    return h.hexdigest()


def test_deterministic_and_head_independent():
    w = WORKLOADS["tiny"]
    assert _digest(make_qkv(w)) == _digest(make_qkv(w))
    full = make_qkv(w)
    one = make_qkv(w, heads=[1])
    for a, b in zip(full, one):
        assert torch.equal(a[:, 1:2], b)
    assert _digest(make_qkv(w.with_(seed=1))) != _digest(full)


def test_tiny_statistics():
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w)
    assert q.shape == (1, 2, 2048, 64) and q.dtype == torch.float32
    for x in (q, k):
        assert abs(x.pow(2).mean().sqrt().item() - 1.0) < 1e-4
    assert abs(v.std().item() - 1.0) < 0.02
    # Q and K share the smooth field: strongly but not perfectly correlated.
    c = torch.corrcoef(torch.stack([q.flatten(), k.flatten()]))[0, 1].item()
    assert 0.85 < c < 0.97


def test_video_statistics_and_copies():
    w = WORKLOADS["480p"]
    q, k, v = make_qkv(w, heads=[0])
    assert q.dtype == torch.bfloat16 and q.shape == (1, 1, w.N, w.d)
    assert torch.equal(q, k)  # Q and K are the same field in this recipe
    F = q[0, 0].float().reshape(w.T, w.Hs, w.Ws, w.d)
    assert abs(F.pow(2).mean().sqrt().item() - 1.0) < 0.01
    # Lag-1 temporal correlation is rho before the copies (each copied block breaks two lags).
    F0 = make_qkv(w.with_(copy_frac=0.0), heads=[0])[0][0, 0].float().reshape(F.shape)
    a, b = F0[:-1].flatten(), F0[1:].flatten()
    rho = (a * b).mean() / (a.pow(2).mean() * b.pow(2).mean()).sqrt()
    assert abs(rho.item() - w.rho) < 0.03
    # Spatially smooth: neighbouring tokens are strongly correlated.
    a, b = F[:, :, :-1].flatten(), F[:, :, 1:].flatten()
    assert (a * b).mean().item() > 0.9
    # round(5% of nb) blocks are exact copies of a block >= max(2, T//4) frames away.
    P, nbh, nbw = w.P, w.Hs // w.P, w.Ws // w.P
    blocks = F.reshape(w.T, nbh, P, nbw, P, w.d).permute(0, 1, 3, 2, 4, 5).reshape(w.nb, -1)
    _, inv, cnt = np.unique(blocks.numpy(), axis=0, return_inverse=True, return_counts=True)
    dup = cnt[inv.reshape(-1)] > 1
    n_copy = int(round(w.copy_frac * w.nb))
    assert n_copy <= dup.sum() <= 2 * n_copy
    t_of = np.arange(w.nb) // (nbh * nbw)
    for grp in np.unique(inv.reshape(-1)[dup]):
        ts = t_of[inv.reshape(-1) == grp]
        assert ts.max() - ts.min() >= max(2, w.T // 4)
    assert abs(v.float().std().item() - 1.0) < 0.01


def test_random_qkv_shapes():
    q, k, v = make_random_qkv(1, 2, 2, 8, 16, 64, dtype="f32")
    assert q.shape == (1, 2, 256, 64) and not torch.equal(q, k)
