"""Comparison helpers for the GPU parity tests (test infrastructure).

Mask rule: the GPU's block mask must equal the oracle's bit for bit, except on
blocks whose decision sits within 1e-5 of the threshold (cumulative mass in CDF
mode, logit edge in dynamic mode); STA blocks are never exempt.
Attention rule: evaluated on the GPU's own mask (after it passed the mask
check), bf16: max |dO| <= 2e-2 and ||dO||_2 / ||O||_2 <= 5e-3; float32: max |dO| <= 1e-4.
Gradient rule (bf16 backward, on the GPU's mask, O and lse): per tensor,
||dG||_2 / ||G||_2 <= 1e-2 and max |dG| <= 2e-2 * max |G|. The kernels round P and dS to
bf16 for the products (relative error <= 2^-9 each) and the results to bf16 (another
2^-9): about 2e-3 in relative L2 for sums of many terms, so 1e-2 leaves a 5x margin.
"""
import dataclasses
import json
import math
import os

import numpy as np
import torch

from oracle import nabla_ref as R

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
F32_MAX_ABS = 1e-4
BAND = 1e-5


def geoms(B, H, T, Hs, Ws, d, P=8):
    import block_sparse_attention_21_amd as A
    return A.Geometry(B, H, T, Hs, Ws, d, P), R.Geom(B, H, T, Hs, Ws, d, P)


def oracle_params(p) -> R.MaskParams:
    return R.MaskParams(mode=p.mode, thr=p.thr, tau=p.tau, pool_scale=p.pool_scale, sta=tuple(p.sta),
                        gamma=p.gamma, lam=p.lam)


def host_words(words: torch.Tensor) -> np.ndarray:
    return words.cpu().numpy().view(np.uint32)


@dataclasses.dataclass
class MaskReport:
    diff: int
    exempt_diff: int
    kept: int
    total: int
    band: int = 0  # blocks inside the band (where a difference would be allowed)


def record(**fields):
    """Append one JSON line of parity statistics to the file ABLA_PARITY_RECORDS names (if any)."""
    path = os.environ.get("ABLA_PARITY_RECORDS")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps(fields) + "\n")


def check_mask(words, counts, lists, mres: R.MaskResult, prm: R.MaskParams, og: R.Geom, heads=None) -> MaskReport:
    """Compare GPU mask outputs (device tensors) with the oracle's MaskResult; returns GPU bool mask."""
    w = host_words(words)
    gm = R.unpack_bits(w, og.nb)
    om = mres.mask
    if heads is not None:
        gm = gm[:, heads]
    assert gm.shape == om.shape
    # Pad bits beyond nb are zero.
    pad = og.nb % 32
    if pad:
        assert (w[..., -1] >> np.uint32(pad) == 0).all()
    ex = R.exemption_sets(mres, prm, BAND)
    diff = gm != om
    bad = diff & ~ex
    assert not bad.any(), f"{int(bad.sum())} mask bits differ outside the {BAND} band, first at {np.argwhere(bad)[:5]}"
    # STA blocks are always kept.
    assert (gm | ~mres.sta[None, None]).all()
    # counts = popcount; lists ascending and equal to the set bits.
    c = counts.cpu().numpy()
    if heads is not None:
        c = c[:, heads]
    assert np.array_equal(c, gm.sum(-1))
    if lists is not None:
        L = lists.cpu().numpy()
        if heads is not None:
            L = L[:, heads]
        for idx in np.ndindex(gm.shape[:-1]):
            n = c[idx]
            assert np.array_equal(L[idx][:n], np.nonzero(gm[idx])[0]), idx
    return MaskReport(int(diff.sum()), int((diff & ex).sum()), int(gm.sum()), int(gm.size), int(ex.sum()))


def gpu_mask(words, og: R.Geom) -> np.ndarray:
    return R.unpack_bits(host_words(words), og.nb)


def compare_attention(out_gpu: np.ndarray, out_ref: np.ndarray, dtype: str):
    d = np.abs(out_gpu.astype(np.float64) - out_ref)
    max_abs = float(d.max()) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(out_ref), 1e-300))
    if dtype == "bf16":
        assert max_abs <= BF16_MAX_ABS, f"max |dO| {max_abs}"
        assert rel <= BF16_REL_L2, f"rel L2 {rel}"
    else:
        assert max_abs <= F32_MAX_ABS, f"max |dO| {max_abs}"
    return max_abs, rel


BWD_REL_L2 = 1e-2
BWD_MAX_REL = 2e-2
# float32 gradients: no rounding of P, dS or the outputs, float32 sums of a few thousand terms
# (relative error of order 1e-6); the bar leaves two orders of magnitude.
BWD_F32_REL_L2 = 1e-4
BWD_F32_MAX_REL = 1e-3


def grad_errors(gpu: np.ndarray, ref: np.ndarray):
    """(relative L2 error, max error / max |ref|); (0, 0) when both are zero, inf when only ref is."""
    d = np.abs(gpu.astype(np.float64) - ref)
    peak = float(np.abs(ref).max()) if ref.size else 0.0
    if peak == 0.0:
        return (0.0, 0.0) if not d.any() else (math.inf, math.inf)
    return float(np.linalg.norm(d) / np.linalg.norm(ref)), float(d.max()) / peak


def compare_grad(gpu: np.ndarray, ref: np.ndarray, name: str, dtype: str = "bf16"):
    """Gradient rule: relative L2 and max error relative to the largest reference entry."""
    rel, mx = grad_errors(gpu, ref)
    bar_rel, bar_max = (BWD_REL_L2, BWD_MAX_REL) if dtype == "bf16" else (BWD_F32_REL_L2, BWD_F32_MAX_REL)
    assert rel <= bar_rel, f"{name}: rel L2 {rel:.3e}"
    assert mx <= bar_max, f"{name}: max err / max |ref| {mx:.3e}"
    return rel, mx


def sample_rows(og: R.Geom, blocks) -> np.ndarray:
    """All 64 query rows (fractal order) of the given query blocks."""
    return np.concatenate([np.arange(b * og.bs, (b + 1) * og.bs) for b in blocks])
