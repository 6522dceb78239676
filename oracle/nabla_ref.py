"""CPU oracle for NABLA block-sparse video attention and its dynamic-threshold variant.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never calls it, and it shares no code, tables or constants
with that path.

Everything here is plain numpy in float64 and follows the method's steps in the
order the pages give them. Sources (page title, then section):

* [NABLA] "NABLA: Neighborhood Adaptive Block-Level Attention" -- technical
  summary, Method: token reordering (Fractal Flattening); adaptive mask
  construction (down-sampling, reduced attention, CDF thresholding,
  expansion); hybrid integration with STA (M = M_nabla OR M_STA).
* [DynamicRad] "DynamicRad: Content-Adaptive Sparse Attention for Long Video
  Diffusion" -- Methodology A, dual-mode strategy: the Dynamic-Threshold mode
  uses pre-softmax attention logits as the importance proxy and filters by a
  threshold; the Static-Ratio mode scores nothing and keeps blocks at a fixed
  retention ratio that depends on the temporal distance (decay coefficient
  gamma, long-range factor lambda).

Readings taken where the pages leave a step open (each is also listed in the
design notes):

1. CDF direction: rows are ranked by importance first; the kept set is the
   shortest prefix of the descending order whose mass reaches thr. With
   C_excl(r) the mass ranked before r, rank r is kept iff C_excl(r) < thr.
   This equals the page's "cumulative probability (ascending) exceeds 1 - thr".
2. A block is one P x P patch of one frame (P*P = 64 tokens); block i has
   coordinates (t, hp, wp) with i = (t*nbh + hp)*nbw + wp.
3. Fractal order: frame outermost, then patch row/column, then the token's
   row/column inside its patch.
4. Pooled logits and attention both use scale 1/sqrt(d) unless given.
5. Ties in the ranking are broken by lower block index first.
6. thr >= 1 keeps every block; thr <= 0 keeps none (before the STA union).
7. Dynamic threshold at block level on pooled logits: keep j iff
   S_ij >= max_j S_ij - tau.
8. STA window (wt, wh, ww), odd sizes, centred and truncated at the grid
   border; (0, 0, 0) turns it off.
9. A query row with no allowed key gives O = 0 and LSE = -inf.
10. Static-Ratio retention law (the pages name gamma and lambda but give no
    formula): r(0) = 1 and r(dt) = r(dt - 1) * gamma, an exponential decay in
    the frame distance dt evaluated by repeated multiplication; a key frame at
    distance dt keeps k(dt) = min(F, max(ceil(F * lambda), ceil(F * r(dt))))
    of its F blocks, lambda being the long-range floor; the kept blocks of a
    frame are the k(dt) nearest to the query block's spatial position, ordered
    by squared distance in blocks, ties by lower position index. The result is
    OR-ed with the STA window like the other modes.

Parity pins: every function is checked in tests/test_oracle.py against brute
force, closed forms or library routines. The 1/sqrt(d) scales (reading 4) are
conventions the pages do not fix: "parity unpinned" for their value.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Geom:
    B: int
    H: int
    T: int
    Hs: int
    Ws: int
    d: int
    P: int = 8

    @property
    def N(self) -> int:
        return self.T * self.Hs * self.Ws

    @property
    def nbh(self) -> int:
        return self.Hs // self.P

    @property
    def nbw(self) -> int:
        return self.Ws // self.P

    @property
    def nb(self) -> int:
        return self.T * self.nbh * self.nbw

    @property
    def bs(self) -> int:
        return self.P * self.P

    def check(self) -> None:
        if min(self.B, self.H, self.T, self.Hs, self.Ws, self.d, self.P) <= 0:
            raise ValueError("non-positive dimension")
        if self.Hs % self.P or self.Ws % self.P:
            raise ValueError("Hs and Ws must be multiples of P")


@dataclasses.dataclass(frozen=True)
class MaskParams:
    mode: str = "cdf"  # "cdf", "dyn" or "static"
    thr: float = 0.9
    tau: float = 4.0
    pool_scale: float = 0.0  # 0 -> 1/sqrt(d)
    sta: tuple = (3, 3, 3)  # (0, 0, 0) -> off
    gamma: float = 0.5  # static: retention decay per frame of distance
    lam: float = 0.05  # static: long-range floor of the retention ratio


# --------------------------------------------------------------------------
# [NABLA] Method: token reordering (Fractal Flattening).
# Tokens of each P x P spatial patch become one contiguous run; the temporal
# order is kept (frames stay outermost).
# --------------------------------------------------------------------------
def fractal_positions(g: Geom) -> np.ndarray:
    """pos[n] = index in the reordered sequence of original token n = (t*Hs + y)*Ws + x."""
    t, y, x = np.meshgrid(np.arange(g.T), np.arange(g.Hs), np.arange(g.Ws), indexing="ij")
    hp, py = np.divmod(y, g.P)
    wp, px = np.divmod(x, g.P)
    block = (t * g.nbh + hp) * g.nbw + wp
    within = py * g.P + px
    return (block * g.bs + within).reshape(-1)


def reorder(X: np.ndarray, g: Geom) -> np.ndarray:
    """X[..., n, :] in original order -> X_r[..., pos[n], :] in fractal order."""
    pos = fractal_positions(g)
    Y = np.empty_like(X)
    Y[..., pos, :] = X
    return Y


def inverse_reorder(Xr: np.ndarray, g: Geom) -> np.ndarray:
    """Undo `reorder`: X[..., n, :] = X_r[..., pos[n], :]."""
    return Xr[..., fractal_positions(g), :]


def block_coords(g: Geom) -> np.ndarray:
    """(t, hp, wp) of every block index i, shape [nb, 3]."""
    i = np.arange(g.nb)
    t, r = np.divmod(i, g.nbh * g.nbw)
    hp, wp = np.divmod(r, g.nbw)
    return np.stack([t, hp, wp], axis=1)


# --------------------------------------------------------------------------
# [NABLA] Method: adaptive mask construction -- down-sampling.
# Q and K are reshaped and mean-pooled over N x N blocks (64-token blocks).
# --------------------------------------------------------------------------
def block_means(Xr: np.ndarray, g: Geom) -> np.ndarray:
    """Mean of each run of P*P reordered tokens: [..., N, d] -> [..., nb, d] (float64)."""
    Xr = np.asarray(Xr, dtype=np.float64)
    return Xr.reshape(Xr.shape[:-2] + (g.nb, g.bs, Xr.shape[-1])).mean(axis=-2)


# --------------------------------------------------------------------------
# [NABLA] Method: reduced attention -- a full attention map over the pooled
# block representations.
# --------------------------------------------------------------------------
def pooled_logits(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """S_ij = scale * <qbar_i, kbar_j> (pre-softmax), [..., nb, nb].

    Every dot product is summed in the same order (numpy's own loop, not a
    blocked BLAS kernel), so blocks with identical pooled keys get identical
    logits and stay exactly tied, as the definition makes them.
    """
    return scale * np.einsum("...ic,...jc->...ij", qbar, kbar, optimize=False)


def softmax_rows(S: np.ndarray) -> np.ndarray:
    m = S.max(axis=-1, keepdims=True)
    e = np.exp(S - m)
    return e / e.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# [NABLA] Method: CDF thresholding. For each row of the reduced map the blocks
# are ranked by probability and the row's cumulative distribution decides
# which blocks survive; per attention head and per input.
# --------------------------------------------------------------------------
def rank_order(p: np.ndarray) -> np.ndarray:
    """Block indices of one row in ranking order: probability descending, index ascending."""
    j = np.arange(p.shape[-1])
    return np.lexsort((j, -p))


def cdf_select_row(p: np.ndarray, thr: float):
    """Keep flags and C_excl (mass ranked strictly before each block) for one row."""
    n = p.shape[-1]
    order = rank_order(p)
    mass_sorted = p[order]
    c_excl_sorted = np.concatenate([[0.0], np.cumsum(mass_sorted)[:-1]])
    c_excl = np.empty(n)
    c_excl[order] = c_excl_sorted
    if thr >= 1.0:
        keep = np.ones(n, dtype=bool)
    else:
        keep = c_excl < thr
    return keep, c_excl


# --------------------------------------------------------------------------
# [DynamicRad] Methodology A: Dynamic-Threshold mode -- pre-softmax logits as
# the importance proxy, filtered by a threshold (here relative to the row max).
# --------------------------------------------------------------------------
def dyn_select_row(s: np.ndarray, tau: float) -> np.ndarray:
    return s >= s.max() - tau


# --------------------------------------------------------------------------
# [NABLA] Method: hybrid integration with Sliding Tile Attention -- the final
# mask is the logical OR of the adaptive mask and a static local tile window.
# --------------------------------------------------------------------------
def sta_block_mask(g: Geom, window: Sequence[int]) -> np.ndarray:
    wt, wh, ww = (int(w) for w in window)
    if (wt, wh, ww) == (0, 0, 0):
        return np.zeros((g.nb, g.nb), dtype=bool)
    c = block_coords(g)
    rt, rh, rw = (wt - 1) // 2, (wh - 1) // 2, (ww - 1) // 2
    dt = np.abs(c[:, None, 0] - c[None, :, 0])
    dh = np.abs(c[:, None, 1] - c[None, :, 1])
    dw = np.abs(c[:, None, 2] - c[None, :, 2])
    return (dt <= rt) & (dh <= rh) & (dw <= rw)


# --------------------------------------------------------------------------
# [DynamicRad] Methodology A, Static-Ratio mode: no content scoring; each key
# frame keeps a share of its blocks fixed by its temporal distance to the query
# block (reading 10 above for the law the pages leave open).
# --------------------------------------------------------------------------
def static_ratio_counts(g: Geom, gamma: float, lam: float) -> np.ndarray:
    """k(dt) for dt = 0 .. T-1: blocks kept in a key frame at frame distance dt."""
    F = g.nbh * g.nbw
    floor_k = math.ceil(F * lam)
    out = np.empty(g.T, dtype=np.int64)
    r = 1.0
    for dt in range(g.T):
        out[dt] = min(F, max(floor_k, math.ceil(F * r)))
        r = r * gamma
    return out


def static_ratio_ranks(g: Geom) -> np.ndarray:
    """rank[p, q]: place of frame position q in the ordering of all positions of a frame by
    (squared block distance to position p, position index); positions p = hp * nbw + wp."""
    F = g.nbh * g.nbw
    hp, wp = np.divmod(np.arange(F), g.nbw)
    rank = np.empty((F, F), dtype=np.int64)
    for p in range(F):
        d2 = (hp - hp[p]) ** 2 + (wp - wp[p]) ** 2
        order = np.lexsort((np.arange(F), d2))  # by d2, then by index
        rank[p, order] = np.arange(F)
    return rank


def static_ratio_block_mask(g: Geom, gamma: float, lam: float) -> np.ndarray:
    """[nb, nb] bool: query block i keeps key block j iff j's rank around i's position is
    below the count of j's frame distance."""
    c = block_coords(g)
    k = static_ratio_counts(g, gamma, lam)
    rank = static_ratio_ranks(g)
    pos = c[:, 1] * g.nbw + c[:, 2]
    dt = np.abs(c[:, None, 0] - c[None, :, 0])
    return rank[pos[:, None], pos[None, :]] < k[dt]


@dataclasses.dataclass
class MaskResult:
    S: np.ndarray  # pooled logits [B,H,nb,nb]
    Pm: np.ndarray  # pooled probabilities [B,H,nb,nb]
    sel: np.ndarray  # content-selected blocks (before STA) [B,H,nb,nb] bool
    sta: np.ndarray  # STA window [nb,nb] bool
    mask: np.ndarray  # final block mask [B,H,nb,nb] bool
    c_excl: Optional[np.ndarray]  # CDF mode: mass ranked before each block [B,H,nb,nb]


def build_block_mask(qbar: np.ndarray, kbar: np.ndarray, g: Geom, prm: MaskParams) -> MaskResult:
    """Steps: reduced attention -> per-row selection (CDF or dynamic threshold) -> OR STA.
    Static-Ratio mode: the content-independent selection -> OR STA (qbar, kbar unused)."""
    if prm.mode == "static":
        sel = np.broadcast_to(static_ratio_block_mask(g, prm.gamma, prm.lam), (g.B, g.H, g.nb, g.nb)).copy()
        sta = sta_block_mask(g, prm.sta)
        return MaskResult(S=None, Pm=None, sel=sel, sta=sta, mask=sel | sta, c_excl=None)
    scale = prm.pool_scale if prm.pool_scale > 0 else 1.0 / math.sqrt(g.d)
    S = pooled_logits(np.asarray(qbar, np.float64), np.asarray(kbar, np.float64), scale)
    Pm = softmax_rows(S)
    sel = np.zeros(S.shape, dtype=bool)
    cex = np.zeros(S.shape) if prm.mode == "cdf" else None
    for idx in np.ndindex(S.shape[:-1]):
        if prm.mode == "cdf":
            sel[idx], cex[idx] = cdf_select_row(Pm[idx], prm.thr)
        elif prm.mode == "dyn":
            sel[idx] = dyn_select_row(S[idx], prm.tau)
        else:
            raise ValueError(prm.mode)
    sta = sta_block_mask(g, prm.sta)
    return MaskResult(S=S, Pm=Pm, sel=sel, sta=sta, mask=sel | sta, c_excl=cex)


def exemption_sets(res: MaskResult, prm: MaskParams, band: float = 1e-5) -> np.ndarray:
    """Blocks whose decision sits within `band` of the threshold (and outside STA).

    CDF mode: |C_excl - thr| <= band. Dynamic mode: |S_ij - (max_j S_ij - tau)| <= band.
    """
    if prm.mode == "static":
        return np.zeros(res.mask.shape, dtype=bool)
    if prm.mode == "cdf":
        if prm.thr >= 1.0 or prm.thr <= 0.0:
            ex = np.zeros(res.mask.shape, dtype=bool)
        else:
            ex = np.abs(res.c_excl - prm.thr) <= band
    else:
        edge = res.S.max(axis=-1, keepdims=True) - prm.tau
        ex = np.abs(res.S - edge) <= band
    return ex & ~res.sta


# --------------------------------------------------------------------------
# [NABLA] Method: expansion -- the binary block mask is expanded back to token
# resolution; it names the N x N attention blocks that are computed. Here it is
# kept in two compact forms: packed bits and ascending per-row lists.
# --------------------------------------------------------------------------
def pack_bits(mask: np.ndarray) -> np.ndarray:
    """[..., nb] bool -> [..., ceil(nb/32)] uint32; bit j%32 of word j//32 (LSB first)."""
    nb = mask.shape[-1]
    W = (nb + 31) // 32
    out = np.zeros(mask.shape[:-1] + (W,), dtype=np.uint64)
    for j in range(nb):
        out[..., j // 32] |= mask[..., j].astype(np.uint64) << np.uint64(j % 32)
    return out.astype(np.uint32)


def unpack_bits(words: np.ndarray, nb: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint64)
    j = np.arange(nb)
    return ((words[..., j // 32] >> (j % 32).astype(np.uint64)) & np.uint64(1)).astype(bool)


def kept_lists(mask: np.ndarray):
    """counts [..., nb_rows] and lists [..., nb_rows, nb] (ascending kept indices, rest -1)."""
    counts = mask.sum(axis=-1).astype(np.int32)
    lists = np.full(mask.shape, -1, dtype=np.int32)
    for idx in np.ndindex(mask.shape[:-1]):
        kj = np.nonzero(mask[idx])[0]
        lists[idx][: len(kj)] = kj
    return counts, lists


def expand_to_tokens(block_mask: np.ndarray, g: Geom) -> np.ndarray:
    """Token-level mask in fractal order: allowed[m, m'] = block_mask[m // bs, m' // bs]."""
    b = np.arange(g.N) // g.bs
    return block_mask[..., b[:, None], b[None, :]]


# --------------------------------------------------------------------------
# Block-sparse attention: ordinary scaled dot-product attention in which query
# token m only sees the keys of the blocks its block keeps.
# --------------------------------------------------------------------------
def masked_attention_head(Qr, Kr, Vr, block_mask, g: Geom, scale: float,
                          rows: Optional[np.ndarray] = None, chunk: int = 256):
    """One head in fractal order. Returns (O_r [R, d], lse [R]) for `rows` (default: all).

    Disallowed entries of each score row are set to -inf before the softmax;
    a row with nothing allowed gives O = 0 and lse = -inf.
    """
    Qr = np.asarray(Qr, np.float64)
    Kr = np.asarray(Kr, np.float64)
    Vr = np.asarray(Vr, np.float64)
    rows = np.arange(g.N) if rows is None else np.asarray(rows)
    key_block = np.arange(g.N) // g.bs
    O = np.zeros((len(rows), Vr.shape[-1]))
    lse = np.full(len(rows), -np.inf)
    for s in range(0, len(rows), chunk):
        r = rows[s:s + chunk]
        allowed = block_mask[(r // g.bs)[:, None], key_block[None, :]]
        sc = scale * (Qr[r] @ Kr.T)
        sc = np.where(allowed, sc, -np.inf)
        mx = sc.max(axis=1)
        live = np.isfinite(mx)
        e = np.exp(sc[live] - mx[live, None])
        z = e.sum(axis=1)
        O[s:s + chunk][live] = (e @ Vr) / z[:, None]
        lse[s:s + chunk][live] = mx[live] + np.log(z)
    return O, lse


def masked_attention_blocks(Qr, Kr, Vr, block_mask, g: Geom, scale: float, blocks):
    """The rows of the given query blocks of one head (fractal order), each attending only to
    the tokens of the key blocks its mask row keeps. Same definition as masked_attention_head
    (a dropped key's weight is exp(-inf) = 0, so leaving it out changes nothing); the cost is
    the kept fraction of the dense row. Returns (O [len(blocks)*bs, d], lse [len(blocks)*bs])
    with the rows of block blocks[n] at n*bs .. n*bs + bs - 1.
    """
    Qr = np.asarray(Qr, np.float64)
    Kr = np.asarray(Kr, np.float64)
    Vr = np.asarray(Vr, np.float64)
    bs = g.bs
    O = np.zeros((len(blocks) * bs, Vr.shape[-1]))
    lse = np.full(len(blocks) * bs, -np.inf)
    within = np.arange(bs)
    for n, i in enumerate(blocks):
        kept = np.nonzero(block_mask[i])[0]
        if len(kept) == 0:
            continue
        keys = (kept[:, None] * bs + within[None, :]).reshape(-1)
        sc = scale * (Qr[i * bs:(i + 1) * bs] @ Kr[keys].T)
        mx = sc.max(axis=1)
        e = np.exp(sc - mx[:, None])
        z = e.sum(axis=1)
        O[n * bs:(n + 1) * bs] = (e @ Vr[keys]) / z[:, None]
        lse[n * bs:(n + 1) * bs] = mx + np.log(z)
    return O, lse


def masked_attention_backward_head(Qr, Kr, Vr, dOr, block_mask, g: Geom, scale: float,
                                   rows: Optional[np.ndarray] = None, O: Optional[np.ndarray] = None,
                                   chunk: int = 256):
    """Gradients of the block-sparse attention of one head (fractal order), float64.

    With S = scale * Q K^T restricted to the allowed blocks, P = row softmax of S (zero
    outside the allowed blocks, and zero rows where nothing is allowed), O = P V and the
    incoming gradient dO, the chain rule gives
        dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij = <dO_i, O_i>,
        dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
    Returns (dQ, dK, dV): dQ [R, d] for the query rows `rows` (default: all N), dK and dV
    [N, d] summed over those rows only. A query row contributes nothing to the keys of the
    blocks its mask row drops, so dK / dV of a key block are complete once `rows` holds
    every row of every query block that keeps it. Rows are processed in chunks of `chunk`.
    `O` ([N, d], fractal order) is the forward output the backward is handed, as stored (for
    instance rounded to bf16); D is then <dO_i, O_i> of that O. By default O is the exact
    P V recomputed here.
    """
    Qr, Kr, Vr, dOr = (np.asarray(x, np.float64) for x in (Qr, Kr, Vr, dOr))
    rows = np.arange(g.N) if rows is None else np.asarray(rows)
    key_block = np.arange(g.N) // g.bs
    dQ = np.zeros((len(rows), Qr.shape[-1]))
    dK = np.zeros_like(Kr)
    dV = np.zeros_like(Vr)
    for s in range(0, len(rows), chunk):
        r = rows[s:s + chunk]
        allowed = block_mask[(r // g.bs)[:, None], key_block[None, :]]
        sc = np.where(allowed, scale * (Qr[r] @ Kr.T), -np.inf)
        mx = sc.max(axis=1)
        live = np.isfinite(mx)
        P = np.zeros_like(sc)
        e = np.exp(sc[live] - mx[live, None])
        P[live] = e / e.sum(axis=1, keepdims=True)
        Orow = P @ Vr if O is None else np.asarray(O, np.float64)[r]
        dP = dOr[r] @ Vr.T
        D = np.sum(dOr[r] * Orow, axis=1)
        dS = P * (dP - D[:, None])
        dQ[s:s + len(r)] = scale * (dS @ Kr)
        dK += scale * (dS.T @ Qr[r])
        dV += P.T @ dOr[r]
    return dQ, dK, dV


@dataclasses.dataclass
class NablaResult:
    O: np.ndarray  # [B,H,N,d] original order
    O_r: np.ndarray  # [B,H,N,d] fractal order
    lse_r: np.ndarray  # [B,H,N] fractal order
    qbar: np.ndarray
    kbar: np.ndarray
    mask: MaskResult


def to64(x) -> np.ndarray:
    """Host float64 copy of a numpy array or a (CPU or GPU) torch tensor, exactly upcast."""
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def nabla_attention(Q, K, V, g: Geom, prm: MaskParams, attn_scale: float = 0.0,
                    block_mask: Optional[np.ndarray] = None) -> NablaResult:
    """The whole path: reorder -> pool -> mask -> block-sparse attention -> inverse reorder.

    If `block_mask` is given it replaces the oracle's own mask in the attention
    step (used to evaluate the attention on a mask produced elsewhere).
    """
    g.check()
    Q, K, V = to64(Q), to64(K), to64(V)
    Qr, Kr, Vr = reorder(Q, g), reorder(K, g), reorder(V, g)
    qbar, kbar = block_means(Qr, g), block_means(Kr, g)
    mres = build_block_mask(qbar, kbar, g, prm)
    bm = mres.mask if block_mask is None else block_mask
    scale = attn_scale if attn_scale > 0 else 1.0 / math.sqrt(g.d)
    O_r = np.zeros_like(Qr)
    lse = np.zeros(Qr.shape[:-1])
    for b in range(g.B):
        for h in range(g.H):
            O_r[b, h], lse[b, h] = masked_attention_head(Qr[b, h], Kr[b, h], Vr[b, h], bm[b, h], g, scale)
    return NablaResult(O=inverse_reorder(O_r, g), O_r=O_r, lse_r=lse, qbar=qbar, kbar=kbar, mask=mres)
