/*
 * abla -- block-sparse 3D self-attention for video diffusion transformers on
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes the NABLA attention path ("NABLA: Neighborhood Adaptive
 * Block-Level Attention", technical summary, Method section) and the
 * dynamic-threshold selection of "DynamicRad: Content-Adaptive Sparse
 * Attention for Long Video Diffusion" (Methodology A, Dynamic-Threshold mode):
 *
 *   abla_reorder          fractal flattening of the tokens + block mean-pooling
 *   abla_pool_qk_reorder_v  the layer's first step (Q, K pooling, V reorder) in one launch
 *   abla_build_mask       reduced attention over pooled blocks, per-row CDF cut
 *                         (or logit threshold), OR the sliding-tile window
 *   abla_sparse_attn_fwd  attention restricted to the kept 64 x 64 blocks
 *   abla_sparse_attn_bwd  its gradients dQ, dK, dV through the same mask
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * - Geometry: a video latent of T frames of Hs x Ws tokens, N = T*Hs*Ws tokens,
 *   B batches, H heads, head dim d. Blocks are P x P spatial patches of one
 *   frame; only P*P = 64 is implemented. nbh = Hs/P, nbw = Ws/P,
 *   nb = T*nbh*nbw. Block i has coordinates (t, hp, wp) with
 *   i = (t*nbh + hp)*nbw + wp.
 * - Original token order: n = (t*Hs + y)*Ws + x.
 * - Fractal order: token (t, y, x) sits at m = i*64 + (y % P)*P + (x % P)
 *   where i is its block: each patch is one contiguous run, frames stay
 *   outermost ("Fractal Flattening", NABLA Method section).
 * - All pointers are device pointers owned by the caller, contiguous,
 *   row-major and 16-byte aligned (a misaligned pointer is rejected with
 *   ABLA_ERR_INVALID). The library never allocates, frees or
 *   synchronises and keeps no pointer after a call returns; its only mutable
 *   global state is the scratch array of abla_sparse_attn_fwd_noalloc (one
 *   per GPU, below). Work is enqueued on `stream` (a hipStream_t; NULL is the
 *   default stream) and results are valid when the stream reaches them.
 * - Arguments are validated on the host before anything is enqueued, so
 *   every ABLA_ERR_INVALID / _UNSUPPORTED / _WORKSPACE return has enqueued
 *   nothing. ABLA_ERR_HIP means a launch failed (hipGetLastError).
 * - No C++ exception crosses this interface.
 */
#ifndef ABLA_H
#define ABLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ABLA_OK = 0,
  ABLA_ERR_INVALID = 1,     /* null or misaligned pointer, bad size, NaN threshold, even window, aliasing */
  ABLA_ERR_UNSUPPORTED = 2, /* valid but not implemented: P*P != 64, d not in {64,128}, nb > 4096 */
  ABLA_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than the *_workspace_bytes value */
  ABLA_ERR_HIP = 4          /* a kernel launch failed */
} abla_status;

typedef enum { ABLA_F32 = 0, ABLA_BF16 = 1 } abla_dtype;

/* Output layout of abla_reorder.
 * ABLA_LAYOUT_TOKENS:  [B, H, N, d], token-major, fractal order.
 * ABLA_LAYOUT_BLOCK_T: [B, H, nb, d, 64]: each 64-token block stored
 *                      channel-major (element (m, c) of block i at
 *                      ((b*H + h)*nb + i)*d*64 + c*64 + m%64). This is the
 *                      layout abla_sparse_attn_fwd takes V in. */
typedef enum { ABLA_LAYOUT_TOKENS = 0, ABLA_LAYOUT_BLOCK_T = 1 } abla_layout;

typedef struct {
  int64_t B, H, T, Hs, Ws, d;
  int32_t P;
} abla_geom;

typedef enum { ABLA_MASK_CDF = 0, ABLA_MASK_DYN = 1, ABLA_MASK_STATIC = 2 } abla_mask_mode;

/* How the CDF cut finds the last kept rank of a row. All give the same bits.
 * ABLA_CUT_RADIX:      radix select on the 64-bit (probability, ~index) keys with exact
 *                      fixed-point mass histograms (default; no full sort). Rows of up
 *                      to 1280 blocks run on one or two waves each.
 * ABLA_CUT_BITONIC:    full LDS bitonic sort of the keys, then an exact prefix sum.
 * ABLA_CUT_RADIX_WIDE: the radix select with four waves per row whatever nb is, so the
 *                      same rows run at another workgroup size and LDS partition (a
 *                      cross-check for races). It applies to every mode: DYN and STATIC
 *                      rows then run on four waves too; the other values leave them on
 *                      the default width. */
typedef enum { ABLA_CUT_RADIX = 0, ABLA_CUT_BITONIC = 1, ABLA_CUT_RADIX_WIDE = 2 } abla_cut_algorithm;

typedef struct {
  int32_t mode;       /* abla_mask_mode */
  double thr;         /* CDF mode: probability-mass threshold; >= 1 keeps all, <= 0 keeps none */
  double tau;         /* DYN mode: keep j iff S_ij >= max_j S_ij - tau (pooled, scaled logits) */
  double pool_scale;  /* scale of the pooled logits; 0 means 1/sqrt(d) */
  int32_t sta_t, sta_h, sta_w; /* sliding-tile window in blocks, odd; all 0 = no STA */
  int32_t cut;        /* abla_cut_algorithm */
  double gamma;       /* STATIC mode: retention decay per frame of temporal distance, in [0, 1] */
  double lambda;      /* STATIC mode: long-range floor of the retention ratio, in [0, 1] */
} abla_mask_params;

/* Fractal reordering and block mean-pooling of one tensor.
 * Source: NABLA, Method -- "Fractal Flattening" (patch tokens made contiguous,
 * time order kept) and "down-sampling" (Q and K mean-pooled over 64-token
 * blocks).
 *
 * inverse = 0: x is [B,H,N,d] in original order; y receives the fractal-order
 *   tensor in `layout`. If `pooled` is not NULL it receives [B,H,nb,d] float64
 *   block means: the 64 input values of a block summed in float64 (exact for
 *   bf16 inputs) and divided by 64. The mask decisions downstream are taken in
 *   float64 so that they do not hinge on float32 rounding.
 *   With y = NULL (ABLA_LAYOUT_TOKENS, pooled given) only the block means are
 *   written: the pooling pass for consumers that read x in its original order
 *   (abla_sparse_attn_fwd with ABLA_ATTN_QK_ORIGINAL).
 * inverse = 1: x is [B,H,N,d] in fractal order (ABLA_LAYOUT_TOKENS only) and
 *   y receives the original order; `pooled` must be NULL.
 * dtype: element type of x and y. x and y must not overlap.
 * Errors: INVALID for null x, null y other than the pooling-only form, x == y, bad
 * geometry, unknown dtype or layout, inverse with BLOCK_T or with pooled; UNSUPPORTED for P*P != 64, d not in
 * {64, 128}, more than 2^31 - 1 tokens per head or B*H*nb above 2^31 - 1. */
abla_status abla_reorder(const abla_geom* g, int32_t dtype, int32_t inverse, int32_t layout,
                         const void* x, void* y, double* pooled, void* stream);

/* The first step of a layer in one launch: block means of q and k, and v reordered into
 * channel-major blocks. Results are identical to three abla_reorder calls:
 *   abla_reorder(q, y = NULL, qbar), abla_reorder(k, y = NULL, kbar) (pooling only; q and k
 *   stay in the original order for abla_sparse_attn_fwd with ABLA_ATTN_QK_ORIGINAL), and
 *   abla_reorder(v, v_rt, layout ABLA_LAYOUT_BLOCK_T, no pooling).
 * Source: NABLA, Method -- "Fractal Flattening" and "down-sampling" (as abla_reorder).
 * q, k, v: [B,H,N,d] of `dtype` in the original token order.
 * qbar, kbar: [B,H,nb,d] float64 outputs; v_rt: [B,H,nb,d,64] of `dtype` output.
 * One grid of 3*B*H*nb workgroups instead of three launches. With v = v_rt = NULL only q
 * and k are pooled, in one grid of 2*B*H*nb workgroups (the first step when the attention
 * reads V in the original order, ABLA_ATTN_V_ORIGINAL).
 * Errors: INVALID for a null q, k, qbar or kbar, exactly one of v and v_rt null, unknown
 * dtype, bad geometry, an output overlapping an input or another output; UNSUPPORTED for
 * the geometry limits of abla_reorder or 3*B*H*nb above 2^31 - 1. */
abla_status abla_pool_qk_reorder_v(const abla_geom* g, int32_t dtype, const void* q, const void* k, const void* v,
                                   double* qbar, double* kbar, void* v_rt, void* stream);

/* Bytes of scratch abla_build_mask needs: B*H*nb*nb*8 (the float64 pooled score matrix;
 * not used by the STATIC mode). */
size_t abla_build_mask_workspace_bytes(const abla_geom* g);

/* Block mask from pooled Q and K.
 * Source: NABLA, Method -- "reduced attention" (softmax over the pooled block
 * scores), "CDF thresholding" (rank each row, keep the blocks needed for the
 * row's cumulative probability to reach thr), hybrid with STA
 * (M = M_nabla OR M_STA); DynamicRad, Methodology A -- Dynamic-Threshold mode
 * (pre-softmax logits filtered by a threshold) and Static-Ratio mode (no content
 * scoring; a retention ratio fixed by temporal distance, decay gamma, long-range
 * factor lambda).
 *
 * qbar, kbar: [B,H,nb,d] float64 (as written by abla_reorder); not read, and may be
 * NULL, in STATIC mode.
 * Per row (b,h,i): S_ij = pool_scale * <qbar_i, kbar_j>, all in float64.
 *   CDF: P_i. = softmax(S_i.); rank blocks by (P desc, index asc); keep the
 *        block at rank r iff the mass ranked before it is < thr.
 *   DYN: keep j iff S_ij >= max_j S_ij - tau.
 *   STATIC (no scores; the pages name gamma and lambda but give no law, this is the
 *        one implemented): with F = nbh*nbw blocks per frame, r(0) = 1 and
 *        r(dt) = r(dt-1) * gamma (float64 products), a key frame at frame distance
 *        dt = |t_i - t_j| keeps k(dt) = min(F, max(ceil(F*lambda), ceil(F*r(dt))))
 *        blocks: the ones nearest to block i's position (hp, wp), ordered by squared
 *        distance in blocks, ties by lower position index. Identical for every (b, h).
 *   Then OR the STA window: |t_i-t_j| <= (sta_t-1)/2 and likewise for hp, wp.
 * Outputs:
 *   mask_words [B,H,nb,ceil(nb/32)] uint32: bit j%32 of word j/32 (LSB first)
 *              is block j; pad bits are 0.
 *   counts     [B,H,nb] int32: kept blocks per row.
 *   lists      [B,H,nb,nb] int32 or NULL: the kept block indices of each row in
 *              ascending order in the first counts[row] entries; the rest of
 *              the row is left untouched.
 * workspace: at least abla_build_mask_workspace_bytes(g) bytes of device memory (may be
 * NULL in STATIC mode).
 * Errors: INVALID for null inputs/outputs, unknown mode or cut algorithm, NaN thr/tau, negative
 * or NaN pool_scale, gamma or lambda outside [0, 1] in STATIC mode, windows that are even,
 * negative or partly zero, and outputs or the workspace overlapping each other or qbar/kbar;
 * UNSUPPORTED for nb > 4096 or the geometry limits of abla_reorder;
 * WORKSPACE if the workspace is missing or too small. */
abla_status abla_build_mask(const abla_geom* g, const abla_mask_params* p,
                            const double* qbar, const double* kbar,
                            uint32_t* mask_words, int32_t* counts, int32_t* lists,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch abla_sparse_attn_fwd needs: B*H*nb*4 + 256 (the visiting order of the
 * query blocks, chosen from the kept counts on the device, and one word of walk mode). */
size_t abla_sparse_attn_workspace_bytes(const abla_geom* g);

/* Block-sparse attention forward over the kept 64 x 64 blocks.
 * Source: NABLA, Method -- "expansion" (the block mask names which N x N
 * attention blocks are computed) and the block-sparse attention it feeds.
 *
 * For every query token m of block i (fractal order):
 *   O[m] = sum over keys m' in the blocks listed for row i of
 *          softmax_m'(scale * <Q[m], K[m']>) * V[m'].
 * q_r, k_r: [B,H,N,d] fractal order, ABLA_LAYOUT_TOKENS; or, with ABLA_ATTN_QK_ORIGINAL,
 *           the caller's [B,H,N,d] tensors in the original token order (the kernel then
 *           gathers each 64-token block as its 8 runs of 8 tokens, so no reordered copies of
 *           Q and K are needed; the result is the same).
 * v_rt:     fractal order, ABLA_LAYOUT_BLOCK_T; or, with ABLA_ATTN_V_ORIGINAL, the caller's
 *           [B,H,N,d] V in the original token order (bf16: its tiles are staged token-major and
 *           the V^T operand is read with the LDS transpose load).
 * counts, lists: as produced by abla_build_mask (lists ascending).
 * layout_flags: ABLA_ATTN_OUT_ORIGINAL (out in the original token order, else fractal order)
 *      | ABLA_ATTN_QK_ORIGINAL (q_r / k_r given in the original order)
 *      | ABLA_ATTN_V_ORIGINAL (v_rt given in the original order); other bits INVALID.
 * out: [B,H,N,d], same dtype, in the order layout_flags names.
 * lse: [B,H,N] float32 or NULL: natural-log sum of exp(scale * scores) over
 *      the allowed keys, indexed in fractal order; -inf for a row whose list
 *      is empty (its output is 0).
 * scale: 0 means 1/sqrt(d).
 * Arithmetic: bf16 inputs use bf16 matrix-core products with float32
 * accumulation and a float32 online softmax; the probabilities are rounded
 * to bf16 for the value product and the output is rounded once. float32
 * inputs are computed in float32 throughout.
 * workspace: at least abla_sparse_attn_workspace_bytes(g) bytes.
 * Errors: as abla_reorder, plus INVALID for null counts/lists/out, out, lse or the
 * workspace overlapping each other or any input, unknown layout_flags bits, and WORKSPACE. */
enum { ABLA_ATTN_OUT_ORIGINAL = 1, ABLA_ATTN_QK_ORIGINAL = 2, ABLA_ATTN_V_ORIGINAL = 4 };

abla_status abla_sparse_attn_fwd(const abla_geom* g, int32_t dtype, float scale,
                                 const void* q_r, const void* k_r, const void* v_rt,
                                 const int32_t* counts, const int32_t* lists,
                                 void* out, int32_t layout_flags, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* abla_sparse_attn_fwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, results and errors are those of abla_sparse_attn_fwd, computed by the same kernels.
 * Its scratch (the visiting order, abla_sparse_attn_workspace_bytes(g) bytes) lives in a
 * 1 MiB array inside the library, one per GPU, kept until the process ends; the call allocates
 * nothing. Limit: B*H*nb*4 + 256 <= 1 MiB (B*H*nb <= 262080 query blocks), else
 * ABLA_ERR_WORKSPACE before anything is enqueued. Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (different streams, or host threads) race. */
abla_status abla_sparse_attn_fwd_noalloc(const abla_geom* g, int32_t dtype, float scale, const void* q_r,
                                         const void* k_r, const void* v_rt, const int32_t* counts,
                                         const int32_t* lists, void* out, int32_t layout_flags, float* lse,
                                         void* stream);

/* Bytes of scratch abla_sparse_attn_bwd needs: two [B,H,N] float32 rows (D and log2(e)*lse),
 * the column counts [B,H,nb] and lists [B,H,nb,nb] int32 and a [B,H,nb] int32 workgroup
 * visiting order, each rounded up to 256 bytes.
 * (The kernels read q, k, v and dout in their original token order; no copies are made.) */
size_t abla_sparse_attn_bwd_workspace_bytes(const abla_geom* g);

/* Gradients of the block-sparse attention forward (abla_sparse_attn_fwd with the same mask).
 * Source: NABLA, Results -- the mask is used in training as well (forward and backward through
 * the same block mask). With S = scale * Q K^T on the kept blocks, P its row softmax, O = P V:
 *   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 * q, k, v, o, dout: [B,H,N,d] of `dtype` (bf16 or float32) in the ORIGINAL token order (o is
 *   the forward's output, dout the incoming gradient).
 * lse: [B,H,N] float32 in fractal order, as written by abla_sparse_attn_fwd for the same inputs
 *   (natural log); P is recomputed from it.
 * mask_words, counts, lists: the mask of abla_build_mask (words and lists must agree).
 * dq, dk, dv: [B,H,N,d] outputs of `dtype` in the original order; no overlap with each other or
 *   the inputs. Rows of dq whose block keeps nothing are 0; keys no block keeps get dk = dv = 0.
 * scale: 0 means 1/sqrt(d); it must equal the forward's.
 * Arithmetic: bf16 inputs use bf16 matrix-core products with float32 accumulation; P and dS are
 *   rounded to bf16 for the products, D is summed in float32, the outputs are rounded once.
 *   float32 inputs are computed in float32 throughout.
 * workspace: at least abla_sparse_attn_bwd_workspace_bytes(g) bytes.
 * Errors: INVALID for null pointers, NaN/negative scale, unknown dtype, an output or the
 * workspace overlapping another output or any input;
 * UNSUPPORTED for nb > 4096 and the geometry limits of abla_reorder;
 * WORKSPACE if the workspace is missing or too small. */
abla_status abla_sparse_attn_bwd(const abla_geom* g, int32_t dtype, float scale, const void* q, const void* k,
                                 const void* v, const void* o, const void* dout, const float* lse,
                                 const uint32_t* mask_words, const int32_t* counts, const int32_t* lists,
                                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Static, NUL-terminated description of a status code. */
const char* abla_status_str(int32_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t abla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ABLA_H */
