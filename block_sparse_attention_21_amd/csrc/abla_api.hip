// C-ABI entry points: argument validation (host only, before anything is
// enqueued) and dispatch to the kernel launchers.
#include <limits.h>
#include <math.h>

#include <initializer_list>

#include "common.h"

using namespace abla;

namespace {

constexpr int kVersion = 200;  // 0.2.0: adds the backward entry points

abla_status check_geom(const abla_geom* g) {
  if (!g) return ABLA_ERR_INVALID;
  if (g->B <= 0 || g->H <= 0 || g->T <= 0 || g->Hs <= 0 || g->Ws <= 0 || g->d <= 0 || g->P <= 0)
    return ABLA_ERR_INVALID;
  if (g->Hs % g->P != 0 || g->Ws % g->P != 0) return ABLA_ERR_INVALID;
  if (g->P != kP) return ABLA_ERR_UNSUPPORTED;
  if (g->d != 64 && g->d != 128) return ABLA_ERR_UNSUPPORTED;
  if (g->B > INT_MAX || g->H > INT_MAX || g->T > INT_MAX || g->Hs > INT_MAX || g->Ws > INT_MAX)
    return ABLA_ERR_UNSUPPORTED;
  const long double nb = (long double)g->T * (g->Hs / g->P) * (g->Ws / g->P);
  if ((long double)g->B * g->H * nb > (long double)INT_MAX) return ABLA_ERR_UNSUPPORTED;  // grid size
  if ((long double)g->T * g->Hs * g->Ws > (long double)INT_MAX) return ABLA_ERR_UNSUPPORTED;  // tokens per head
  if ((long double)g->B * g->H * g->T * g->Hs * g->Ws * g->d > 9.0e18L) return ABLA_ERR_UNSUPPORTED;
  return ABLA_OK;
}

bool valid_dtype(int32_t dt) { return dt == ABLA_F32 || dt == ABLA_BF16; }

int64_t nb_of(const abla_geom* g) { return (int64_t)g->T * (g->Hs / g->P) * (g->Ws / g->P); }

// B*H, and the element count of one [B,H,N,d] tensor, in 64-bit arithmetic.
size_t bh_of(const abla_geom* g) { return (size_t)g->B * (size_t)g->H; }
size_t tok_elems(const abla_geom* g) {
  return bh_of(g) * (size_t)g->T * (size_t)g->Hs * (size_t)g->Ws * (size_t)g->d;
}

size_t tokens_of(const abla_geom* g) { return (size_t)g->T * (size_t)g->Hs * (size_t)g->Ws; }
// Bytes of the mask outputs and of the pooled vectors.
size_t words_bytes(const abla_geom* g) {
  const size_t nb = (size_t)nb_of(g);
  return bh_of(g) * nb * ((nb + 31) / 32) * 4;
}
size_t counts_bytes(const abla_geom* g) { return bh_of(g) * (size_t)nb_of(g) * 4; }
size_t lists_bytes(const abla_geom* g) { return bh_of(g) * (size_t)nb_of(g) * (size_t)nb_of(g) * 4; }
size_t pooled_bytes(const abla_geom* g) { return bh_of(g) * (size_t)nb_of(g) * (size_t)g->d * sizeof(double); }
size_t rows_bytes(const abla_geom* g) { return bh_of(g) * tokens_of(g) * 4; }

bool window_ok(int32_t t, int32_t h, int32_t w) {
  if (t == 0 && h == 0 && w == 0) return true;
  for (int32_t v : {t, h, w})
    if (v <= 0 || v % 2 == 0) return false;
  return true;
}

size_t elem_bytes(int32_t dt) { return dt == ABLA_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

// A device buffer named in an argument check: base pointer and byte length.
struct Span {
  const void* p;
  size_t n;
};

// True if some written span overlaps another written span or a read span (NULL spans and
// empty ones are skipped).
bool conflicts(std::initializer_list<Span> writes, std::initializer_list<Span> reads) {
  for (auto w = writes.begin(); w != writes.end(); ++w) {
    if (!w->p || !w->n) continue;
    for (auto v = w + 1; v != writes.end(); ++v)
      if (v->p && v->n && overlaps(w->p, w->n, v->p, v->n)) return true;
    for (const Span& r : reads)
      if (r.p && r.n && overlaps(w->p, w->n, r.p, r.n)) return true;
  }
  return false;
}

// Every device pointer must be 16-byte aligned: the kernels move 16-byte vectors and issue
// 16-byte buffer loads from these bases. NULL passes (optional arguments are checked apart).
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15u) return false;
  return true;
}

abla_status from_hip(hipError_t e) { return e == hipSuccess ? ABLA_OK : ABLA_ERR_HIP; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Backward scratch: D and L2 ([B,H,N] float32), column counts [B,H,nb], column lists
// [B,H,nb,nb] and the workgroup visiting order [B,H,nb] (int32) followed by one int (the
// counter of the dynamically claimed items), each 256-aligned.
size_t bwd_parts(const abla_geom* g, BwdWorkspace* ws, char* base) {
  const size_t bh = bh_of(g), nb = (size_t)nb_of(g);
  const size_t n = (size_t)g->T * (size_t)g->Hs * (size_t)g->Ws;
  const size_t rows = align256(bh * n * 4);
  const size_t cc = align256(bh * nb * 4), cl = align256(bh * nb * nb * 4);
  if (ws) {
    ws->D = reinterpret_cast<float*>(base);
    ws->L2 = reinterpret_cast<float*>(base + rows);
    ws->col_counts = reinterpret_cast<int32_t*>(base + 2 * rows);
    ws->col_lists = reinterpret_cast<int32_t*>(base + 2 * rows + cc);
    ws->order = reinterpret_cast<int32_t*>(base + 2 * rows + cc + cl);
    ws->tail_cnt = ws->order + bh * nb;
  }
  return 2 * rows + cc + cl + align256(bh * nb * 4 + 4);
}

// Argument checks of the attention forward, all but the scratch: pointers, flags, scale,
// limits, 16-byte alignment, and out / lse overlapping each other or any input.
abla_status check_fwd(const abla_geom* g, int32_t dtype, float scale, const void* q_r, const void* k_r,
                      const void* v_rt, const int32_t* counts, const int32_t* lists, void* out,
                      int32_t layout_flags, float* lse) {
  abla_status st = check_geom(g);
  if (st != ABLA_OK) return st;
  if (!valid_dtype(dtype) || !q_r || !k_r || !v_rt || !counts || !lists || !out) return ABLA_ERR_INVALID;
  if (!aligned16({q_r, k_r, v_rt, counts, lists, out, lse})) return ABLA_ERR_INVALID;
  if (layout_flags & ~(ABLA_ATTN_OUT_ORIGINAL | ABLA_ATTN_QK_ORIGINAL | ABLA_ATTN_V_ORIGINAL))
    return ABLA_ERR_INVALID;
  if (isnan(scale) || scale < 0.f || isinf(scale)) return ABLA_ERR_INVALID;
  if (nb_of(g) > kMaxBlocks) return ABLA_ERR_UNSUPPORTED;
  const size_t bytes = tok_elems(g) * elem_bytes(dtype);
  if (conflicts({{out, bytes}, {lse, lse ? rows_bytes(g) : 0}},
                {{q_r, bytes}, {k_r, bytes}, {v_rt, bytes}, {counts, counts_bytes(g)}, {lists, lists_bytes(g)}}))
    return ABLA_ERR_INVALID;
  return ABLA_OK;
}

abla_status launch_fwd(const abla_geom* g, int32_t dtype, float scale, const void* q_r, const void* k_r,
                       const void* v_rt, const int32_t* counts, const int32_t* lists, void* out,
                       int32_t layout_flags, float* lse, int32_t* scratch, void* stream) {
  const float s = scale > 0.f ? scale : 1.0f / sqrtf((float)g->d);
  return from_hip(launch_sparse_attn(make_kgeom(*g), dtype, s, q_r, k_r, v_rt, counts, lists, out,
                                     (layout_flags & ABLA_ATTN_OUT_ORIGINAL) != 0,
                                     (layout_flags & ABLA_ATTN_QK_ORIGINAL) != 0,
                                     (layout_flags & ABLA_ATTN_V_ORIGINAL) != 0, lse, scratch,
                                     (hipStream_t)stream));
}

}  // namespace

extern "C" {

int32_t abla_version(void) { return kVersion; }

const char* abla_status_str(int32_t status) {
  switch (status) {
    case ABLA_OK: return "ok";
    case ABLA_ERR_INVALID: return "invalid argument";
    case ABLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case ABLA_ERR_WORKSPACE: return "workspace missing or too small";
    case ABLA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

abla_status abla_reorder(const abla_geom* g, int32_t dtype, int32_t inverse, int32_t layout, const void* x,
                         void* y, double* pooled, void* stream) {
  abla_status st = check_geom(g);
  if (st != ABLA_OK) return st;
  if (!valid_dtype(dtype) || !x) return ABLA_ERR_INVALID;
  if (layout != ABLA_LAYOUT_TOKENS && layout != ABLA_LAYOUT_BLOCK_T) return ABLA_ERR_INVALID;
  if (inverse != 0 && inverse != 1) return ABLA_ERR_INVALID;
  if (inverse && (layout != ABLA_LAYOUT_TOKENS || pooled)) return ABLA_ERR_INVALID;
  // y may be NULL only to pool without reordering (forward, token layout, pooled given).
  if (!y && (inverse || layout != ABLA_LAYOUT_TOKENS || !pooled)) return ABLA_ERR_INVALID;
  if (!aligned16({x, y, pooled})) return ABLA_ERR_INVALID;
  const size_t bytes = tok_elems(g) * elem_bytes(dtype);
  if (y && overlaps(x, bytes, y, bytes)) return ABLA_ERR_INVALID;
  if (pooled) {
    const size_t pbytes = bh_of(g) * (size_t)nb_of(g) * (size_t)g->d * sizeof(double);
    if (overlaps(pooled, pbytes, x, bytes) || (y && overlaps(pooled, pbytes, y, bytes))) return ABLA_ERR_INVALID;
  }
  return from_hip(launch_reorder(make_kgeom(*g), dtype, inverse, layout, x, y, pooled, (hipStream_t)stream));
}

abla_status abla_pool_qk_reorder_v(const abla_geom* g, int32_t dtype, const void* q, const void* k, const void* v,
                                   double* qbar, double* kbar, void* v_rt, void* stream) {
  abla_status st = check_geom(g);
  if (st != ABLA_OK) return st;
  if (!valid_dtype(dtype) || !q || !k || !qbar || !kbar || (!v != !v_rt)) return ABLA_ERR_INVALID;
  const bool with_v = v != nullptr;  // else pool q and k only
  if (!aligned16({q, k, qbar, kbar}) || (with_v && !aligned16({v, v_rt}))) return ABLA_ERR_INVALID;
  if ((long double)3 * bh_of(g) * nb_of(g) > (long double)INT_MAX) return ABLA_ERR_UNSUPPORTED;  // grid size
  const size_t bytes = tok_elems(g) * elem_bytes(dtype);
  const size_t pbytes = bh_of(g) * (size_t)nb_of(g) * (size_t)g->d * sizeof(double);
  const size_t vbytes = with_v ? bytes : 0;  // overlaps() of an empty range is false
  // Outputs must overlap no input and no other output.
  const void* ins[3] = {q, k, v};
  for (const void* in : ins)
    if (in && (overlaps(v_rt, vbytes, in, bytes) || overlaps(qbar, pbytes, in, bytes) ||
               overlaps(kbar, pbytes, in, bytes)))
      return ABLA_ERR_INVALID;
  if (overlaps(qbar, pbytes, kbar, pbytes) || overlaps(qbar, pbytes, v_rt, vbytes) ||
      overlaps(kbar, pbytes, v_rt, vbytes))
    return ABLA_ERR_INVALID;
  return from_hip(launch_pool_qk_reorder_v(make_kgeom(*g), dtype, q, k, v, qbar, kbar, v_rt, (hipStream_t)stream));
}

size_t abla_build_mask_workspace_bytes(const abla_geom* g) {
  if (check_geom(g) != ABLA_OK) return 0;
  const int64_t nb = nb_of(g);
  return bh_of(g) * (size_t)nb * (size_t)nb * sizeof(double);
}

abla_status abla_build_mask(const abla_geom* g, const abla_mask_params* p, const double* qbar, const double* kbar,
                            uint32_t* mask_words, int32_t* counts, int32_t* lists, void* workspace,
                            size_t workspace_bytes, void* stream) {
  abla_status st = check_geom(g);
  if (st != ABLA_OK) return st;
  if (!p || !mask_words || !counts) return ABLA_ERR_INVALID;
  if (p->mode != ABLA_MASK_CDF && p->mode != ABLA_MASK_DYN && p->mode != ABLA_MASK_STATIC) return ABLA_ERR_INVALID;
  const bool scored = p->mode != ABLA_MASK_STATIC;
  if (scored && (!qbar || !kbar)) return ABLA_ERR_INVALID;
  if (!aligned16({qbar, kbar, mask_words, counts, lists, workspace})) return ABLA_ERR_INVALID;
  if (!scored && !(p->gamma >= 0.0 && p->gamma <= 1.0 && p->lambda >= 0.0 && p->lambda <= 1.0))
    return ABLA_ERR_INVALID;  // also rejects NaN
  if (p->cut != ABLA_CUT_RADIX && p->cut != ABLA_CUT_BITONIC && p->cut != ABLA_CUT_RADIX_WIDE)
    return ABLA_ERR_INVALID;
  if (isnan(p->thr) || isnan(p->tau) || isnan(p->pool_scale) || p->pool_scale < 0.0 || isinf(p->pool_scale))
    return ABLA_ERR_INVALID;
  if (!window_ok(p->sta_t, p->sta_h, p->sta_w)) return ABLA_ERR_INVALID;
  if (nb_of(g) > kMaxBlocks) return ABLA_ERR_UNSUPPORTED;
  if (scored && (!workspace || workspace_bytes < abla_build_mask_workspace_bytes(g))) return ABLA_ERR_WORKSPACE;
  // Outputs (and the scratch) overlap neither each other nor the pooled vectors.
  const size_t pb = scored ? pooled_bytes(g) : 0;
  if (conflicts({{mask_words, words_bytes(g)}, {counts, counts_bytes(g)}, {lists, lists ? lists_bytes(g) : 0},
                 {workspace, scored ? abla_build_mask_workspace_bytes(g) : 0}},
                {{qbar, pb}, {kbar, pb}}))
    return ABLA_ERR_INVALID;
  return from_hip(launch_build_mask(make_kgeom(*g), *p, qbar, kbar, mask_words, counts, lists,
                                    static_cast<double*>(workspace), (hipStream_t)stream));
}

size_t abla_sparse_attn_workspace_bytes(const abla_geom* g) {
  if (check_geom(g) != ABLA_OK) return 0;
  // Visiting order (at most nb ints per (b, h)), then the walk mode and the counter of the
  // dynamically claimed items (one int each), padded to 256 bytes.
  return bh_of(g) * (size_t)nb_of(g) * sizeof(int32_t) + 256;
}

abla_status abla_sparse_attn_fwd(const abla_geom* g, int32_t dtype, float scale, const void* q_r,
                                 const void* k_r, const void* v_rt, const int32_t* counts, const int32_t* lists,
                                 void* out, int32_t layout_flags, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  abla_status st = check_fwd(g, dtype, scale, q_r, k_r, v_rt, counts, lists, out, layout_flags, lse);
  if (st != ABLA_OK) return st;
  if (!aligned16({workspace})) return ABLA_ERR_INVALID;
  if (!workspace || workspace_bytes < abla_sparse_attn_workspace_bytes(g)) return ABLA_ERR_WORKSPACE;
  // The scratch overlaps neither an output nor any input.
  const size_t bytes = tok_elems(g) * elem_bytes(dtype);
  if (conflicts({{workspace, abla_sparse_attn_workspace_bytes(g)}, {out, bytes}, {lse, lse ? rows_bytes(g) : 0}},
                {{q_r, bytes}, {k_r, bytes}, {v_rt, bytes}, {counts, counts_bytes(g)}, {lists, lists_bytes(g)}}))
    return ABLA_ERR_INVALID;
  return launch_fwd(g, dtype, scale, q_r, k_r, v_rt, counts, lists, out, layout_flags, lse,
                    static_cast<int32_t*>(workspace), stream);
}

abla_status abla_sparse_attn_fwd_noalloc(const abla_geom* g, int32_t dtype, float scale, const void* q_r,
                                         const void* k_r, const void* v_rt, const int32_t* counts,
                                         const int32_t* lists, void* out, int32_t layout_flags, float* lse,
                                         void* stream) {
  abla_status st = check_fwd(g, dtype, scale, q_r, k_r, v_rt, counts, lists, out, layout_flags, lse);
  if (st != ABLA_OK) return st;
  if (abla_sparse_attn_workspace_bytes(g) > kNoAllocScratchBytes) return ABLA_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (noalloc_scratch(&scratch) != hipSuccess) return ABLA_ERR_HIP;
  return launch_fwd(g, dtype, scale, q_r, k_r, v_rt, counts, lists, out, layout_flags, lse,
                    static_cast<int32_t*>(scratch), stream);
}

size_t abla_sparse_attn_bwd_workspace_bytes(const abla_geom* g) {
  if (check_geom(g) != ABLA_OK) return 0;
  return bwd_parts(g, nullptr, nullptr);
}

abla_status abla_sparse_attn_bwd(const abla_geom* g, int32_t dtype, float scale, const void* q, const void* k,
                                 const void* v, const void* o, const void* dout, const float* lse,
                                 const uint32_t* mask_words, const int32_t* counts, const int32_t* lists,
                                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  abla_status st = check_geom(g);
  if (st != ABLA_OK) return st;
  if (!valid_dtype(dtype)) return ABLA_ERR_INVALID;
  if (!q || !k || !v || !o || !dout || !lse || !mask_words || !counts || !lists || !dq || !dk || !dv)
    return ABLA_ERR_INVALID;
  if (!aligned16({q, k, v, o, dout, lse, mask_words, counts, lists, dq, dk, dv, workspace})) return ABLA_ERR_INVALID;
  if (isnan(scale) || scale < 0.f || isinf(scale)) return ABLA_ERR_INVALID;
  if (nb_of(g) > kMaxBlocks) return ABLA_ERR_UNSUPPORTED;
  const size_t bytes = tok_elems(g) * elem_bytes(dtype);
  const void* ins[5] = {q, k, v, o, dout};
  void* outs[3] = {dq, dk, dv};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 5; ++b)
      if (overlaps(outs[a], bytes, ins[b], bytes)) return ABLA_ERR_INVALID;
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], bytes, outs[b], bytes)) return ABLA_ERR_INVALID;
  }
  if (!workspace || workspace_bytes < abla_sparse_attn_bwd_workspace_bytes(g)) return ABLA_ERR_WORKSPACE;
  // The scratch overlaps no input and no output; the outputs overlap none of the mask inputs.
  if (conflicts({{dq, bytes}, {dk, bytes}, {dv, bytes}, {workspace, abla_sparse_attn_bwd_workspace_bytes(g)}},
                {{q, bytes}, {k, bytes}, {v, bytes}, {o, bytes}, {dout, bytes}, {lse, rows_bytes(g)},
                 {mask_words, words_bytes(g)}, {counts, counts_bytes(g)}, {lists, lists_bytes(g)}}))
    return ABLA_ERR_INVALID;
  BwdWorkspace ws;
  bwd_parts(g, &ws, static_cast<char*>(workspace));
  const float s = scale > 0.f ? scale : 1.0f / sqrtf((float)g->d);
  return from_hip(launch_sparse_attn_bwd(make_kgeom(*g), dtype, s, q, k, v, o, dout, lse, mask_words, counts, lists,
                                         dq, dk, dv, ws, (hipStream_t)stream));
}

}  // extern "C"
