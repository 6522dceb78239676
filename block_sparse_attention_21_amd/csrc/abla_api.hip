// C-ABI entry points: argument validation (host only, before anything is
// enqueued) and dispatch to the kernel launchers.
#include <limits.h>
#include <math.h>

#include "common.h"

using namespace abla;

namespace {

constexpr int kVersion = 100;  // 0.1.0

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
  if ((long double)g->B * g->H * g->T * g->Hs * g->Ws * g->d > 9.0e18L) return ABLA_ERR_UNSUPPORTED;
  return ABLA_OK;
}

bool valid_dtype(int32_t dt) { return dt == ABLA_F32 || dt == ABLA_BF16; }

int64_t nb_of(const abla_geom* g) { return g->T * (g->Hs / g->P) * (g->Ws / g->P); }

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

abla_status from_hip(hipError_t e) { return e == hipSuccess ? ABLA_OK : ABLA_ERR_HIP; }

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
  if (!valid_dtype(dtype) || !x || !y) return ABLA_ERR_INVALID;
  if (layout != ABLA_LAYOUT_TOKENS && layout != ABLA_LAYOUT_BLOCK_T) return ABLA_ERR_INVALID;
  if (inverse != 0 && inverse != 1) return ABLA_ERR_INVALID;
  if (inverse && (layout != ABLA_LAYOUT_TOKENS || pooled)) return ABLA_ERR_INVALID;
  const size_t bytes = (size_t)(g->B * g->H * g->T * g->Hs * g->Ws * g->d) * elem_bytes(dtype);
  if (overlaps(x, bytes, y, bytes)) return ABLA_ERR_INVALID;
  if (pooled) {
    const size_t pbytes = (size_t)(g->B * g->H * nb_of(g) * g->d) * sizeof(double);
    if (overlaps(pooled, pbytes, x, bytes) || overlaps(pooled, pbytes, y, bytes)) return ABLA_ERR_INVALID;
  }
  return from_hip(launch_reorder(make_kgeom(*g), dtype, inverse, layout, x, y, pooled, (hipStream_t)stream));
}

size_t abla_build_mask_workspace_bytes(const abla_geom* g) {
  if (check_geom(g) != ABLA_OK) return 0;
  const int64_t nb = nb_of(g);
  return (size_t)(g->B * g->H * nb * nb) * sizeof(double);
}

abla_status abla_build_mask(const abla_geom* g, const abla_mask_params* p, const double* qbar, const double* kbar,
                            uint32_t* mask_words, int32_t* counts, int32_t* lists, void* workspace,
                            size_t workspace_bytes, void* stream) {
  abla_status st = check_geom(g);
  if (st != ABLA_OK) return st;
  if (!p || !qbar || !kbar || !mask_words || !counts) return ABLA_ERR_INVALID;
  if (p->mode != ABLA_MASK_CDF && p->mode != ABLA_MASK_DYN) return ABLA_ERR_INVALID;
  if (p->cut != ABLA_CUT_RADIX && p->cut != ABLA_CUT_BITONIC) return ABLA_ERR_INVALID;
  if (isnan(p->thr) || isnan(p->tau) || isnan(p->pool_scale) || p->pool_scale < 0.0 || isinf(p->pool_scale))
    return ABLA_ERR_INVALID;
  if (!window_ok(p->sta_t, p->sta_h, p->sta_w)) return ABLA_ERR_INVALID;
  if (nb_of(g) > kMaxBlocks) return ABLA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < abla_build_mask_workspace_bytes(g)) return ABLA_ERR_WORKSPACE;
  return from_hip(launch_build_mask(make_kgeom(*g), *p, qbar, kbar, mask_words, counts, lists,
                                    static_cast<double*>(workspace), (hipStream_t)stream));
}

size_t abla_sparse_attn_workspace_bytes(const abla_geom* g) {
  if (check_geom(g) != ABLA_OK) return 0;
  // Visiting order (at most nb ints per (b, h)), then one int of walk mode, padded to 256 bytes.
  return (size_t)(g->B * g->H * nb_of(g)) * sizeof(int32_t) + 256;
}

abla_status abla_sparse_attn_fwd(const abla_geom* g, int32_t dtype, float scale, const void* q_r,
                                 const void* k_r, const void* v_rt, const int32_t* counts, const int32_t* lists,
                                 void* out, int32_t out_original_order, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  abla_status st = check_geom(g);
  if (st != ABLA_OK) return st;
  if (!valid_dtype(dtype) || !q_r || !k_r || !v_rt || !counts || !lists || !out) return ABLA_ERR_INVALID;
  if (isnan(scale) || scale < 0.f || isinf(scale)) return ABLA_ERR_INVALID;
  if (nb_of(g) > kMaxBlocks) return ABLA_ERR_UNSUPPORTED;
  const size_t bytes = (size_t)(g->B * g->H * g->T * g->Hs * g->Ws * g->d) * elem_bytes(dtype);
  if (overlaps(out, bytes, q_r, bytes) || overlaps(out, bytes, k_r, bytes) || overlaps(out, bytes, v_rt, bytes))
    return ABLA_ERR_INVALID;
  if (!workspace || workspace_bytes < abla_sparse_attn_workspace_bytes(g)) return ABLA_ERR_WORKSPACE;
  const float s = scale > 0.f ? scale : 1.0f / sqrtf((float)g->d);
  return from_hip(launch_sparse_attn(make_kgeom(*g), dtype, s, q_r, k_r, v_rt, counts, lists, out,
                                     out_original_order != 0, lse, static_cast<int32_t*>(workspace),
                                     (hipStream_t)stream));
}

}  // extern "C"
