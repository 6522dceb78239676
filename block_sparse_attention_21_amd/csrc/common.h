// Internal declarations shared by the abla kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "abla.h"

namespace abla {

// Only 8 x 8 patches (64-token blocks) are implemented.
constexpr int kP = 8;
constexpr int kBlock = 64;
constexpr int kMaxBlocks = 4096;  // per-row limit of the mask builder (one LDS-resident row)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// Geometry in the form the kernels take it (plain ints; products are formed in 64 bits).
struct KGeom {
  int B, H, T, Hs, Ws, d;
  int nbh, nbw, nb;
  long long N;  // tokens per (b, h)
};

inline KGeom make_kgeom(const abla_geom& g) {
  KGeom k;
  k.B = (int)g.B; k.H = (int)g.H; k.T = (int)g.T; k.Hs = (int)g.Hs; k.Ws = (int)g.Ws; k.d = (int)g.d;
  k.nbh = (int)(g.Hs / g.P); k.nbw = (int)(g.Ws / g.P);
  k.nb = (int)(g.T * k.nbh * k.nbw);
  k.N = g.T * g.Hs * g.Ws;
  return k;
}

// Original-order index of the token at position r (0..63) of fractal block i.
__device__ __forceinline__ long long token_of(const KGeom& g, int i, int r) {
  const int per_frame = g.nbh * g.nbw;
  const int t = i / per_frame;
  const int rem = i - t * per_frame;
  const int hp = rem / g.nbw;
  const int wp = rem - hp * g.nbw;
  const int y = hp * kP + (r >> 3);
  const int x = wp * kP + (r & 7);
  return ((long long)t * g.Hs + y) * g.Ws + x;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Launchers (one per kernel family). Each returns hipGetLastError() after enqueueing.
hipError_t launch_reorder(const KGeom& g, int dtype, int inverse, int layout, const void* x, void* y,
                          double* pooled, hipStream_t s);
hipError_t launch_pool_qk_reorder_v(const KGeom& g, int dtype, const void* q, const void* k, const void* v,
                                    double* qbar, double* kbar, void* vrt, hipStream_t s);
hipError_t launch_build_mask(const KGeom& g, const abla_mask_params& p, const double* qbar, const double* kbar,
                             uint32_t* words, int32_t* counts, int32_t* lists, double* scores, hipStream_t s);
hipError_t launch_sparse_attn(const KGeom& g, int dtype, float scale, const void* q, const void* k,
                              const void* vt, const int32_t* counts, const int32_t* lists, void* out,
                              int out_original_order, int qk_original_order, int v_original_order, float* lse,
                              int32_t* row_order, hipStream_t s);

// Scratch of abla_sparse_attn_fwd_noalloc: a file-scope device array of this many bytes (one
// copy per GPU). Its device address on the current device, looked up once per device.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
hipError_t noalloc_scratch(void** ptr);

// Device scratch of the backward pass, carved out of the caller's workspace
// (see abla_sparse_attn_bwd_workspace_bytes).
struct BwdWorkspace {
  float *D, *L2;                    // [B,H,N] fractal order
  int32_t *col_counts, *col_lists;  // [B,H,nb], [B,H,nb,nb]
  int32_t* order;                   // [B,H,nb] workgroup visiting order (dQ, then dK/dV)
  int32_t* tail_cnt;                // one int after the order: items claimed by tail workgroups
};
hipError_t launch_sparse_attn_bwd(const KGeom& g, int dtype, float scale, const void* q, const void* k,
                                  const void* v, const void* o, const void* dout, const float* lse,
                                  const uint32_t* words, const int32_t* counts, const int32_t* lists, void* dq,
                                  void* dk, void* dv, const BwdWorkspace& ws, hipStream_t s);

}  // namespace abla
