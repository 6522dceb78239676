// Matrix-core rate probes for the benchmark: loops of independent MFMAs with no memory traffic,
// timed on the board to give the sustained bf16 (v_mfma_f32_32x32x16_bf16) and float32
// (v_mfma_f32_32x32x2_f32) rates that the attention kernels are compared against, next to the
// datasheet peaks. Not part of the attention path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "abla_probe.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kChains = 4;  // independent accumulators per wave: back-to-back issue

// Operands vary with the lane (not constant-folded, and not all-zero: zeros draw less power).
template <bool BF16>
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f32x16_t acc[kChains];
#pragma unroll
  for (int u = 0; u < kChains; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
  if constexpr (BF16) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (float)(lane + 3 * i + 1));
      b[i] = (__bf16)(0.001f * (float)(2 * lane - i + 7));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int u = 0; u < kChains; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
  } else {
    const float a = 0.001f * (float)(lane + 1), b = 0.001f * (float)(2 * lane + 7);
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int u = 0; u < kChains; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[u], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kChains; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[u][r];
  if (s == -1.0f) sink[blockIdx.x] = s;  // sums of positive products: never true; keeps the loop
}

}  // namespace

extern "C" {

int32_t abla_probe_mfma(int32_t kind, int32_t grid, int32_t iters, float* sink, void* stream) {
  if (grid <= 0 || iters <= 0 || !sink || (kind != 0 && kind != 1)) return 1;
  if (kind == 0)
    k_mfma_loop<true><<<dim3((unsigned)grid), 256, 0, (hipStream_t)stream>>>(iters, sink);
  else
    k_mfma_loop<false><<<dim3((unsigned)grid), 256, 0, (hipStream_t)stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

double abla_probe_mfma_flops(int32_t kind, int32_t grid, int32_t iters) {
  const double per = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 2;  // one MFMA
  return per * kChains * 4.0 /* waves */ * (double)grid * (double)iters;
}

}  // extern "C"
