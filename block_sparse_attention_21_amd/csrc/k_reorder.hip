// Fractal reordering of the token axis, fused with block mean-pooling.
//
// NABLA, Method: "Fractal Flattening" makes the tokens of each P x P patch one
// contiguous run while frames stay outermost; "down-sampling" mean-pools Q
// and K over those 64-token blocks.
//
// One workgroup moves one 64-token block. The source block is 8 runs of 8
// tokens (one run per patch row), each run d*sizeof(E)*8 bytes contiguous in
// the original order; the destination block is contiguous. Every thread moves
// 16-byte chunks: consecutive threads take consecutive chunks of a token row,
// so both the reads and the writes of a wave cover whole rows. The pooled
// mean is accumulated in float64 in a fixed order (per thread over its rows,
// then over threads): exact for bf16 inputs and deterministic. HBM-bound: read
// + write of the tensor plus d*8 bytes of pooled output per block. Without an
// output tensor the pass only pools (read + pooled output), for consumers that
// read the tensor in its original order themselves.
#include "common.h"

namespace abla {
namespace {

constexpr int kThreads = 256;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <typename E, int D>
struct Shape {
  static constexpr int EPC = 16 / sizeof(E);         // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                 // chunks per token row
  static constexpr int RPP = kThreads / CPR;          // token rows per pass
  static constexpr int PASSES = kBlock / RPP;         // passes over the 64 rows
  static_assert(kThreads % CPR == 0 && kBlock % RPP == 0, "unsupported head dim");
};

template <typename E>
__device__ __forceinline__ void add_chunk(double* acc, const uint4& v);

template <>
__device__ __forceinline__ void add_chunk<float>(double* acc, const uint4& v) {
  acc[0] += (double)__uint_as_float(v.x);
  acc[1] += (double)__uint_as_float(v.y);
  acc[2] += (double)__uint_as_float(v.z);
  acc[3] += (double)__uint_as_float(v.w);
}

template <>
__device__ __forceinline__ void add_chunk<uint16_t>(double* acc, const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc[2 * k] += (double)__uint_as_float(w[k] << 16);
    acc[2 * k + 1] += (double)__uint_as_float(w[k] & 0xFFFF0000u);
  }
}

// LDS bytes of one block move: the channel-major transpose tile, or the pooling partials.
template <typename E, int D>
constexpr int kSmemBytes = (kBlock * D * (int)sizeof(E)) > (kThreads * Shape<E, D>::EPC * 8)
                               ? kBlock * D * (int)sizeof(E)
                               : kThreads * Shape<E, D>::EPC * 8;

// Forward, one 64-token block `blk` (over B*H*nb): original order -> fractal order (token
// rows, or channel-major blocks); with STORE = false only the pooled means are written.
// smem: kSmemBytes<E, D> bytes, 16-byte aligned.
template <typename E, int D, bool POOL, bool BLOCK_T, bool STORE = true>
__device__ __forceinline__ void reorder_block(const E* __restrict__ x, E* __restrict__ y, double* __restrict__ pooled,
                                              const KGeom& g, int blk, char* smem) {
  using S = Shape<E, D>;
  // Channel-major transpose tile: token row r holds its D elements as CPR 16-byte chunks, chunk
  // cc stored at position cc ^ ((r / EPC) % CPR). The gathers below (EPC tokens of one channel
  // per lane, one group of EPC tokens per lane of a run of kBlock/EPC lanes) then hit distinct
  // banks, and the 16-byte row writes stay conflict-free.
  E* tile = reinterpret_cast<E*>(smem);
  double* red = reinterpret_cast<double*>(smem);

  const int bh = blk / g.nb;
  const int i = blk - bh * g.nb;
  const int t = threadIdx.x;
  const int cc = t % S::CPR;
  const int r0 = t / S::CPR;
  const E* xh = x + (long long)bh * g.N * D;

  double acc[S::EPC];
#pragma unroll
  for (int e = 0; e < S::EPC; ++e) acc[e] = 0.0;

#pragma unroll
  for (int p = 0; p < S::PASSES; ++p) {
    const int r = r0 + p * S::RPP;
    const long long n = token_of(g, i, r);
    // Each input chunk is read exactly once: a non-temporal load (nt) streams it past the caches
    // instead of displacing lines the next kernels reuse (first step 480p 0.085 -> 0.071 ms,
    // 720p 0.614 -> 0.587 ms).
    const u32x4_t raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(xh + n * D + cc * S::EPC));
    const uint4 v = make_uint4(raw.x, raw.y, raw.z, raw.w);
    if constexpr (BLOCK_T) {
      *reinterpret_cast<uint4*>(&tile[r * D + ((cc ^ ((r / S::EPC) % S::CPR)) * S::EPC)]) = v;
    } else if constexpr (STORE) {
      *reinterpret_cast<uint4*>(y + ((long long)bh * g.N + (long long)i * kBlock + r) * D + cc * S::EPC) = v;
    }
    if constexpr (POOL) add_chunk<E>(acc, v);
  }

  if constexpr (BLOCK_T) {
    __syncthreads();
    // Output block is [D][64]; chunk oc covers tokens grp*EPC .. +EPC-1 of channel c, with
    // grp = oc % G and c = oc / G (G = 64 / EPC): each run of G lanes writes one channel's
    // whole 128- or 256-byte row.
    constexpr int G = kBlock / S::EPC;
    constexpr int OUT_CHUNKS = D * kBlock / S::EPC;
    E* yb = y + ((long long)bh * g.nb + i) * D * kBlock;
#pragma unroll
    for (int oc = t; oc < OUT_CHUNKS; oc += kThreads) {
      const int grp = oc % G;
      const int c = oc / G;
      const int pos = ((c / S::EPC) ^ (grp % S::CPR)) * S::EPC + c % S::EPC;  // rows grp*EPC+e share r/EPC = grp
      E vals[S::EPC];
#pragma unroll
      for (int e = 0; e < S::EPC; ++e) vals[e] = tile[(grp * S::EPC + e) * D + pos];
      uint4 v;
      __builtin_memcpy(&v, vals, 16);
      *reinterpret_cast<uint4*>(yb + c * kBlock + grp * S::EPC) = v;
    }
  }

  if constexpr (POOL) {
    if constexpr (BLOCK_T) __syncthreads();  // the partials reuse the transpose tile's LDS
#pragma unroll
    for (int e = 0; e < S::EPC; ++e) red[t * S::EPC + e] = acc[e];
    __syncthreads();
    if (t < D) {
      const int c = t;
      const int ccc = c / S::EPC, e = c % S::EPC;
      double s = 0.0;
      for (int rr = 0; rr < S::RPP; ++rr) s += red[(rr * S::CPR + ccc) * S::EPC + e];
      pooled[((long long)bh * g.nb + i) * D + c] = s * (1.0 / kBlock);
    }
  }
}

template <typename E, int D, bool POOL, bool BLOCK_T, bool STORE = true>
__global__ __launch_bounds__(kThreads) void k_reorder_fwd(const E* __restrict__ x, E* __restrict__ y,
                                                          double* __restrict__ pooled, KGeom g, int first) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes<E, D>];
  reorder_block<E, D, POOL, BLOCK_T, STORE>(x, y, pooled, g, first + (int)blockIdx.x, smem);
}

// The layer's first step in one launch: workgroup 3b pools Q's block b, 3b+1 pools K's (both
// read in the original order, not copied) and 3b+2 reorders V's into a channel-major block,
// b < n = B*H*nb (workgroup `first` + blockIdx.x of the whole grid, which larger inputs split
// into several launches). One grid instead of three saves two launch gaps and two ramp-down tails;
// interleaving the read-only pooling with the read-write reorder (rather than Q, then K,
// then V) measured 5% faster at 480p and 720p (5.6 TB/s for the stage). With WITH_V false
// the grid is 2*n workgroups pooling Q (2b) and K (2b+1) only.
template <typename E, int D, bool WITH_V>
__global__ __launch_bounds__(kThreads) void k_pool_qk_reorder_v(const E* __restrict__ q, const E* __restrict__ k,
                                                                const E* __restrict__ v, double* __restrict__ qbar,
                                                                double* __restrict__ kbar, E* __restrict__ vrt,
                                                                KGeom g, int first) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes<E, D>];
  constexpr int kParts = WITH_V ? 3 : 2;
  const int wg = first + (int)blockIdx.x;
  const int which = wg % kParts;
  const int blk = wg / kParts;
  if (which == 0)
    reorder_block<E, D, true, false, false>(q, nullptr, qbar, g, blk, smem);
  else if (which == 1)
    reorder_block<E, D, true, false, false>(k, nullptr, kbar, g, blk, smem);
  else if constexpr (WITH_V)
    reorder_block<E, D, false, true, true>(v, vrt, nullptr, g, blk, smem);
}

// Inverse: fractal order (token rows) -> original order.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_reorder_inv(const E* __restrict__ x, E* __restrict__ y, KGeom g,
                                                          int first) {
  using S = Shape<E, D>;
  const int blk = first + (int)blockIdx.x;
  const int bh = blk / g.nb;
  const int i = blk - bh * g.nb;
  const int t = threadIdx.x;
  const int cc = t % S::CPR;
  const int r0 = t / S::CPR;
  E* yh = y + (long long)bh * g.N * D;
#pragma unroll
  for (int p = 0; p < S::PASSES; ++p) {
    const int r = r0 + p * S::RPP;
    const uint4 v = *reinterpret_cast<const uint4*>(x + ((long long)bh * g.N + (long long)i * kBlock + r) * D +
                                                    cc * S::EPC);
    *reinterpret_cast<uint4*>(yh + token_of(g, i, r) * D + cc * S::EPC) = v;
  }
}

// Grids of at most 2^22 workgroups: a grid dimension holds at most 2^32 work-items, and the
// block count B*H*nb (times 3 for the first step) may exceed 2^24.
constexpr int kChunk = 1 << 22;

template <typename E, int D>
hipError_t dispatch(const KGeom& g, int inverse, int layout, const void* x, void* y, double* pooled,
                    hipStream_t s) {
  const int total = (int)(g.B * g.H * g.nb);
  const E* xi = static_cast<const E*>(x);
  E* yo = static_cast<E*>(y);
  for (int first = 0; first < total; first += kChunk) {
    const dim3 grid((unsigned)min(kChunk, total - first));
    if (inverse) {
      k_reorder_inv<E, D><<<grid, kThreads, 0, s>>>(xi, yo, g, first);
    } else if (layout == ABLA_LAYOUT_BLOCK_T) {
      if (pooled)
        k_reorder_fwd<E, D, true, true><<<grid, kThreads, 0, s>>>(xi, yo, pooled, g, first);
      else
        k_reorder_fwd<E, D, false, true><<<grid, kThreads, 0, s>>>(xi, yo, nullptr, g, first);
    } else if (!yo) {
      k_reorder_fwd<E, D, true, false, false><<<grid, kThreads, 0, s>>>(xi, nullptr, pooled, g, first);
    } else {
      if (pooled)
        k_reorder_fwd<E, D, true, false><<<grid, kThreads, 0, s>>>(xi, yo, pooled, g, first);
      else
        k_reorder_fwd<E, D, false, false><<<grid, kThreads, 0, s>>>(xi, yo, nullptr, g, first);
    }
  }
  return hipGetLastError();
}

template <typename E, int D>
hipError_t dispatch_qkv(const KGeom& g, const void* q, const void* k, const void* v, double* qbar, double* kbar,
                        void* vrt, hipStream_t s) {
  const bool with_v = v != nullptr;
  const int total = (int)((with_v ? 3LL : 2LL) * g.B * g.H * g.nb);
  for (int first = 0; first < total; first += kChunk) {
    const dim3 grid((unsigned)min(kChunk, total - first));
    if (with_v)
      k_pool_qk_reorder_v<E, D, true><<<grid, kThreads, 0, s>>>(static_cast<const E*>(q), static_cast<const E*>(k),
                                                                static_cast<const E*>(v), qbar, kbar,
                                                                static_cast<E*>(vrt), g, first);
    else
      k_pool_qk_reorder_v<E, D, false><<<grid, kThreads, 0, s>>>(static_cast<const E*>(q), static_cast<const E*>(k),
                                                                 nullptr, qbar, kbar, nullptr, g, first);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool_qk_reorder_v(const KGeom& g, int dtype, const void* q, const void* k, const void* v,
                                    double* qbar, double* kbar, void* vrt, hipStream_t s) {
  if (dtype == ABLA_F32) {
    return g.d == 64 ? dispatch_qkv<float, 64>(g, q, k, v, qbar, kbar, vrt, s)
                     : dispatch_qkv<float, 128>(g, q, k, v, qbar, kbar, vrt, s);
  }
  return g.d == 64 ? dispatch_qkv<uint16_t, 64>(g, q, k, v, qbar, kbar, vrt, s)
                   : dispatch_qkv<uint16_t, 128>(g, q, k, v, qbar, kbar, vrt, s);
}

hipError_t launch_reorder(const KGeom& g, int dtype, int inverse, int layout, const void* x, void* y,
                          double* pooled, hipStream_t s) {
  if (dtype == ABLA_F32) {
    return g.d == 64 ? dispatch<float, 64>(g, inverse, layout, x, y, pooled, s)
                     : dispatch<float, 128>(g, inverse, layout, x, y, pooled, s);
  }
  return g.d == 64 ? dispatch<uint16_t, 64>(g, inverse, layout, x, y, pooled, s)
                   : dispatch<uint16_t, 128>(g, inverse, layout, x, y, pooled, s);
}

}  // namespace abla
