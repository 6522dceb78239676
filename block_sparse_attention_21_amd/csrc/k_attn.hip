// Block-sparse attention forward over the kept 64 x 64 blocks.
//
// NABLA, Method: "expansion" -- the block mask names which N x N attention
// blocks are computed; everything else is skipped. For query block i the
// kernel walks the ascending list of kept key blocks with an online softmax.
//
// bf16 path (k_attn_bf16), one workgroup per query block, two waves of 32
// query rows each, gfx950 MFMA v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T   A = K rows from LDS, B = Q rows held in registers. The
//                 result puts one query per lane (lanes l and l^32 share it),
//                 so the row max / sum stay in-lane plus one permlane swap.
//   O^T += V^T P^T  A = V^T rows from LDS (V is stored channel-major per
//                 block by the reorder pass), B = the probabilities exactly as
//                 the S^T registers hold them, rounded to bf16. The key order
//                 of the S^T result (keys 0-3,8-11 in lanes 0-31, 4-7,12-15 in
//                 lanes 32-63 of each 16-key step) is matched by the V^T read.
// K and V^T tiles go global -> LDS directly (global_load_lds_dwordx4), with a
// per-row XOR swizzle of 16-byte chunks so the MFMA operand reads are free of
// bank conflicts. Rows are visited longest-first within each head (row_order)
// so the long rows of the kept-count distribution do not form the tail.
//
// float32 path (k_attn_f32): plain FMA arithmetic, two threads per query row.
#include <math.h>

#include "common.h"

namespace abla {
namespace {

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;
  const int32_t* counts;
  const int32_t* lists;
  const int32_t* order;
  uint16_t* out;
  float* lse;
  KGeom g;
  float c2;     // scale * log2(e)
  float scale;
  int orig;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int D>
struct Tile {
  static constexpr int KBYTES = kBlock * D * 2;   // K tile, token-major
  static constexpr int VBYTES = D * kBlock * 2;   // V^T tile, channel-major
  static constexpr int BYTES = KBYTES + VBYTES;
  static constexpr int KCH = D / 8;               // 16-byte chunks per K row
  static constexpr int KUNITS = KBYTES / 16;
  static constexpr int VUNITS = VBYTES / 16;
  static constexpr int LOADS_PER_WAVE = (KUNITS + VUNITS) / 128;
};

// Swizzled chunk position of logical 16-byte chunk ch in K row r.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

template <int D>
__device__ __forceinline__ void issue_tile_loads(char* stage, const uint16_t* kblk, const uint16_t* vblk, int w,
                                                 int lane) {
  using TT = Tile<D>;
#pragma unroll
  for (int it = 0; it < TT::KUNITS / 128; ++it) {
    const int u0 = w * 64 + it * 128;
    const int u = u0 + lane;
    const int r = u / TT::KCH, pc = u % TT::KCH;
    const int ch = pc ^ k_swz<D>(r);
    __builtin_amdgcn_global_load_lds(kblk + r * D + ch * 8, (lds_ptr_t)(stage + u0 * 16), 16, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < TT::VUNITS / 128; ++it) {
    const int u0 = w * 64 + it * 128;
    const int u = u0 + lane;
    const int dd = u >> 3, pc = u & 7;
    const int ch = pc ^ v_swz(dd);
    __builtin_amdgcn_global_load_lds(vblk + dd * kBlock + ch * 8, (lds_ptr_t)(stage + TT::KBYTES + u0 * 16), 16, 0,
                                     0);
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float swap_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bf16(AttnArgs a) {
  using TT = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char smem[TT::BYTES];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const KGeom& g = a.g;
  const int nb = g.nb;
  const int bh = blockIdx.x / nb;
  const int pos = blockIdx.x - bh * nb;
  const int i = a.order ? a.order[(long long)bh * nb + pos] : pos;
  const long long row = (long long)bh * nb + i;
  const int cnt = min(max(a.counts[row], 0), nb);
  const int32_t* lst = a.lists + row * nb;
  const int q_local = w * 32 + (lane & 31);
  const int hi = lane >> 5;

  // Q operand: lane holds Q[q_local][ks*16 + 8*hi .. +7] for every k-step.
  bf16x8_t qv[D / 16];
  {
    const uint16_t* qrow = a.q + ((long long)bh * g.N + (long long)i * kBlock + q_local) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qv[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
  }

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const uint16_t* kbase = a.k + (long long)bh * g.N * D;
  const uint16_t* vbase = a.vt + (long long)bh * nb * D * kBlock;
  const char* ks_lds = smem;
  const char* vs_lds = smem + TT::KBYTES;

  for (int tt = 0; tt < cnt; ++tt) {
    const int j = min(max(lst[tt], 0), nb - 1);
    issue_tile_loads<D>(smem, kbase + (long long)j * kBlock * D, vbase + (long long)j * D * kBlock, w, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // S^T = K Q^T for the two 32-key halves of the tile.
    f32x16_t sacc[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kh][r] = 0.f;
      const int krow = kh * 32 + (lane & 31);
      const char* rowp = ks_lds + krow * (D * 2);
      const int swz = k_swz<D>(krow);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int ch = (ks * 2 + hi) ^ swz;
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(rowp + ch * 16);
        sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qv[ks], sacc[kh], 0, 0, 0);
      }
    }

    // Online softmax for this lane's query over the tile's 64 keys.
    float mx = sacc[0][0];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kh][r]);
    mx = swap_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_fast((m_run - m_new) * a.c2);
    m_run = m_new;
    const float mc = m_new * a.c2;
    float psum = 0.f;
    bf16x8_t pb[4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(fmaf(sacc[kh][r], a.c2, -mc));
        psum += p;
        pb[kh * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

    // O^T += V^T P^T.
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int dd = dt * 32 + (lane & 31);
      const char* vrow = vs_lds + dd * (kBlock * 2);
      const int swz = v_swz(dd);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (((2 * kk) ^ swz) * 16) + 8 * hi);
        const uint2 hi8 = *reinterpret_cast<const uint2*>(vrow + (((2 * kk + 1) ^ swz) * 16) + 8 * hi);
        const uint4 packed = make_uint4(lo.x, lo.y, hi8.x, hi8.y);
        bf16x8_t av;
        __builtin_memcpy(&av, &packed, 16);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kk], o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Epilogue: normalise, round once to bf16, write (original order if asked).
  const float l_tot = swap_sum(l_run);
  const float inv = cnt > 0 ? 1.0f / l_tot : 0.f;
  const long long n = a.orig ? token_of(g, i, q_local) : (long long)i * kBlock + q_local;
  uint16_t* orow = a.out + ((long long)bh * g.N + n) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      __bf16 h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (__bf16)(o[dt][4 * g4 + e] * inv);
      uint2 v;
      __builtin_memcpy(&v, h, 8);
      *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * g4 + 4 * hi) = v;
    }
  if (a.lse && hi == 0) {
    a.lse[(long long)bh * g.N + (long long)i * kBlock + q_local] =
        cnt > 0 ? m_run * a.scale + logf(l_tot) : -INFINITY;
  }
}

// float32 path: 128 threads per query block, thread pair (2r, 2r+1) owns query row r,
// each holding half of the channels.
struct AttnArgsF32 {
  const float* q;
  const float* k;
  const float* vt;
  const int32_t* counts;
  const int32_t* lists;
  const int32_t* order;
  float* out;
  float* lse;
  KGeom g;
  float scale;
  int orig;
};

template <int D>
__global__ __launch_bounds__(128) void k_attn_f32(AttnArgsF32 a) {
  constexpr int H2 = D / 2;
  constexpr int KC = 16;  // keys per softmax chunk
  __shared__ __attribute__((aligned(16))) float ks[kBlock * D];
  __shared__ __attribute__((aligned(16))) float vs[D * kBlock];
  const int t = threadIdx.x;
  const int r = t >> 1, half = t & 1;
  const KGeom& g = a.g;
  const int nb = g.nb;
  const int bh = blockIdx.x / nb;
  const int pos = blockIdx.x - bh * nb;
  const int i = a.order ? a.order[(long long)bh * nb + pos] : pos;
  const long long row = (long long)bh * nb + i;
  const int cnt = min(max(a.counts[row], 0), nb);
  const int32_t* lst = a.lists + row * nb;

  float q[H2], o[H2];
  const float* qrow = a.q + ((long long)bh * g.N + (long long)i * kBlock + r) * D + half * H2;
#pragma unroll
  for (int c = 0; c < H2; ++c) {
    q[c] = qrow[c];
    o[c] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float* kbase = a.k + (long long)bh * g.N * D;
  const float* vbase = a.vt + (long long)bh * nb * D * kBlock;

  for (int tt = 0; tt < cnt; ++tt) {
    const int j = min(max(lst[tt], 0), nb - 1);
    const float4* kg = reinterpret_cast<const float4*>(kbase + (long long)j * kBlock * D);
    const float4* vg = reinterpret_cast<const float4*>(vbase + (long long)j * D * kBlock);
    for (int u = t; u < kBlock * D / 4; u += 128) {
      reinterpret_cast<float4*>(ks)[u] = kg[u];
      reinterpret_cast<float4*>(vs)[u] = vg[u];
    }
    __syncthreads();
    for (int kc = 0; kc < kBlock; kc += KC) {
      float s[KC];
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const float* krow = ks + (kc + kk) * D + half * H2;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < H2; ++c) part = fmaf(q[c], krow[c], part);
        const float other = __shfl_xor(part, 1);
        s[kk] = (half ? other + part : part + other) * a.scale;
        mx = fmaxf(mx, s[kk]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float alpha = expf(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        s[kk] = expf(s[kk] - m_new);
        psum += s[kk];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int c = 0; c < H2; ++c) {
        float acc = o[c] * alpha;
        const float* vcol = vs + (half * H2 + c) * kBlock + kc;
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) acc = fmaf(s[kk], vcol[kk], acc);
        o[c] = acc;
      }
    }
    __syncthreads();
  }
  const float inv = cnt > 0 ? 1.0f / l_run : 0.f;
  const long long n = a.orig ? token_of(g, i, r) : (long long)i * kBlock + r;
  float* orow = a.out + ((long long)bh * g.N + n) * D + half * H2;
#pragma unroll
  for (int c = 0; c < H2; ++c) orow[c] = o[c] * inv;
  if (a.lse && half == 0)
    a.lse[(long long)bh * g.N + (long long)i * kBlock + r] = cnt > 0 ? m_run + logf(l_run) : -INFINITY;
}

// Longest-first order of the query blocks of each (b, h): a counting sort of the kept counts.
__global__ __launch_bounds__(1024) void k_row_order(const int32_t* __restrict__ counts, int32_t* __restrict__ order,
                                                    int nb) {
  __shared__ int hist[kMaxBlocks + 1];
  const int t = threadIdx.x;
  const long long bh = blockIdx.x;
  const int32_t* c = counts + bh * nb;
  for (int v = t; v <= nb; v += 1024) hist[v] = 0;
  __syncthreads();
  for (int r = t; r < nb; r += 1024) atomicAdd(&hist[min(max(c[r], 0), nb)], 1);
  __syncthreads();
  if (t == 0) {
    // hist[v] becomes the first position of count v in descending order.
    int run = 0;
    for (int v = nb; v >= 0; --v) {
      const int h = hist[v];
      hist[v] = run;
      run += h;
    }
  }
  __syncthreads();
  for (int r = t; r < nb; r += 1024) {
    const int p = atomicAdd(&hist[min(max(c[r], 0), nb)], 1);
    order[bh * nb + p] = r;
  }
}

}  // namespace

hipError_t launch_sparse_attn(const KGeom& g, int dtype, float scale, const void* q, const void* k,
                              const void* vt, const int32_t* counts, const int32_t* lists, void* out,
                              int out_original_order, float* lse, int32_t* row_order, hipStream_t s) {
  const unsigned bhs = (unsigned)(g.B * g.H);
  k_row_order<<<dim3(bhs), 1024, 0, s>>>(counts, row_order, g.nb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((long long)bhs * g.nb));
  if (dtype == ABLA_BF16) {
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.vt = static_cast<const uint16_t*>(vt);
    a.counts = counts;
    a.lists = lists;
    a.order = row_order;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.g = g;
    a.scale = scale;
    a.c2 = scale * 1.4426950408889634f;
    a.orig = out_original_order;
    if (g.d == 128)
      k_attn_bf16<128><<<grid, 128, 0, s>>>(a);
    else
      k_attn_bf16<64><<<grid, 128, 0, s>>>(a);
  } else {
    AttnArgsF32 a;
    a.q = static_cast<const float*>(q);
    a.k = static_cast<const float*>(k);
    a.vt = static_cast<const float*>(vt);
    a.counts = counts;
    a.lists = lists;
    a.order = row_order;
    a.out = static_cast<float*>(out);
    a.lse = lse;
    a.g = g;
    a.scale = scale;
    a.orig = out_original_order;
    if (g.d == 128)
      k_attn_f32<128><<<grid, 128, 0, s>>>(a);
    else
      k_attn_f32<64><<<grid, 128, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace abla
