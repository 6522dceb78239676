// Block-sparse attention backward: dQ, dK, dV of the forward over the kept 64 x 64 blocks.
//
// NABLA is used for training as well as inference (technical summary, Results: training
// speed-up with the same sparse mask), so the gradient of the block-sparse attention is
// needed with the same mask. With S = scale * Q K^T on the kept blocks, P = softmax rows of
// S (recomputed from the forward's log-sum-exp), O = P V and the incoming gradient dO:
//   dV = P^T dO,  dP = dO V^T,  D_i = <dO_i, O_i>,  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Pre-passes: D and log2(e) * lse per fractal row (k_bwd_delta); for every key block the
// ascending list of query blocks that keep it (k_col_lists); fractal reorders of Q, K, V, dO
// into the token-major and channel-major layouts the MFMA operands read.
//
// k_bwd_dq, one workgroup (two waves of 32 queries) per query block, walks the block's kept
// list like the forward: S^T = K Q^T and dP^T = V dO^T with the K / V rows in the forward's
// key permutation, so each lane's accumulators hold 8 consecutive keys of its query;
// dS^T = P^T * (dP^T - D) rounded to bf16 is then the B operand of dQ^T += K^T dS^T, with
// K^T rows read from the channel-major copy of K.
//
// k_bwd_dkdv, one workgroup (two waves of 32 keys) per key block, walks the key block's
// column list with the roles of Q and K swapped: S = Q K^T and dP = dO V^T with the query
// rows permuted, so each lane holds 8 consecutive queries of its key; then
// dV^T += dO^T P and dK^T += Q^T dS with channel-major copies of dO and Q.
//
// Both write their gradient rows in the original token order. bf16 inputs and outputs,
// float32 accumulation, P and dS rounded to bf16 for the MFMA products.
#include <math.h>

#include "common.h"
#include "mfma_tiles.h"

namespace abla {
namespace {

constexpr int kBwdThreads = 128;  // two waves, 32 rows each
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------- pre-passes
// D[m] = <dO[n], O[n]> (float32 sums of the bf16 products) and L2[m] = lse[m] * log2(e) for
// fractal row m of token n. D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_delta(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                   const float* __restrict__ lse, float* __restrict__ Dm,
                                                   float* __restrict__ L2, KGeom g) {
  constexpr int LPR = D / 8;
  const long long rows = (long long)g.B * g.H * g.N;
  const long long row = ((long long)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const long long bh = row / g.N;
    const int m = (int)(row - bh * g.N);
    const long long n = token_of(g, m / kBlock, m % kBlock);
    const long long off = (bh * g.N + n) * D + sub * 8;
    const uint4 a = *reinterpret_cast<const uint4*>(o + off);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + off);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(__uint_as_float(wa[k] << 16), __uint_as_float(wb[k] << 16), acc);
      acc = fmaf(__uint_as_float(wa[k] & 0xFFFF0000u), __uint_as_float(wb[k] & 0xFFFF0000u), acc);
    }
  }
#pragma unroll
  for (int s = 1; s < LPR; s <<= 1) acc += __shfl_xor(acc, s);
  if (row < rows && sub == 0) {
    Dm[row] = acc;
    L2[row] = lse[row] * kLog2e;
  }
}

// For key block j of each (b, h): the ascending list of query blocks whose mask row keeps j.
__global__ __launch_bounds__(256) void k_col_lists(const uint32_t* __restrict__ words, int32_t* __restrict__ col_counts,
                                                   int32_t* __restrict__ col_lists, int nb, int W) {
  const long long bh = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= nb) return;
  const uint32_t* wcol = words + bh * nb * W + (j >> 5);
  const int bit = j & 31;
  int32_t* out = col_lists + (bh * nb + j) * nb;
  int c = 0;
  for (int i = 0; i < nb; ++i)
    if ((wcol[(long long)i * W] >> bit) & 1u) out[c++] = i;
  col_counts[bh * nb + j] = c;
}

// ------------------------------------------------------------------- tile loads
// 128-thread global->LDS loads of one 64-row tile. Token-major tiles (K, V, Q, dO rows) take
// the forward's K layout: LDS row r holds row kperm(r), its 16-byte chunks XOR-swizzled by
// k_swz(r). Channel-major tiles (K^T, Q^T, dO^T) take the forward's V^T layout. Unit u of the
// tile sits at LDS byte u*16; thread t fills units it*128 + t.
template <int D, bool TOKEN_MAJOR>
__device__ __forceinline__ void load_tile128(char* slot, i32x4_t rsrc, uint32_t tile) {
  constexpr int UNITS = kBlock * D * 2 / 16;
  constexpr int LOADS = UNITS / kBwdThreads;
  const int t = threadIdx.x, w = t >> 6;
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int u = it * kBwdThreads + t;
    uint32_t off;
    if constexpr (TOKEN_MAJOR) {
      constexpr int KCH = D / 8;
      const int r = u / KCH, pc = u % KCH;
      off = (uint32_t)(kperm(r) * D * 2 + ((pc ^ k_swz<D>(r)) * 16));
    } else {
      const int dd = u >> 3, pc = u & 7;
      off = (uint32_t)(dd * kBlock * 2 + ((pc ^ v_swz(dd)) * 16));
    }
    raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) uint32_t*)(slot + it * kBwdThreads * 16 + w * 1024),
                        16, (int)off, (int)tile, 0, 0);
  }
}

// A-operand chunk of a token-major tile: row (half*32 + lane%32), k-step ks.
template <int D>
__device__ __forceinline__ bf16x8_t row_chunk(const char* tile, int half, int lane, int ks) {
  const int row = half * 32 + (lane & 31);
  const int c = (ks * 2 + (lane >> 5)) ^ k_swz<D>(row);
  return *reinterpret_cast<const bf16x8_t*>(tile + row * D * 2 + c * 16);
}

// A-operand chunk of a channel-major tile: channel (dt*32 + lane%32), 16-row step kk.
__device__ __forceinline__ bf16x8_t chan_chunk(const char* tile, int dt, int lane, int kk) {
  const int ch = dt * 32 + (lane & 31);
  const int c = (2 * kk + (lane >> 5)) ^ v_swz(ch);
  return *reinterpret_cast<const bf16x8_t*>(tile + ch * kBlock * 2 + c * 16);
}

// Write one wave's transposed accumulators acc[dt][r] = X^T[channel dt*32 + 8*(r/4) + 4*hi + r%4]
// [row lane%32] as bf16 rows x * mul of the original-order tensor y, row = token of (blk, row_local).
template <int D>
__device__ __forceinline__ void write_rows(uint16_t* y, const KGeom& g, long long bh, int blk, int row_local,
                                           const f32x16_t* acc, float mul, int hi) {
  const long long n = token_of(g, blk, row_local);
  uint16_t* orow = y + (bh * g.N + n) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      __bf16 h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (__bf16)(acc[dt][4 * g4 + e] * mul);
      uint2 v;
      __builtin_memcpy(&v, h, 8);
      *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * g4 + 4 * hi) = v;
    }
}

// ------------------------------------------------------------------- dQ
struct DqArgs {
  const uint16_t *q_r, *k_r, *k_rt, *v_r, *do_r;
  const float *Dm, *L2;
  const int32_t *counts, *lists;
  uint16_t* dq;
  KGeom g;
  float c2, scale;
};

template <int D>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_dq(DqArgs a) {
  constexpr int TB = kBlock * D * 2;
  __shared__ __attribute__((aligned(1024))) char smem[3 * TB];  // K, V (token-major), K^T
  char* ks_lds = smem;
  char* vs_lds = smem + TB;
  char* kt_lds = smem + 2 * TB;

  const KGeom& g = a.g;
  const int nb = g.nb;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, hi = lane >> 5;
  const long long bh = blockIdx.x / nb;
  const int i = blockIdx.x - (int)(bh * nb);
  const long long row = bh * nb + i;
  const int cnt = min(max(ld_const(a.counts, row), 0), nb);
  const int q_local = w * 32 + (lane & 31);
  const long long m = (long long)i * kBlock + q_local;  // fractal row of this lane's query

  bf16x8_t qv[D / 16], dov[D / 16];
  {
    const uint16_t* qrow = a.q_r + (bh * g.N + m) * D + 8 * hi;
    const uint16_t* drow = a.do_r + (bh * g.N + m) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qv[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
      dov[ks] = *reinterpret_cast<const bf16x8_t*>(drow + ks * 16);
    }
  }
  const float l2 = a.L2[bh * g.N + m];
  const float dq_d = a.Dm[bh * g.N + m];

  const uint32_t head_bytes = (uint32_t)(g.N * D * 2);
  const i32x4_t krs = make_rsrc(a.k_r + bh * g.N * D, head_bytes);
  const i32x4_t vrs = make_rsrc(a.v_r + bh * g.N * D, head_bytes);
  const i32x4_t ktrs = make_rsrc(a.k_rt + bh * g.N * D, head_bytes);

  f32x16_t acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  const int32_t* lst = a.lists + row * nb;
  for (int u = 0; u < cnt; ++u) {
    const int j = min(max(ld_const(lst, u), 0), nb - 1);
    load_tile128<D, true>(ks_lds, krs, (uint32_t)j * TB);
    load_tile128<D, true>(vs_lds, vrs, (uint32_t)j * TB);
    load_tile128<D, false>(kt_lds, ktrs, (uint32_t)j * TB);
    wait_vm_lgkm_barrier();

    f32x16_t s[2], dp[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kh][r] = 0.f;
        dp[kh][r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk<D>(ks_lds, kh, lane, ks), qv[ks], s[kh], 0, 0, 0);
        dp[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk<D>(vs_lds, kh, lane, ks), dov[ks], dp[kh], 0, 0, 0);
      }
    }
    bf16x8_t dsb[4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(fmaf(s[kh][r], a.c2, -l2));
        dsb[kh * 2 + (r >> 3)][r & 7] = (__bf16)(p * (dp[kh][r] - dq_d));
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(chan_chunk(kt_lds, dt, lane, kk), dsb[kk], acc[dt], 0, 0, 0);
    wait_vm_lgkm_barrier();  // every wave is done with the tiles before they are refilled
  }
  write_rows<D>(a.dq, g, bh, i, q_local, acc, a.scale, hi);
}

// ------------------------------------------------------------------- dK, dV
struct DkvArgs {
  const uint16_t *k_r, *v_r, *q_r, *q_rt, *do_r, *do_rt;
  const float *Dm, *L2;
  const int32_t *col_counts, *col_lists;
  uint16_t *dk, *dv;
  KGeom g;
  float c2, scale;
};

template <int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_bwd_dkdv(DkvArgs a) {
  constexpr int TB = kBlock * D * 2;
  __shared__ __attribute__((aligned(1024))) char smem[4 * TB + 2 * kBlock * 4];  // Q, dO, Q^T, dO^T, L2, D
  char* q_lds = smem;
  char* do_lds = smem + TB;
  char* qt_lds = smem + 2 * TB;
  char* dot_lds = smem + 3 * TB;
  float* l2_lds = reinterpret_cast<float*>(smem + 4 * TB);
  float* d_lds = l2_lds + kBlock;

  const KGeom& g = a.g;
  const int nb = g.nb;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, hi = lane >> 5;
  const long long bh = blockIdx.x / nb;
  const int j = blockIdx.x - (int)(bh * nb);
  const long long col = bh * nb + j;
  const int cnt = min(max(ld_const(a.col_counts, col), 0), nb);
  const int k_local = w * 32 + (lane & 31);
  const long long mk = (long long)j * kBlock + k_local;  // fractal row of this lane's key

  bf16x8_t kb[D / 16], vb[D / 16];
  {
    const uint16_t* krow = a.k_r + (bh * g.N + mk) * D + 8 * hi;
    const uint16_t* vrow = a.v_r + (bh * g.N + mk) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kb[ks] = *reinterpret_cast<const bf16x8_t*>(krow + ks * 16);
      vb[ks] = *reinterpret_cast<const bf16x8_t*>(vrow + ks * 16);
    }
  }
  const uint32_t head_bytes = (uint32_t)(g.N * D * 2);
  const i32x4_t qrs = make_rsrc(a.q_r + bh * g.N * D, head_bytes);
  const i32x4_t dors = make_rsrc(a.do_r + bh * g.N * D, head_bytes);
  const i32x4_t qtrs = make_rsrc(a.q_rt + bh * g.N * D, head_bytes);
  const i32x4_t dotrs = make_rsrc(a.do_rt + bh * g.N * D, head_bytes);
  const i32x4_t l2rs = make_rsrc(a.L2 + bh * g.N, (uint32_t)(g.N * 4));
  const i32x4_t drs = make_rsrc(a.Dm + bh * g.N, (uint32_t)(g.N * 4));

  f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  const int32_t* lst = a.col_lists + col * nb;
  for (int u = 0; u < cnt; ++u) {
    const int i = min(max(ld_const(lst, u), 0), nb - 1);
    load_tile128<D, true>(q_lds, qrs, (uint32_t)i * TB);
    load_tile128<D, true>(do_lds, dors, (uint32_t)i * TB);
    load_tile128<D, false>(qt_lds, qtrs, (uint32_t)i * TB);
    load_tile128<D, false>(dot_lds, dotrs, (uint32_t)i * TB);
    if (t < 16) {  // 64 floats of L2 and 64 of D: 16 lanes x 16 bytes each
      raw_buffer_load_lds(l2rs, (__attribute__((address_space(3))) uint32_t*)l2_lds, 16, t * 16, i * kBlock * 4, 0, 0);
      raw_buffer_load_lds(drs, (__attribute__((address_space(3))) uint32_t*)d_lds, 16, t * 16, i * kBlock * 4, 0, 0);
    }
    wait_vm_lgkm_barrier();

    // S = Q K^T, dP = dO V^T: accumulator register r of half qh holds query
    // qh*32 + 16*(r/8) + 8*hi + r%8 of this lane's key (query rows permuted like K rows).
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[qh][r] = 0.f;
        dp[qh][r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s[qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk<D>(q_lds, qh, lane, ks), kb[ks], s[qh], 0, 0, 0);
        dp[qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk<D>(do_lds, qh, lane, ks), vb[ks], dp[qh], 0, 0, 0);
      }
    }
    bf16x8_t pb[4], dsb[4];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int q8 = 0; q8 < 2; ++q8) {
        const int q0 = qh * 32 + 16 * q8 + 8 * hi;
        const float4 la = *reinterpret_cast<const float4*>(l2_lds + q0);
        const float4 lb = *reinterpret_cast<const float4*>(l2_lds + q0 + 4);
        const float4 da = *reinterpret_cast<const float4*>(d_lds + q0);
        const float4 db = *reinterpret_cast<const float4*>(d_lds + q0 + 4);
        const float lq[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
        const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = q8 * 8 + e;
          const float p = exp2_fast(fmaf(s[qh][r], a.c2, -lq[e]));
          pb[qh * 2 + q8][e] = (__bf16)p;
          dsb[qh * 2 + q8][e] = (__bf16)(p * (dp[qh][r] - dd[e]));
        }
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(chan_chunk(dot_lds, dt, lane, kk), pb[kk], dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(chan_chunk(qt_lds, dt, lane, kk), dsb[kk], dk[dt], 0, 0, 0);
      }
    wait_vm_lgkm_barrier();  // every wave is done with the tiles before they are refilled
  }
  write_rows<D>(a.dk, g, bh, j, k_local, dk, a.scale, hi);
  write_rows<D>(a.dv, g, bh, j, k_local, dv, 1.0f, hi);
}

}  // namespace

hipError_t launch_sparse_attn_bwd(const KGeom& g, float scale, const void* q, const void* k, const void* v,
                                  const void* o, const void* dout, const float* lse, const uint32_t* words,
                                  const int32_t* counts, const int32_t* lists, void* dq, void* dk, void* dv,
                                  const BwdWorkspace& ws, hipStream_t s) {
  // Fractal copies: token-major Q, K, V, dO; channel-major Q, K, dO.
  hipError_t e;
  if ((e = launch_reorder(g, ABLA_BF16, 0, ABLA_LAYOUT_TOKENS, q, ws.q_r, nullptr, s)) != hipSuccess) return e;
  if ((e = launch_reorder(g, ABLA_BF16, 0, ABLA_LAYOUT_BLOCK_T, q, ws.q_rt, nullptr, s)) != hipSuccess) return e;
  if ((e = launch_reorder(g, ABLA_BF16, 0, ABLA_LAYOUT_TOKENS, k, ws.k_r, nullptr, s)) != hipSuccess) return e;
  if ((e = launch_reorder(g, ABLA_BF16, 0, ABLA_LAYOUT_BLOCK_T, k, ws.k_rt, nullptr, s)) != hipSuccess) return e;
  if ((e = launch_reorder(g, ABLA_BF16, 0, ABLA_LAYOUT_TOKENS, v, ws.v_r, nullptr, s)) != hipSuccess) return e;
  if ((e = launch_reorder(g, ABLA_BF16, 0, ABLA_LAYOUT_TOKENS, dout, ws.do_r, nullptr, s)) != hipSuccess) return e;
  if ((e = launch_reorder(g, ABLA_BF16, 0, ABLA_LAYOUT_BLOCK_T, dout, ws.do_rt, nullptr, s)) != hipSuccess) return e;

  const long long rows = (long long)g.B * g.H * g.N;
  const unsigned bhs = (unsigned)(g.B * g.H);
  const int lpr = g.d / 8;
  const unsigned dgrid = (unsigned)((rows * lpr + 255) / 256);
  const uint16_t* o16 = static_cast<const uint16_t*>(o);
  const uint16_t* do16 = static_cast<const uint16_t*>(dout);
  if (g.d == 128)
    k_bwd_delta<128><<<dim3(dgrid), 256, 0, s>>>(o16, do16, lse, ws.D, ws.L2, g);
  else
    k_bwd_delta<64><<<dim3(dgrid), 256, 0, s>>>(o16, do16, lse, ws.D, ws.L2, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_col_lists<<<dim3((unsigned)((g.nb + 255) / 256), bhs), 256, 0, s>>>(words, ws.col_counts, ws.col_lists, g.nb,
                                                                       (g.nb + 31) / 32);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const float c2 = scale * kLog2e;
  const dim3 grid((unsigned)((long long)bhs * g.nb));
  DqArgs qa{ws.q_r, ws.k_r, ws.k_rt, ws.v_r, ws.do_r, ws.D, ws.L2, counts, lists,
            static_cast<uint16_t*>(dq), g, c2, scale};
  if (g.d == 128)
    k_bwd_dq<128><<<grid, kBwdThreads, 0, s>>>(qa);
  else
    k_bwd_dq<64><<<grid, kBwdThreads, 0, s>>>(qa);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  DkvArgs ka{ws.k_r, ws.v_r, ws.q_r, ws.q_rt, ws.do_r, ws.do_rt, ws.D, ws.L2, ws.col_counts, ws.col_lists,
             static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), g, c2, scale};
  if (g.d == 128)
    k_bwd_dkdv<128><<<grid, kBwdThreads, 0, s>>>(ka);
  else
    k_bwd_dkdv<64><<<grid, kBwdThreads, 0, s>>>(ka);
  return hipGetLastError();
}

}  // namespace abla
