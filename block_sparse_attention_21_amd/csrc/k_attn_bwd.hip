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
// ascending list of query blocks that keep it (k_col_lists). Q, K, V and dO are read in their
// original token order: a 64-token block is gathered as its 8 runs of 8 tokens, so no
// reordered copies are made.
//
// k_bwd_dq, one workgroup of four waves per query block, walks the block's kept list: wave
// (qh, kh) forms S^T = K Q^T and dP^T = V dO^T for keys kh*32.. and queries qh*32.. with the K /
// V rows in the forward's key permutation, so each lane's accumulators hold 8 consecutive keys
// of its query; dS^T = P^T * (dP^T - D) rounded to bf16 is then the B operand of
// dQ^T += K^T dS^T, whose K^T operand is read from the same token-major K tile with the gfx950
// LDS transpose load. The two key halves are summed through LDS at the end.
//
// k_bwd_dkdv, one workgroup of four waves per key block, walks the key block's column list with
// the roles of Q and K swapped: S = Q K^T and dP = dO V^T with the query rows permuted, then
// dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read by transpose loads; the key block's V
// tile stays in LDS for the whole walk.
//
// Both kernels double-buffer their tiles in LDS (the loads of tile u+1 run during the products
// of tile u) and write their gradient rows in the original token order. bf16 inputs and
// outputs, float32 accumulation, P and dS rounded to bf16 for the MFMA products.
#include <math.h>

#include "common.h"
#include "mfma_tiles.h"

namespace abla {
namespace {

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
// One wave per key block (four per workgroup): lane l tests row i0 + l, and a ballot places
// the keeping rows of each 64-row chunk in order. (One thread per key block scanning all nb
// rows left the GPU nearly idle: 36 workgroups at 480p.) A one-dimensional grid of
// ceil(nb / kColWaves) workgroups per (b, h).
constexpr int kColWaves = 4;
__global__ __launch_bounds__(64 * kColWaves) void k_col_lists(const uint32_t* __restrict__ words,
                                                              int32_t* __restrict__ col_counts,
                                                              int32_t* __restrict__ col_lists, int nb, int W) {
  const int per_head = (nb + kColWaves - 1) / kColWaves;
  const long long bh = blockIdx.x / per_head;
  const int lane = threadIdx.x & 63;
  const int j = ((int)blockIdx.x - (int)bh * per_head) * kColWaves + (threadIdx.x >> 6);
  if (j >= nb) return;  // whole waves
  const uint32_t* wcol = words + bh * nb * W + (j >> 5);
  const int bit = j & 31;
  int32_t* out = col_lists + (bh * nb + j) * nb;
  const unsigned long long below = (1ull << lane) - 1;
  int c = 0;
  for (int i0 = 0; i0 < nb; i0 += 64) {
    const int i = i0 + lane;
    const bool keep = i < nb && ((wcol[(long long)i * W] >> bit) & 1u);
    const unsigned long long m = __builtin_amdgcn_ballot_w64(keep);
    if (keep) out[c + __builtin_popcountll(m & below)] = i;
    c += __builtin_popcountll(m);
  }
  if (lane == 0) col_counts[bh * nb + j] = c;
}

// ------------------------------------------------------------------- operands
// Token-major tiles gathered from a tensor in the original token order: block j is 8 runs of
// 8 tokens (one per patch row); in LDS, row r holds token kperm(r) of the block with its
// 16-byte chunks XOR-swizzled by kt_swz(r). orig_tile_off gives thread t's fixed offset from the block's
// corner token (LDS row r = t / KCH holds key kperm(r), kperm(r) / 8 patch rows of Ws tokens
// and kperm(r) % 8 tokens in); consecutive loads of a thread are 16 (d = 128) or 32 (d = 64)
// LDS rows, i.e. 2 or 4 patch rows, 512 * Ws bytes apart; orig_tile_base is the corner's byte
// offset inside the head.
template <int D>
__device__ __forceinline__ uint32_t orig_tile_off(int t, int Ws) {
  constexpr int KCH = D / 8;
  const int r = t / KCH, pc = t % KCH;
  const int kr = kperm(r);
  return (uint32_t)(((kr >> 3) * Ws + (kr & 7)) * D * 2 + ((pc ^ kt_swz<D>(r)) * 16));
}
template <int D>
__device__ __forceinline__ uint32_t orig_tile_base(const KGeom& g, int j) {
  const int F = g.nbh * g.nbw;
  const int tf = j / F, rem = j - tf * F;
  const int hp = rem / g.nbw, wp = rem - hp * g.nbw;
  return (uint32_t)(((tf * g.Hs + hp * kP) * g.Ws + wp * kP) * D * 2);
}

// A-operand chunk of a token-major tile: row (half*32 + lane%32), k-step ks.
template <int D>
__device__ __forceinline__ bf16x8_t row_chunk(const char* tile, int half, int lane, int ks) {
  const int row = half * 32 + (lane & 31);
  const int c = (ks * 2 + (lane >> 5)) ^ kt_swz<D>(row);
  return *reinterpret_cast<const bf16x8_t*>(tile + row * D * 2 + c * 16);
}

// Write rows of one wave's transposed accumulators acc[k][r] = X^T[channel (dt0+k)*32 + 8*(r/4)
// + 4*hi + r%4][row lane%32], k < NDT, as bf16 x * mul into the original-order tensor y, row =
// token of (blk, row_local).
template <int D, int NDT>
__device__ __forceinline__ void write_rows(uint16_t* y, const KGeom& g, long long bh, int blk, int row_local,
                                           const f32x16_t* acc, int dt0, float mul, int hi) {
  const long long n = token_of(g, blk, row_local);
  uint16_t* orow = y + (bh * g.N + n) * D + dt0 * 32 + 4 * hi;
#pragma unroll
  for (int k = 0; k < NDT; ++k)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      __bf16 h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (__bf16)(acc[k][4 * g4 + e] * mul);
      uint2 v;
      __builtin_memcpy(&v, h, 8);
      *reinterpret_cast<uint2*>(orow + k * 32 + 8 * g4) = v;
    }
}

// Store / add NT accumulator tiles acc[first .. first+NT) through LDS, layout float [NT][16][64]
// (lane-contiguous). Indices are compile-time so the accumulators stay in registers.
template <int FIRST, int NT>
__device__ __forceinline__ void stash(float* dst, const f32x16_t* acc, int lane) {
#pragma unroll
  for (int k = 0; k < NT; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[(k * 16 + r) * 64 + lane] = acc[FIRST + k][r];
}
template <int FIRST, int NT>
__device__ __forceinline__ void unstash_add(const float* src, f32x16_t* acc, int lane) {
#pragma unroll
  for (int k = 0; k < NT; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[FIRST + k][r] += src[(k * 16 + r) * 64 + lane];
}

constexpr int kBwdThreads = 256;  // four waves

// Block visited by workgroup `wg`: the blocks of one patch in successive frames (a temporal
// column) run back to back on one XCD, columns dealt round-robin to the 8 XCDs (workgroup w
// runs on XCD w % 8). Temporally adjacent blocks keep largely the same key (or query) blocks,
// so the tiles one workgroup fetches are still in that XCD's L2 for the next. The position
// within a head maps to a column-major index (column * T + frame); columns that do not fill a
// last cycle over the 8 XCDs keep their column-major place. Heads run in order.
__device__ __forceinline__ void column_order(int wg, const KGeom& g, long long& bh, int& blk) {
  const int F = g.nbh * g.nbw, T = g.T, nb = g.nb;
  bh = wg / nb;
  const int pos = wg - (int)(bh * nb);
  const int full = (F / 8) * 8 * T;  // positions in whole cycles of 8 columns
  int cm = pos;
  if (pos < full) {
    const int x = pos & 7, k = pos >> 3;
    cm = (8 * (k / T) + x) * T + k % T;
  }
  blk = (cm % T) * F + cm / T;
}

// The bf16 kernels read their block from a table: the column order above. When the list
// lengths are heavy-tailed (the longest above 3x the mean), each XCD's queue (the workgroups
// w with w % 8 == x, in order) is partitioned so that the blocks whose list is longer than
// 1.25x the mean come first, both parts in queue order. Started late, the longest lists
// formed a tail in which a quarter of the slots sat idle (dQ at 480p: 73% slot use). In
// either case the queue's last 128 positions (two generations of the XCD's resident
// workgroups) are written longest-first. Workgroup x writes the queue of XCD x; `cnt` holds
// the list lengths (counts for dQ, column counts for dK/dV); order[w] = bh * nb + block.
constexpr int kBwdQueueTail = 128;

// Items main .. grid-1 (the last kBwdQueueTail positions of every XCD's queue, its shortest
// lists, longest-first) are claimed at run time by kBwdTailOversub workgroups per item, so the
// XCDs that finish their static share first take more of them (as the forward's claim_item).
// `slot` is one int of LDS; returns the item or -1.
constexpr int kBwdTailOversub = 2;
__device__ __forceinline__ int bwd_claim_item(int main, int grid, int32_t* tail_cnt, int* slot) {
  if ((int)blockIdx.x < main) return (int)blockIdx.x;
  if (threadIdx.x == 0) *slot = atomicAdd(tail_cnt, 1);  // a vector-memory atomic, one lane
  __syncthreads();
  const int it = main + *slot;
  __syncthreads();  // the slot is LDS the tiles reuse
  return it < grid ? it : -1;
}
__global__ __launch_bounds__(1024) void k_bwd_order(const int32_t* __restrict__ cnt, int32_t* __restrict__ order,
                                                    int32_t* __restrict__ tail_cnt, KGeom g, int bhs) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *tail_cnt = 0;  // for bwd_claim_item
  __shared__ long long wsum[16];
  __shared__ int wpart[16];
  __shared__ int tail_gi[kBwdQueueTail], tail_cost[kBwdQueueTail];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int x = blockIdx.x, nb = g.nb;
  const int grid = bhs * nb;
  long long part = 0;
  int mx = 0;
  for (int r = t; r < grid; r += 1024) {
    const int c = min(max(cnt[r], 0), nb);
    part += c;
    mx = max(mx, c);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    part += __shfl_xor(part, o);
    mx = max(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) {
    wsum[wv] = part;
    wpart[wv] = mx;
  }
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < 16; ++w) {
    total += wsum[w];
    mx = max(mx, wpart[w]);
  }

  auto item = [&](int k) {  // queue rank k of this XCD = workgroup 8k + x
    long long bh;
    int blk;
    column_order(8 * k + x, g, bh, blk);
    return (int)bh * nb + blk;
  };
  auto cost = [&](int gi) { return min(max(cnt[gi], 0), nb); };
  auto block_scan = [&](int v, int& total_out) {  // exclusive prefix of v over the workgroup
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == 63) wpart[wv] = incl;
    __syncthreads();
    int base = 0, all = 0;
    for (int w = 0; w < 16; ++w) {
      base += w < wv ? wpart[w] : 0;
      all += wpart[w];
    }
    total_out = all;
    return base + incl - v;
  };
  const int n_x = (grid - x + 7) / 8;
  const int tail0 = max(n_x - kBwdQueueTail, 0);
  // Position p of the queue gets item gi: the last kBwdQueueTail positions are collected in
  // LDS and written longest-first at the end, so the queue ends with its shortest lists.
  auto place = [&](int p, int gi) {
    if (p >= tail0) {
      tail_gi[p - tail0] = gi;
      tail_cost[p - tail0] = cost(gi);
    } else {
      order[8 * p + x] = gi;
    }
  };
  // Without a heavy tail (longest list at most 3x the mean) the column order is kept up to
  // the queue's end: at 720p moving the longer lists forward only cost L2 reuse.
  if ((long long)mx * grid <= 3ll * total) {
    for (int k = t; k < n_x; k += 1024) place(k, item(k));
  } else {
    int c = 0;
    for (int k = t; k < n_x; k += 1024) c += 4ll * cost(item(k)) * grid > 5ll * total ? 1 : 0;
    int nlong;
    block_scan(c, nlong);
    int base_l = 0, base_s = nlong;
    for (int c0 = 0; c0 < n_x; c0 += 1024) {
      const int k = c0 + t;
      const bool valid = k < n_x;
      const int gi = valid ? item(k) : 0;
      const bool lg = valid && 4ll * cost(gi) * grid > 5ll * total;
      int both;
      const int v = (lg ? 1 : 0) | ((valid && !lg) ? 1 << 16 : 0);  // two counts <= 1024, packed
      const int ex = block_scan(v, both);
      if (valid) place(lg ? base_l + (ex & 0xffff) : base_s + (ex >> 16), gi);
      base_l += both & 0xffff;
      base_s += both >> 16;
    }
  }
  __syncthreads();
  const int nt = n_x - tail0;
  if (t < nt) {
    const int c = tail_cost[t];
    int rank = 0;
    for (int u = 0; u < nt; ++u) rank += (tail_cost[u] > c) || (tail_cost[u] == c && u < t);
    order[8 * (tail0 + rank) + x] = tail_gi[t];
  }
}

// ------------------------------------------------------------------- dQ
struct DqArgs {
  const uint16_t *q, *k, *v, *dout;  // original token order
  const float *Dm, *L2;
  const int32_t *counts, *lists;
  const int32_t* order;  // visiting order (k_bwd_order)
  int32_t* tail_cnt;
  int main_grid, items;
  uint16_t* dq;
  KGeom g;
  float c2, scale;
};

// One workgroup per query block i, four waves: wave (qh, kh) takes queries qh*32.. and keys
// kh*32.. of every kept key tile. K and V tiles (token-major) are double-buffered in LDS: the
// loads of tile u+1 run during the products of tile u.
template <int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dq(DqArgs a) {
  constexpr int TB = kBlock * D * 2;
  constexpr int DT = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[4 * TB];  // K0, K1, V0, V1
  const KGeom& g = a.g;
  const int nb = g.nb;
  const int t = threadIdx.x, lane = t & 63, hi = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int qh = w & 1, kh = w >> 1;
  const int item = bwd_claim_item(a.main_grid, a.items, a.tail_cnt, reinterpret_cast<int*>(smem));
  if (item < 0) return;
  const int gi = ld_const(a.order, (long long)item);
  const long long bh = gi / nb;
  const int i = gi - (int)bh * nb;
  const long long row = bh * nb + i;
  const int cnt = min(max(ld_const(a.counts, row), 0), nb);
  const int q_local = qh * 32 + (lane & 31);
  const long long m = (long long)i * kBlock + q_local;  // fractal row of this lane's query

  bf16x8_t qv[D / 16], dov[D / 16];
  {
    const long long n = token_of(g, i, q_local);  // its token in the original order
    const uint16_t* qrow = a.q + (bh * g.N + n) * D + 8 * hi;
    const uint16_t* drow = a.dout + (bh * g.N + n) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qv[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
      dov[ks] = *reinterpret_cast<const bf16x8_t*>(drow + ks * 16);
    }
  }
  const float l2 = a.L2[bh * g.N + m];
  const float dq_d = a.Dm[bh * g.N + m];

  const uint32_t head_bytes = (uint32_t)(g.N * D * 2);
  const i32x4_t krs = make_rsrc(a.k + bh * g.N * D, head_bytes);
  const i32x4_t vrs = make_rsrc(a.v + bh * g.N * D, head_bytes);
  const uint32_t off = orig_tile_off<D>(t, g.Ws);
  const uint32_t stride = 512u * (uint32_t)g.Ws;

  f32x16_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  // K^T operand reads: offsets inside a K tile for each channel tile (keys kh*32 ..); the
  // second 16 keys are 16 rows further, an immediate offset.
  uint32_t trel[2 * DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) tr_rel<D>(dt, kh * 32, lane, trel[2 * dt], trel[2 * dt + 1]);

  const int32_t* lst = a.lists + row * nb;
  if (cnt > 0) {
    const uint32_t j0 = (uint32_t)min(max(ld_const(lst, 0), 0), nb - 1);
    const uint32_t b0 = orig_tile_base<D>(g, (int)j0);
    issue_rows<TB>(smem, w, krs, b0, off, stride);
    issue_rows<TB>(smem + 2 * TB, w, vrs, b0, off, stride);
  }
  for (int u = 0; u < cnt; ++u) {
    wait_vm_lgkm_barrier();  // tile u has landed; every wave is done with tile u-1
    if (u + 1 < cnt) {
      const uint32_t jn = (uint32_t)min(max(ld_const(lst, u + 1), 0), nb - 1);
      const uint32_t bn = orig_tile_base<D>(g, (int)jn);
      issue_rows<TB>(smem + ((u + 1) & 1) * TB, w, krs, bn, off, stride);
      issue_rows<TB>(smem + 2 * TB + ((u + 1) & 1) * TB, w, vrs, bn, off, stride);
    }
    const char* ks_lds = smem + (u & 1) * TB;
    const char* vs_lds = smem + 2 * TB + (u & 1) * TB;

    // S^T and dP^T for keys kh*32.. (rows of the MFMA) and this wave's 32 queries (columns).
    f32x16_t s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk<D>(ks_lds, kh, lane, ks), qv[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk<D>(vs_lds, kh, lane, ks), dov[ks], dp, 0, 0, 0);
    }
    // Register r holds key kh*32 + 16*(r/8) + 8*hi + r%8 of this lane's query.
    bf16x8_t dsb[2];
    __builtin_amdgcn_s_setprio(1);  // exponential phase at raised priority, as in dK/dV
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(fmaf(s[r], a.c2, -l2));
      dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dq_d));
    }
    __builtin_amdgcn_s_setprio(0);
    // dQ^T += K^T dS^T over this wave's 32 keys; K^T comes from the K tile by transpose loads.
    uint32_t ta[2 * DT];
    const uint32_t kbase = lds_offset(ks_lds);
#pragma unroll
    for (int k = 0; k < 2 * DT; ++k) ta[k] = kbase + trel[k];
    {
      bf16x8_t kt[DT];
      tr_chunks_at<DT, 0>(ta, kt);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[dt], dsb[0], acc[dt], 0, 0, 0);
    }
    {
      bf16x8_t kt[DT];
      tr_chunks_at<DT, 16 * D * 2>(ta, kt);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[dt], dsb[1], acc[dt], 0, 0, 0);
    }
  }
  // Waves (qh, 0) and (qh, 1) hold partial dQ^T over their key halves: wave (qh, kh) finishes
  // channel tiles [kh*DT/2, kh*DT/2 + DT/2) and hands the other half to its partner.
  wait_vm_lgkm_barrier();
  constexpr int H = DT / 2;
  float* xch = reinterpret_cast<float*>(smem);
  float* mine = xch + (qh * 2 + kh) * (H * 16 * 64);
  const float* theirs = xch + (qh * 2 + (1 - kh)) * (H * 16 * 64);
  if (kh == 0)
    stash<H, H>(mine, acc, lane);
  else
    stash<0, H>(mine, acc, lane);
  wait_vm_lgkm_barrier();
  if (kh == 0) {
    unstash_add<0, H>(theirs, acc, lane);
    write_rows<D, H>(a.dq, g, bh, i, q_local, acc, 0, a.scale, hi);
  } else {
    unstash_add<H, H>(theirs, acc, lane);
    write_rows<D, H>(a.dq, g, bh, i, q_local, acc + H, H, a.scale, hi);
  }
}

// ------------------------------------------------------------------- dK, dV
struct DkvArgs {
  const uint16_t *k, *v, *q, *dout;  // original token order
  const float *Dm, *L2;
  const int32_t *col_counts, *col_lists;
  const int32_t* order;  // visiting order (k_bwd_order)
  int32_t* tail_cnt;
  int main_grid, items;
  uint16_t *dk, *dv;
  KGeom g;
  float c2, scale;
};

// One 16-query half q8 of a dK/dV step: P = exp2(c2*S - L2) and dS = P * (dP - D) for this
// lane's key and queries qh*32 + 16*q8 + 8*hi + 0..7 (registers q8*8 .. q8*8+7 of s and dp),
// then the dV^T and dK^T products over those queries. ta: the transpose-read addresses of the
// Q tile for queries qh*32 ..; the dO tile sits two tiles further.
// Transpose-read addresses base + rel[k], formed right before each read block (an asm add is
// not merged with the others, so the sums hold registers only while the reads are issued).
template <int N>
__device__ __forceinline__ void tr_addrs(const uint32_t* rel, uint32_t base, uint32_t (&out)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) asm volatile("v_add_u32 %0, %1, %2" : "=v"(out[k]) : "s"(base), "v"(rel[k]));
}

template <int D, int DT, int Q8, typename NextLoads>
__device__ __forceinline__ void half_step(const uint32_t* trel, uint32_t qbase, const f32x4v_t (&l2r)[2],
                                          const f32x4v_t (&dr)[2], int hi, float c2, const f32x16_t& s,
                                          const f32x16_t& dp, f32x16_t* dk, f32x16_t* dv, NextLoads next_loads) {
  constexpr int TB = kBlock * D * 2;
  const f32x4v_t la = l2r[0], lb = l2r[1], da = dr[0], db = dr[1];
  const float lq[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
  const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
  bf16x8_t pb, dsb;
  // The exponential phase runs at raised wave priority (as in the forward): the two waves
  // sharing a SIMD then tend to overlap one's VALU work with the other's products.
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = exp2_fast(fmaf(s[Q8 * 8 + e], c2, -lq[e]));
    pb[e] = (__bf16)p;
    dsb[e] = (__bf16)(p * (dp[Q8 * 8 + e] - dd[e]));
  }
  __builtin_amdgcn_s_setprio(0);
  asm volatile("" ::: "memory");
  next_loads();  // the next half's L2 / D, once this half's are consumed
  asm volatile("" ::: "memory");
  // Two channel tiles' transposed operands at a time (fewer registers held by the reads).
#pragma unroll
  for (int h2 = 0; h2 < DT / 2; ++h2) {
    bf16x8_t ot[2];
    uint32_t ta[4];
    tr_addrs(trel + 4 * h2, qbase, ta);
    tr_chunks_at<2, 2 * TB + Q8 * 16 * D * 2>(ta, ot);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      dv[2 * h2 + e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ot[e], pb, dv[2 * h2 + e], 0, 0, 0);
  }
#pragma unroll
  for (int h2 = 0; h2 < DT / 2; ++h2) {
    bf16x8_t qt[2];
    uint32_t ta[4];
    tr_addrs(trel + 4 * h2, qbase, ta);
    tr_chunks_at<2, Q8 * 16 * D * 2>(ta, qt);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      dk[2 * h2 + e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt[e], dsb, dk[2 * h2 + e], 0, 0, 0);
  }
}

// One workgroup per key block j, four waves: wave (kh, qh) takes keys kh*32.. and queries
// qh*32.. of every query tile in the block's column list. Q and dO tiles (token-major) are
// double-buffered in LDS; the key block's V tile stays in LDS for the whole walk (the B
// operand of dP, read like a Q tile), its K rows in registers. Lane l's key is the one in LDS
// row kh*32 + l%32 of such a tile (the tiles' row permutation), and the tiles' L2 / D rows come
// straight from global memory by buffer loads (32 bytes of each per lane and 16-query half: the
// first half's after the S and dP products, the second's during the first half). The transposed
// Q and dO operands are read two channel tiles at a time. With V in registers as well, or four
// channel tiles' operands read at once, the kernel spilled at two waves per SIMD (20 and 6
// registers per lane).
template <int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dkdv(DkvArgs a) {
  constexpr int TB = kBlock * D * 2;
  constexpr int DT = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[5 * TB];  // Q0, Q1, dO0, dO1, V of block j
  const KGeom& g = a.g;
  const int nb = g.nb;
  const int t = threadIdx.x, lane = t & 63, hi = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kh = w & 1, qh = w >> 1;
  const int item = bwd_claim_item(a.main_grid, a.items, a.tail_cnt, reinterpret_cast<int*>(smem));
  if (item < 0) return;
  const int gi = ld_const(a.order, (long long)item);
  const long long bh = gi / nb;
  const int j = gi - (int)bh * nb;
  const long long col = bh * nb + j;
  const int cnt = min(max(ld_const(a.col_counts, col), 0), nb);
  const int k_local = kperm(kh * 32 + (lane & 31));

  const uint32_t head_bytes = (uint32_t)(g.N * D * 2);
  const i32x4_t qrs = make_rsrc(a.q + bh * g.N * D, head_bytes);
  const i32x4_t dors = make_rsrc(a.dout + bh * g.N * D, head_bytes);
  const uint32_t off = orig_tile_off<D>(t, g.Ws);
  const uint32_t stride = 512u * (uint32_t)g.Ws;
  // The V rows of this wave's keys, addressed like its Q rows (the swizzle repeats every 16
  // rows, so the two differ by a wave-uniform offset and share the per-lane offsets).
  const char* v_lds_q = smem + 4 * TB + (kh - qh) * 32 * D * 2;
  issue_rows<TB>(smem + 4 * TB, w, make_rsrc(a.v + bh * g.N * D, head_bytes), orig_tile_base<D>(g, j), off, stride);
  bf16x8_t kb[D / 16];
  {
    const long long n = token_of(g, j, k_local);  // its token in the original order
    const uint16_t* krow = a.k + (bh * g.N + n) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kb[ks] = *reinterpret_cast<const bf16x8_t*>(krow + ks * 16);
  }
  const i32x4_t l2rs = make_rsrc(a.L2 + bh * g.N, (uint32_t)(g.N * 4));
  const i32x4_t drs = make_rsrc(a.Dm + bh * g.N, (uint32_t)(g.N * 4));
  const int rows_off = (qh * 32 + 8 * hi) * 4;  // byte offset of this lane's first query in a tile

  f32x16_t dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  // Loads of query tile i into slot sl: Q and dO tiles.
  auto issue = [&](int sl, int i) {
    const uint32_t base = orig_tile_base<D>(g, i);
    issue_rows<TB>(smem + sl * TB, w, qrs, base, off, stride);
    issue_rows<TB>(smem + (2 + sl) * TB, w, dors, base, off, stride);
  };
  // Q^T / dO^T operand reads: offsets inside a Q tile for each channel tile (queries qh*32 ..);
  // the second 16 queries and the dO tile (two slots further) are immediate offsets.
  uint32_t trel[2 * DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) tr_rel<D>(dt, qh * 32, lane, trel[2 * dt], trel[2 * dt + 1]);

  const int32_t* lst = a.col_lists + col * nb;
  int i_cur = cnt > 0 ? min(max(ld_const(lst, 0), 0), nb - 1) : 0;
  if (cnt > 0) issue(0, i_cur);
  for (int u = 0; u < cnt; ++u) {
    wait_vm_lgkm_barrier();  // tile u (and, first, the V tile) has landed; every wave is done with tile u-1
    const int i_next = u + 1 < cnt ? min(max(ld_const(lst, u + 1), 0), nb - 1) : -1;
    const char* q_lds = smem + (u & 1) * TB;
    const char* do_lds = smem + (2 + (u & 1)) * TB;

    // S = Q K^T and dP = dO V^T for queries qh*32.. (rows) and this lane's key (column):
    // register r holds query qh*32 + 16*(r/8) + 8*hi + r%8.
    f32x16_t s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk<D>(q_lds, qh, lane, ks), kb[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk<D>(do_lds, qh, lane, ks),
                                                   row_chunk<D>(v_lds_q, qh, lane, ks), dp, 0, 0, 0);
    }
    // The next tile's loads go out here, after the products that read the registers this
    // kernel keeps in scratch: a wait for those reloads would otherwise also wait for the
    // prefetch, which shares their counter.
    // L2 and D of queries qh*32 + 16*q8 + 8*hi + 0..7 of tile u, each half q8's loaded just
    // before the half before it, so that they hold no registers during the products.
    const int tile_off = i_cur * kBlock * 4;
    f32x4v_t l2r[2], dr[2];
    l2r[0] = raw_buffer_load_f32x4(l2rs, rows_off, tile_off, 0);
    l2r[1] = raw_buffer_load_f32x4(l2rs, rows_off + 16, tile_off, 0);
    dr[0] = raw_buffer_load_f32x4(drs, rows_off, tile_off, 0);
    dr[1] = raw_buffer_load_f32x4(drs, rows_off + 16, tile_off, 0);
    asm volatile("" ::: "memory");
    if (i_next >= 0) issue((u + 1) & 1, i_next);
    // Per 16-query half q8: P and dS for this lane's key, then dV^T += dO^T P and
    // dK^T += Q^T dS over those queries, the transposed operands from transpose loads (one
    // half's operands live at a time).
    const uint32_t qbase = __builtin_amdgcn_readfirstlane(lds_offset(q_lds));
    f32x4v_t l2s[2], ds[2];
    half_step<D, DT, 0>(trel, qbase, l2r, dr, hi, a.c2, s, dp, dk, dv, [&] {
      l2s[0] = raw_buffer_load_f32x4(l2rs, rows_off + 64, tile_off, 0);
      l2s[1] = raw_buffer_load_f32x4(l2rs, rows_off + 80, tile_off, 0);
      ds[0] = raw_buffer_load_f32x4(drs, rows_off + 64, tile_off, 0);
      ds[1] = raw_buffer_load_f32x4(drs, rows_off + 80, tile_off, 0);
    });
    half_step<D, DT, 1>(trel, qbase, l2s, ds, hi, a.c2, s, dp, dk, dv, [] {});
    i_cur = i_next;
  }
  // Waves (kh, 0) and (kh, 1) hold partial dK^T and dV^T over their query halves: wave qh = 0
  // finishes dK, wave qh = 1 finishes dV; each hands the other its partial.
  wait_vm_lgkm_barrier();
  float* xch = reinterpret_cast<float*>(smem);
  float* mine = xch + (kh * 2 + qh) * (DT * 16 * 64);
  const float* theirs = xch + (kh * 2 + (1 - qh)) * (DT * 16 * 64);
  if (qh == 0)
    stash<0, DT>(mine, dv, lane);
  else
    stash<0, DT>(mine, dk, lane);
  wait_vm_lgkm_barrier();
  if (qh == 0) {
    unstash_add<0, DT>(theirs, dk, lane);
    write_rows<D, DT>(a.dk, g, bh, j, k_local, dk, 0, a.scale, hi);
  } else {
    unstash_add<0, DT>(theirs, dv, lane);
    write_rows<D, DT>(a.dv, g, bh, j, k_local, dv, 0, 1.0f, hi);
  }
}

// ------------------------------------------------------------------- float32 path
// Plain float32 arithmetic throughout (no rounding of P or dS), two threads per row as in the
// float32 forward: thread pair (2r, 2r+1) holds row r, each half of the channels; the dot
// products are combined with one lane swap. Inputs and outputs in the original token order.

// D[m] = <dO[n], O[n]> (float32) and the natural-log lse of fractal row m of token n.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_delta_f32(const float* __restrict__ o, const float* __restrict__ dout,
                                                       const float* __restrict__ lse, float* __restrict__ Dm,
                                                       float* __restrict__ Lr, KGeom g) {
  constexpr int LPR = D / 4;
  const long long rows = (long long)g.B * g.H * g.N;
  const long long row = ((long long)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const long long bh = row / g.N;
    const int m = (int)(row - bh * g.N);
    const long long off = (bh * g.N + token_of(g, m / kBlock, m % kBlock)) * D + sub * 4;
    const float4 a = *reinterpret_cast<const float4*>(o + off);
    const float4 b = *reinterpret_cast<const float4*>(dout + off);
    acc = fmaf(a.x, b.x, fmaf(a.y, b.y, fmaf(a.z, b.z, a.w * b.w)));
  }
#pragma unroll
  for (int s = 1; s < LPR; s <<= 1) acc += __shfl_xor(acc, s);
  if (row < rows && sub == 0) {
    Dm[row] = acc;
    Lr[row] = lse[row];
  }
}

// Stage the 64 rows of block blk (original order) of one head into an LDS tile [64][D].
template <int D>
__device__ __forceinline__ void stage_rows_f32(float* tile, const float* head, const KGeom& g, int blk) {
  for (int u = threadIdx.x; u < kBlock * D / 4; u += 128) {
    const int rr = u / (D / 4), c4 = (u % (D / 4)) * 4;
    *reinterpret_cast<float4*>(tile + rr * D + c4) =
        *reinterpret_cast<const float4*>(head + token_of(g, blk, rr) * D + c4);
  }
}

struct BwdF32Args {
  const float *q, *k, *v, *dout, *Dm, *Lr;
  const int32_t *counts, *lists, *col_counts, *col_lists;
  float *dq, *dk, *dv;
  KGeom g;
  float scale;
};

// dQ: one workgroup per query block, walking its kept list.
template <int D>
__global__ __launch_bounds__(128) void k_bwd_dq_f32(BwdF32Args a) {
  constexpr int H2 = D / 2;
  __shared__ __attribute__((aligned(16))) float ks[kBlock * D];
  __shared__ __attribute__((aligned(16))) float vs[kBlock * D];
  const KGeom& g = a.g;
  const int nb = g.nb, t = threadIdx.x, r = t >> 1, half = t & 1;
  const long long bh = blockIdx.x / nb;
  const int i = blockIdx.x - (int)(bh * nb);
  const long long row = bh * nb + i;
  const int cnt = min(max(a.counts[row], 0), nb);
  const long long n = token_of(g, i, r);
  const float* qrow = a.q + (bh * g.N + n) * D + half * H2;
  const float* drow = a.dout + (bh * g.N + n) * D + half * H2;
  float qv[H2], dov[H2], acc[H2];
#pragma unroll
  for (int c = 0; c < H2; ++c) {
    qv[c] = qrow[c];
    dov[c] = drow[c];
    acc[c] = 0.f;
  }
  const long long m = bh * g.N + (long long)i * kBlock + r;
  const float lq = a.Lr[m], dd = a.Dm[m];
  const float* kh = a.k + bh * g.N * D;
  const float* vh = a.v + bh * g.N * D;
  for (int u = 0; u < cnt; ++u) {
    const int j = min(max(a.lists[row * nb + u], 0), nb - 1);
    stage_rows_f32<D>(ks, kh, g, j);
    stage_rows_f32<D>(vs, vh, g, j);
    __syncthreads();
    for (int kk = 0; kk < kBlock; ++kk) {
      const float* krow = ks + kk * D + half * H2;
      const float* vrow = vs + kk * D + half * H2;
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int c = 0; c < H2; ++c) {
        sp = fmaf(qv[c], krow[c], sp);
        dpp = fmaf(dov[c], vrow[c], dpp);
      }
      const float so = __shfl_xor(sp, 1), dpo = __shfl_xor(dpp, 1);
      const float s = half ? so + sp : sp + so;
      const float dp = half ? dpo + dpp : dpp + dpo;
      const float p = expf(s * a.scale - lq);
      const float ds = p * (dp - dd);
#pragma unroll
      for (int c = 0; c < H2; ++c) acc[c] = fmaf(ds, krow[c], acc[c]);
    }
    __syncthreads();
  }
  float* orow = a.dq + (bh * g.N + n) * D + half * H2;
#pragma unroll
  for (int c = 0; c < H2; ++c) orow[c] = acc[c] * a.scale;
}

// dK, dV: one workgroup per key block, walking its column list.
template <int D>
__global__ __launch_bounds__(128) void k_bwd_dkdv_f32(BwdF32Args a) {
  constexpr int H2 = D / 2;
  __shared__ __attribute__((aligned(16))) float qs[kBlock * D];
  __shared__ __attribute__((aligned(16))) float dos[kBlock * D];
  __shared__ float ls[kBlock], dds[kBlock];
  const KGeom& g = a.g;
  const int nb = g.nb, t = threadIdx.x, r = t >> 1, half = t & 1;
  const long long bh = blockIdx.x / nb;
  const int j = blockIdx.x - (int)(bh * nb);
  const long long col = bh * nb + j;
  const int cnt = min(max(a.col_counts[col], 0), nb);
  const long long n = token_of(g, j, r);
  const float* krow = a.k + (bh * g.N + n) * D + half * H2;
  const float* vrow = a.v + (bh * g.N + n) * D + half * H2;
  float kv[H2], vv[H2], dk[H2], dv[H2];
#pragma unroll
  for (int c = 0; c < H2; ++c) {
    kv[c] = krow[c];
    vv[c] = vrow[c];
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  const float* qh = a.q + bh * g.N * D;
  const float* dh = a.dout + bh * g.N * D;
  for (int u = 0; u < cnt; ++u) {
    const int i = min(max(a.col_lists[col * nb + u], 0), nb - 1);
    stage_rows_f32<D>(qs, qh, g, i);
    stage_rows_f32<D>(dos, dh, g, i);
    if (t < kBlock) {
      ls[t] = a.Lr[bh * g.N + (long long)i * kBlock + t];
      dds[t] = a.Dm[bh * g.N + (long long)i * kBlock + t];
    }
    __syncthreads();
    for (int qq = 0; qq < kBlock; ++qq) {
      const float* qrow = qs + qq * D + half * H2;
      const float* drow = dos + qq * D + half * H2;
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int c = 0; c < H2; ++c) {
        sp = fmaf(qrow[c], kv[c], sp);
        dpp = fmaf(drow[c], vv[c], dpp);
      }
      const float so = __shfl_xor(sp, 1), dpo = __shfl_xor(dpp, 1);
      const float s = half ? so + sp : sp + so;
      const float dp = half ? dpo + dpp : dpp + dpo;
      const float p = expf(s * a.scale - ls[qq]);
      const float ds = p * (dp - dds[qq]);
#pragma unroll
      for (int c = 0; c < H2; ++c) {
        dv[c] = fmaf(p, drow[c], dv[c]);
        dk[c] = fmaf(ds, qrow[c], dk[c]);
      }
    }
    __syncthreads();
  }
  float* dkrow = a.dk + (bh * g.N + n) * D + half * H2;
  float* dvrow = a.dv + (bh * g.N + n) * D + half * H2;
#pragma unroll
  for (int c = 0; c < H2; ++c) {
    dkrow[c] = dk[c] * a.scale;
    dvrow[c] = dv[c];
  }
}

}  // namespace

hipError_t launch_sparse_attn_bwd(const KGeom& g, int dtype, float scale, const void* q, const void* k,
                                  const void* v, const void* o, const void* dout, const float* lse,
                                  const uint32_t* words, const int32_t* counts, const int32_t* lists, void* dq,
                                  void* dk, void* dv, const BwdWorkspace& ws, hipStream_t s) {
  // The kernels read Q, K, V and dO in the original token order (64-token blocks gathered as
  // their 8 runs of 8 tokens), so no reordered copies are made.
  hipError_t e;

  const long long rows = (long long)g.B * g.H * g.N;
  const unsigned bhs = (unsigned)(g.B * g.H);
  if (dtype == ABLA_F32) {
    const unsigned fgrid = (unsigned)((rows * (g.d / 4) + 255) / 256);
    const float* of = static_cast<const float*>(o);
    const float* dof = static_cast<const float*>(dout);
    if (g.d == 128)
      k_bwd_delta_f32<128><<<dim3(fgrid), 256, 0, s>>>(of, dof, lse, ws.D, ws.L2, g);
    else
      k_bwd_delta_f32<64><<<dim3(fgrid), 256, 0, s>>>(of, dof, lse, ws.D, ws.L2, g);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_col_lists<<<dim3((unsigned)((g.nb + kColWaves - 1) / kColWaves) * bhs), 64 * kColWaves, 0, s>>>(
        words, ws.col_counts, ws.col_lists, g.nb, (g.nb + 31) / 32);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    BwdF32Args fa{static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), dof,
                  ws.D, ws.L2, counts, lists, ws.col_counts, ws.col_lists, static_cast<float*>(dq),
                  static_cast<float*>(dk), static_cast<float*>(dv), g, scale};
    const dim3 grid((unsigned)((long long)bhs * g.nb));
    if (g.d == 128) {
      k_bwd_dq_f32<128><<<grid, 128, 0, s>>>(fa);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      k_bwd_dkdv_f32<128><<<grid, 128, 0, s>>>(fa);
    } else {
      k_bwd_dq_f32<64><<<grid, 128, 0, s>>>(fa);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      k_bwd_dkdv_f32<64><<<grid, 128, 0, s>>>(fa);
    }
    return hipGetLastError();
  }
  const int lpr = g.d / 8;
  const unsigned dgrid = (unsigned)((rows * lpr + 255) / 256);
  const uint16_t* o16 = static_cast<const uint16_t*>(o);
  const uint16_t* do16 = static_cast<const uint16_t*>(dout);
  if (g.d == 128)
    k_bwd_delta<128><<<dim3(dgrid), 256, 0, s>>>(o16, do16, lse, ws.D, ws.L2, g);
  else
    k_bwd_delta<64><<<dim3(dgrid), 256, 0, s>>>(o16, do16, lse, ws.D, ws.L2, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_col_lists<<<dim3((unsigned)((g.nb + kColWaves - 1) / kColWaves) * bhs), 64 * kColWaves, 0, s>>>(
      words, ws.col_counts, ws.col_lists, g.nb, (g.nb + 31) / 32);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const float c2 = scale * kLog2e;
  const int items = (int)((long long)bhs * g.nb);
  const int main_grid = max(0, items / 8 - kBwdQueueTail) * 8;
  const dim3 grid((unsigned)(main_grid + kBwdTailOversub * (items - main_grid)));
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  k_bwd_order<<<8, 1024, 0, s>>>(counts, ws.order, ws.tail_cnt, g, (int)bhs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  DqArgs qa{q16, k16, v16, do16, ws.D, ws.L2, counts, lists, ws.order, ws.tail_cnt, main_grid, items,
            static_cast<uint16_t*>(dq), g, c2, scale};
  if (g.d == 128)
    k_bwd_dq<128><<<grid, kBwdThreads, 0, s>>>(qa);
  else
    k_bwd_dq<64><<<grid, kBwdThreads, 0, s>>>(qa);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_bwd_order<<<8, 1024, 0, s>>>(ws.col_counts, ws.order, ws.tail_cnt, g, (int)bhs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  DkvArgs ka{k16, v16, q16, do16, ws.D, ws.L2, ws.col_counts, ws.col_lists, ws.order, ws.tail_cnt, main_grid,
             items, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), g, c2, scale};
  if (g.d == 128)
    k_bwd_dkdv<128><<<grid, kBwdThreads, 0, s>>>(ka);
  else
    k_bwd_dkdv<64><<<grid, kBwdThreads, 0, s>>>(ka);
  return hipGetLastError();
}

}  // namespace abla
