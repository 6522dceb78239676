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
  const int32_t* order;  // pair ids, longest first within each (b, h)
  uint16_t* out;
  float* lse;
  KGeom g;
  int pairs;    // query-block pairs per (b, h): ceil(T/2) * nbh * nbw
  int grid;     // total workgroups
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
  static constexpr int KLOADS = KUNITS / 256;     // per thread per tile
  static constexpr int VLOADS = VUNITS / 256;
};

// 16-byte chunk swizzles (bank-conflict-free MFMA operand reads).
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

// LDS row r of the K tile holds key kperm(r): rows 4-7 and 8-11 of every 16 are swapped,
// which makes each lane's S^T registers cover 8 consecutive keys (see the file header).
__device__ __forceinline__ int kperm(int r) {
  const int m = r & 15;
  const int s = (m >= 4 && m < 8) ? 4 : ((m >= 8 && m < 12) ? -4 : 0);
  return r + s;
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

// Read-only metadata (counts, lists, order) through the constant address space so that
// wave-uniform reads become scalar loads: their waits then do not wait for the
// outstanding K/V tile loads.
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ __forceinline__ int ld_const(const int32_t* p, long long i) {
  return ((cint_ptr)p)[i];
}

// Waits and barriers written with builtins the compiler's wait-count pass understands
// (gfx9 s_waitcnt encoding: vmcnt [3:0]+[15:14], expcnt [6:4], lgkmcnt [11:8]), and
// without a release fence: a fence would also wait for the next tile's loads that are
// meant to stay in flight. Empty asm statements keep memory accesses on their side.
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(N));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lgkm_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Rescale the running output only when a row maximum grows by more than 2^8 in the
// exponent; below that the stale maximum keeps every probability <= 256.
constexpr float kRescaleLog2 = 8.0f;

// Issue this thread's 16-byte global->LDS loads of key tile j into LDS stage `stage`.
template <int D>
__device__ __forceinline__ void issue_tile(char* smem, int stage, int w, const char* kbase, const char* vbase,
                                           int j, const uint32_t* koff, const uint32_t* voff) {
  using TT = Tile<D>;
  const char* kb = kbase + (long long)j * TT::KBYTES;
  const char* vb = vbase + (long long)j * TT::VBYTES;
  char* dst = smem + stage * TT::BYTES + w * 64 * 16;
#pragma unroll
  for (int it = 0; it < TT::KLOADS; ++it)
    __builtin_amdgcn_global_load_lds(kb + koff[it], (lds_ptr_t)(dst + it * 256 * 16), 16, 0, 0);
#pragma unroll
  for (int it = 0; it < TT::VLOADS; ++it)
    __builtin_amdgcn_global_load_lds(vb + voff[it], (lds_ptr_t)(dst + TT::KBYTES + it * 256 * 16), 16, 0, 0);
}

// The union of two ascending kept lists, walked in ascending block order.
struct ListPair {
  const int32_t* la;
  const int32_t* lb;
  int ca, cb, nb;
  int pa, pb;

  __device__ __forceinline__ bool next(int& j, bool& need_a, bool& need_b) {
    const int ja = pa < ca ? min(max(ld_const(la, pa), 0), nb - 1) : 0x7fffffff;
    const int jb = pb < cb ? min(max(ld_const(lb, pb), 0), nb - 1) : 0x7fffffff;
    if (ja == 0x7fffffff && jb == 0x7fffffff) return false;
    j = min(ja, jb);
    need_a = ja == j;
    need_b = jb == j;
    pa += need_a;
    pb += need_b;
    return true;
  }
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bf16(AttnArgs a) {
  using TT = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * TT::BYTES];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;          // waves 0,1: block A; waves 2,3: block B
  const int hi = lane >> 5;
  const KGeom& g = a.g;
  const int nb = g.nb;
  const int F = g.nbh * g.nbw;

  // XCD-aware placement: consecutive logical items run on the same XCD (dispatch is
  // round-robin over 8 XCDs), so one XCD's L2 serves one head's K/V at a time.
  const int p = blockIdx.x;
  const int base = a.grid >> 3, rem = a.grid & 7, x = p & 7;
  const int logical = x * base + min(x, rem) + (p >> 3);
  const int bh = logical / a.pairs;
  const int pos = logical - bh * a.pairs;
  const int pair = ld_const(a.order, (long long)bh * a.pairs + pos);
  const int blk_a = (pair / F) * 2 * F + pair % F;
  const int blk_b = blk_a + F < nb ? blk_a + F : -1;
  const int my_blk = (w < 2) ? blk_a : blk_b;
  const bool active = my_blk >= 0;

  const long long row_a = (long long)bh * nb + blk_a;
  const long long row_b = (long long)bh * nb + (blk_b >= 0 ? blk_b : blk_a);
  const int ca = min(max(ld_const(a.counts, row_a), 0), nb);
  const int cb = blk_b >= 0 ? min(max(ld_const(a.counts, row_b), 0), nb) : 0;
  const int32_t* la = a.lists + row_a * nb;
  const int32_t* lb = a.lists + row_b * nb;

  const int q_local = (w & 1) * 32 + (lane & 31);

  // Q operand: lane holds Q[q_local][ks*16 + 8*hi .. +7] for every k-step.
  bf16x8_t qv[D / 16];
  if (active) {
    const uint16_t* qrow = a.q + ((long long)bh * g.N + (long long)my_blk * kBlock + q_local) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qv[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
  }

  // Per-thread byte offsets of its 16-byte loads inside a tile (the same for every tile).
  uint32_t koff[TT::KLOADS], voff[TT::VLOADS];
#pragma unroll
  for (int it = 0; it < TT::KLOADS; ++it) {
    const int u = it * 256 + t;
    const int r = u / TT::KCH, pc = u % TT::KCH;
    koff[it] = (uint32_t)(kperm(r) * D * 2 + ((pc ^ k_swz<D>(r)) * 16));
  }
#pragma unroll
  for (int it = 0; it < TT::VLOADS; ++it) {
    const int u = it * 256 + t;
    const int dd = u >> 3, pc = u & 7;
    voff[it] = (uint32_t)(dd * kBlock * 2 + ((pc ^ v_swz(dd)) * 16));
  }
  const char* kbase = reinterpret_cast<const char*>(a.k + (long long)bh * g.N * D);
  const char* vbase = reinterpret_cast<const char*>(a.vt + (long long)bh * nb * D * kBlock);
  ListPair lp{la, lb, ca, cb, nb, 0, 0};

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;  // in log2 units (scores * c2)
  float l_run = 0.f;

  int j_cur;
  bool na_cur, nb_cur;
  bool have = lp.next(j_cur, na_cur, nb_cur);
  if (have) issue_tile<D>(smem, 0, w, kbase, vbase, j_cur, koff, voff);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // Q registers and the first tile
  int stage = 0;
  while (have) {
    int j_nxt;
    bool na_nxt, nb_nxt;
    const bool have_nxt = lp.next(j_nxt, na_nxt, nb_nxt);
    if (have_nxt) {
      issue_tile<D>(smem, stage ^ 1, w, kbase, vbase, j_nxt, koff, voff);
      wait_vm_barrier<TT::KLOADS + TT::VLOADS>();  // this tile's loads done, the next tile's in flight
    } else {
      wait_vm_barrier<0>();
    }

    const bool mine = (w < 2) ? na_cur : nb_cur;
    if (mine) {
      const char* ks_lds = smem + stage * TT::BYTES;
      const char* vs_lds = ks_lds + TT::KBYTES;
      // S^T = K Q^T for the two 32-key halves of the tile.
      f32x16_t sacc[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kh][r] = 0.f;
        const int krow = kh * 32 + (lane & 31);
        const char* rowp = ks_lds + krow * (D * 2);
        const int swz = k_swz<D>(krow);
        bf16x8_t kv[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          kv[ks] = *reinterpret_cast<const bf16x8_t*>(rowp + (((ks * 2 + hi) ^ swz) * 16));
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv[ks], qv[ks], sacc[kh], 0, 0, 0);
      }

      // Online softmax in log2 units for this lane's query.
      float mx = sacc[0][0];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kh][r]);
      mx = swap_max(mx) * a.c2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      float psum = 0.f;
      bf16x8_t pb[4];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = exp2_fast(fmaf(sacc[kh][r], a.c2, -m_run));
          psum += pv;
          pb[kh * 2 + (r >> 3)][r & 7] = (__bf16)pv;
        }
      l_run += psum;

      // O^T += V^T P^T: lane reads 8 consecutive keys of one channel row.
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int dd = dt * 32 + (lane & 31);
        const char* vrow = vs_lds + dd * (kBlock * 2);
        const int swz = v_swz(dd);
        bf16x8_t vv[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          vv[kk] = *reinterpret_cast<const bf16x8_t*>(vrow + (((2 * kk + hi) ^ swz) * 16));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[kk], pb[kk], o[dt], 0, 0, 0);
      }
    }
    wait_lgkm_barrier();  // every wave is done reading this stage before it is refilled
    have = have_nxt;
    j_cur = j_nxt;
    na_cur = na_nxt;
    nb_cur = nb_nxt;
    stage ^= 1;
  }

  if (!active) return;
  // Epilogue: normalise, round once to bf16, write (original order if asked).
  const int cnt = (w < 2) ? ca : cb;
  const float l_tot = swap_sum(l_run);
  const float inv = cnt > 0 ? 1.0f / l_tot : 0.f;
  const long long n = a.orig ? token_of(g, my_blk, q_local) : (long long)my_blk * kBlock + q_local;
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
    a.lse[(long long)bh * g.N + (long long)my_blk * kBlock + q_local] =
        cnt > 0 ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
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

// In place: h[v] <- sum of h[v'] for v' > v (the first position of key v in descending
// order). 1024 threads, each owning a contiguous run of keys; `part` holds 16 ints.
__device__ void desc_exclusive_scan(int* h, int n, int* part) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int per = (n + 1023) / 1024;
  const int lo = t * per, hi = min(lo + per, n);
  int local = 0;
  for (int v = lo; v < hi; ++v) local += h[v];
  int incl = local;  // inclusive suffix sum over the lanes of this wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_down(incl, o);
    if (lane + o < 64) incl += x;
  }
  if (lane == 0) part[wv] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = wv + 1; w < 16; ++w) run += part[w];
  for (int v = hi - 1; v >= lo; --v) {
    const int c = h[v];
    h[v] = run;
    run += c;
  }
  __syncthreads();
}

// Longest-first order of the query-block pairs (i, i + nbh*nbw) of each (b, h): a counting
// sort on the pair's total kept count. Pair p covers blocks a = (p / F)*2F + p % F and a + F.
__global__ __launch_bounds__(1024) void k_pair_order(const int32_t* __restrict__ counts, int32_t* __restrict__ order,
                                                     int nb, int F, int pairs) {
  __shared__ int hist[2 * kMaxBlocks + 1];
  __shared__ int scan_part[16];
  const int t = threadIdx.x;
  const long long bh = blockIdx.x;
  const int32_t* c = counts + bh * nb;
  const int kmax = 2 * nb;
  auto key = [&](int pr) {
    const int blk = (pr / F) * 2 * F + pr % F;
    int k = min(max(c[blk], 0), nb);
    if (blk + F < nb) k += min(max(c[blk + F], 0), nb);
    return k;
  };
  for (int v = t; v <= kmax; v += 1024) hist[v] = 0;
  __syncthreads();
  for (int pr = t; pr < pairs; pr += 1024) atomicAdd(&hist[key(pr)], 1);
  __syncthreads();
  desc_exclusive_scan(hist, kmax + 1, scan_part);
  for (int pr = t; pr < pairs; pr += 1024) {
    const int pos = atomicAdd(&hist[key(pr)], 1);
    order[bh * pairs + pos] = pr;
  }
}

// Longest-first order of the query blocks of each (b, h), for the float32 path.
__global__ __launch_bounds__(1024) void k_row_order(const int32_t* __restrict__ counts, int32_t* __restrict__ order,
                                                    int nb) {
  __shared__ int hist[kMaxBlocks + 1];
  __shared__ int scan_part[16];
  const int t = threadIdx.x;
  const long long bh = blockIdx.x;
  const int32_t* c = counts + bh * nb;
  for (int v = t; v <= nb; v += 1024) hist[v] = 0;
  __syncthreads();
  for (int r = t; r < nb; r += 1024) atomicAdd(&hist[min(max(c[r], 0), nb)], 1);
  __syncthreads();
  desc_exclusive_scan(hist, nb + 1, scan_part);
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
  if (dtype == ABLA_BF16) {
    const int F = g.nbh * g.nbw;
    const int pairs = ((g.T + 1) / 2) * F;
    k_pair_order<<<dim3(bhs), 1024, 0, s>>>(counts, row_order, g.nb, F, pairs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
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
    a.pairs = pairs;
    a.grid = (int)((long long)bhs * pairs);
    a.scale = scale;
    a.c2 = scale * 1.4426950408889634f;
    a.orig = out_original_order;
    const dim3 grid((unsigned)a.grid);
    if (g.d == 128)
      k_attn_bf16<128><<<grid, 256, 0, s>>>(a);
    else
      k_attn_bf16<64><<<grid, 256, 0, s>>>(a);
  } else {
    k_row_order<<<dim3(bhs), 1024, 0, s>>>(counts, row_order, g.nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
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
    const dim3 grid((unsigned)((long long)bhs * g.nb));
    if (g.d == 128)
      k_attn_f32<128><<<grid, 128, 0, s>>>(a);
    else
      k_attn_f32<64><<<grid, 128, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace abla
