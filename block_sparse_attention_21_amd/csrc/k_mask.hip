// Content-adaptive block mask: reduced attention over pooled blocks, a per-row
// cut, the sliding-tile union, bit packing and ascending kept lists.
//
// NABLA, Method: "reduced attention" (a full attention map over the pooled
// block vectors), "CDF thresholding" (each row ranked by probability; the
// blocks needed for the row's cumulative probability to reach thr are kept,
// per head and per input), hybrid with STA (M = M_nabla OR M_STA).
// DynamicRad, Methodology A, Dynamic-Threshold mode: the pre-softmax logits
// serve as importance and are filtered by a threshold; Static-Ratio mode: no
// scores, a share of each key frame's blocks fixed by temporal distance.
//
// Two kernels:
//  k_scores  S = pool_scale * Qbar Kbar^T per (b, h), a float64 matrix-core
//            GEMM written to the caller's workspace (fixed summation order).
//  k_select  one workgroup per row (b, h, i): row max, softmax, then either
//            the CDF cut or the logit threshold; OR the STA window; pack bits,
//            count, list. The CDF cut ranks the blocks by (P descending, j
//            ascending) with P's full float64 value as the sort key, and finds
//            the last kept rank: the smallest key K that has a kept block, and
//            how many of the blocks tied at K are kept (the lowest indices
//            first). Two algorithms give the same bits: a radix select over the
//            keys with exact mass histograms (8-bit digits below the row's
//            common key prefix, one bucket per thread) followed by a tie count,
//            or an LDS-resident bitonic sort of (key, index) pairs followed by
//            an exclusive prefix sum.
//
// The decisions are taken in float64 so that two blocks whose probabilities
// agree to float32 precision are still ranked as exactly as the definition
// asks. The prefix sum runs on integers: each probability is converted
// exactly to a 2^-62 fixed-point value, so the cumulative mass before every
// rank is an exact, order-independent sum.
#include <math.h>

#include "common.h"

namespace abla {
namespace {

// ---------------------------------------------------------------- scores
// S = pool_scale * Qbar Kbar^T on the float64 matrix cores (v_mfma_f64_16x16x4_f64,
// same peak rate as float64 FMA but a quarter of the operand traffic per FMA).
// Operand layout of one 16x16x4 product: lane l holds A[l % 16][l / 16] and
// B[l / 16][l % 16]; the result register r of lane l is D[4r + l / 16][l % 16].
// A workgroup computes a TM x TM tile: at TM = 32 one wave takes it whole as 2 x 2 16x16
// tiles; at TM = 128 four waves each take a 64 x 64 quarter as 4 x 4 tiles. The reduction
// runs in chunks of 16 channels, the next chunk's operands loaded after this chunk's
// products (no second register buffer: the lower register count lets more waves hide the
// load latency). Within a chunk,
// product step s uses channel k0 + 4*(l / 16) + s in lane l for both operands, so every
// output element sums its 128 (or 64) products in one fixed order, and two identical
// Kbar rows give bit-identical scores.
typedef double f64x4_t __attribute__((ext_vector_type(4)));

//
// The tiles are numbered in (b, h, tile row, tile column) order, tpr * tpr per (b, h); a
// one-dimensional launch covers the tiles from `base` on. (Giving each XCD a contiguous eighth
// of the tiles, so that it reads the pooled means of only one or two heads, measured 1-2%
// slower at 480p and 1% faster at 720p: the plain order stays.)
template <int TM, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_scores(
    const double* __restrict__ qbar, const double* __restrict__ kbar, double* __restrict__ S, int nb, double scale,
    int tpr, int base) {
  static_assert(TM == 32 || TM == 128, "one wave per 32 x 32 tile, or four per 128 x 128 tile");
  constexpr int NT = TM == 32 ? 2 : 4;  // 16x16 tiles per wave side
  constexpr int NC = D / 16;            // channel chunks
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tile = base + (int)blockIdx.x;
  const int per_head = tpr * tpr;
  const long long bh = tile / per_head;
  const int it = (tile - (int)bh * per_head) / tpr;
  const int jt = tile - (int)bh * per_head - it * tpr;
  const int i0 = it * TM + (TM == 32 ? 0 : (w >> 1) * 64);
  const int j0 = jt * TM + (TM == 32 ? 0 : (w & 1) * 64);
  const double* qh = qbar + bh * nb * D;
  const double* kh = kbar + bh * nb * D;

  f64x4_t acc[NT][NT];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f64x4_t{0.0, 0.0, 0.0, 0.0};

  double av[NT][4], bv[NT][4];
  auto load = [&](int k0, double (&qa)[NT][4], double (&kb)[NT][4]) {
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const int i = i0 + a * 16 + r16;
      double2 x = make_double2(0.0, 0.0), y = x;
      if (i < nb) {
        const double2* src = reinterpret_cast<const double2*>(qh + (long long)i * D + k0 + 4 * kq);
        x = src[0];
        y = src[1];
      }
      qa[a][0] = x.x; qa[a][1] = x.y; qa[a][2] = y.x; qa[a][3] = y.y;
    }
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int j = j0 + b * 16 + r16;
      double2 x = make_double2(0.0, 0.0), y = x;
      if (j < nb) {
        const double2* src = reinterpret_cast<const double2*>(kh + (long long)j * D + k0 + 4 * kq);
        x = src[0];
        y = src[1];
      }
      kb[b][0] = x.x; kb[b][1] = x.y; kb[b][2] = y.x; kb[b][3] = y.y;
    }
  };
  load(0, av, bv);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a][st], bv[b][st], acc[a][b], 0, 0, 0);
    if (c + 1 < NC) load((c + 1) * 16, av, bv);
  }
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + a * 16 + 4 * r + kq;
      if (i >= nb) continue;
#pragma unroll
      for (int b = 0; b < NT; ++b) {
        const int j = j0 + b * 16 + r16;
        if (j < nb) S[(bh * nb + i) * nb + j] = acc[a][b][r] * scale;
      }
    }
}

// ---------------------------------------------------------------- select
constexpr int kSelThreads = 256;  // threads per row for rows of more than 768 blocks

struct SelArgs {
  int mode;        // ABLA_MASK_CDF / ABLA_MASK_DYN / ABLA_MASK_STATIC
  int cut;         // ABLA_CUT_RADIX / ABLA_CUT_BITONIC
  int cdf_all;     // thr >= 1
  int cdf_none;    // thr <= 0
  unsigned long long thr_fx;  // thr in 2^-62 fixed point (CDF, 0 < thr < 1)
  double tau;
  int sta_on, rt, rh, rw;
  int np;          // bitonic size: power of two >= nb
  int W;           // words per row
  double gamma;    // STATIC: retention decay per frame of distance
  int floor_k;     // STATIC: ceil(F * lambda), F = blocks per frame
  long long row0;  // first row of this launch (launches of at most 2^22 rows)
};

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sort key of a probability: its float64 bits. P >= 0, so the sign bit is 0 and the integer
// order of the bits is the order of the values; equal probabilities give equal keys, and the
// ranking breaks those ties by the lower block index separately (tie_kept, the tie ranks).
__device__ __forceinline__ unsigned long long make_key(double p) {
  return (unsigned long long)__double_as_longlong(p);
}

// Probability of a key in 2^-62 fixed point, floor(P * 2^62) (P <= 1: no overflow).
__device__ __forceinline__ unsigned long long mass_fx(unsigned long long key) {
  return (unsigned long long)(__longlong_as_double((long long)key) * 4611686018427387904.0);
}

// Of n blocks tied at a key of mass m, ranked after blocks of total mass `above` (< thr):
// how many are kept. Tie rank r is kept iff above + r*m < thr, i.e. r < ceil((thr - above)/m).
__device__ __forceinline__ unsigned int tie_kept(unsigned long long above, unsigned long long m, unsigned int n,
                                                 unsigned long long thr) {
  if (m == 0) return n;
  const unsigned long long k = (thr - above + m - 1) / m;
  return k < n ? (unsigned int)k : n;
}

// Result of the CDF cut of one row: every block with a key above `key` is kept, and of the
// n_tie blocks whose key equals `key` the n_keep with the lowest indices.
struct Cut {
  unsigned long long key;
  unsigned int n_keep, n_tie;
};

constexpr int kDigitBits = 8;  // one bucket per thread: cheap clears and scans per pass
constexpr int kBuckets = 1 << kDigitBits;

constexpr int kDirect = 64;  // a selected bucket with at most this many keys is resolved directly

template <int NT>
struct RadixScratch {
  unsigned long long mass[kBuckets];
  unsigned int cnt[kBuckets];
  unsigned long long part[NT / 64];  // per-wave bucket-mass totals
  unsigned long long cand_cum[NT];
  unsigned long long cand[kDirect];  // keys of a small selected bucket
  int ncand;
  int bsel;
  unsigned long long found;
  unsigned int n_keep, n_tie;
};

// The CDF cut of one row: the smallest key K that has a kept block (the mass of the keys
// above K is < thr_fx) and how many of the blocks tied at K are kept. MSB-first radix select
// below the row's common key prefix: each pass histograms (count, exact fixed-point mass) the
// next 8-bit digit of the keys that match the prefix fixed so far and descends into the lowest
// bucket whose top key is still kept. Stops when that bucket holds one key or one key value
// (a tie class: every bit fixed), or (rows of at most 1024 blocks) resolves a bucket of at most
// kDirect keys by comparing them directly: rows of near-equal probabilities otherwise took
// up to 7 passes. Every thread returns the same result.
template <int NT, int NPT>
__device__ Cut radix_cut(const unsigned long long* key, int t, int nb, unsigned long long thr_fx,
                         RadixScratch<NT>& rs) {
  constexpr int kWaves = NT / 64;
  constexpr int kBucketsPerThread = kBuckets / NT;
  const int lane = t & 63, wv = t >> 6;
  // All keys of the row share the bits above the highest bit in which the largest and
  // the smallest key differ (sign and high exponent bits, typically): start the digits
  // there, so the first pass already spreads the keys over many buckets.
  unsigned long long kmax = 0, kmin = ~0ull;
#pragma unroll
  for (int k = 0; k < NPT; ++k)
    if (t + NT * k < nb) {
      kmax = key[k] > kmax ? key[k] : kmax;
      kmin = key[k] < kmin ? key[k] : kmin;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long a = __shfl_xor(kmax, o), b = __shfl_xor(kmin, o);
    kmax = a > kmax ? a : kmax;
    kmin = b < kmin ? b : kmin;
  }
  if (lane == 0) {
    rs.part[wv] = kmax;
    rs.cand_cum[wv] = kmin;
  }
  __syncthreads();
  kmax = rs.part[0];
  kmin = rs.cand_cum[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    kmax = rs.part[w] > kmax ? rs.part[w] : kmax;
    kmin = rs.cand_cum[w] < kmin ? rs.cand_cum[w] : kmin;
  }
  __syncthreads();
  if (kmax == kmin) return Cut{kmax, tie_kept(0, mass_fx(kmax), (unsigned)nb, thr_fx), (unsigned)nb};
  int shift = 64 - __clzll((long long)(kmax ^ kmin));  // bits below the common prefix
  unsigned long long pmask = shift == 64 ? 0ull : ~((1ull << shift) - 1);
  unsigned long long pval = kmax & pmask, above = 0;
  while (true) {
    const int db = shift >= kDigitBits ? kDigitBits : shift;
    shift -= db;
    const unsigned long long dmask = (1ull << db) - 1;
    for (int b = t; b < kBuckets; b += NT) {
      rs.mass[b] = 0;
      rs.cnt[b] = 0;
    }
    if (t == 0) rs.bsel = kBuckets;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      if (t + NT * k < nb && (key[k] & pmask) == pval) {
        const int d = (int)((key[k] >> shift) & dmask);
        atomicAdd(&rs.mass[d], mass_fx(key[k]));
        atomicAdd(&rs.cnt[d], 1u);
      }
    }
    __syncthreads();
    // Thread t owns buckets [t*BPT, t*BPT + BPT). Mass of all buckets above its range.
    const int b0 = t * kBucketsPerThread;
    unsigned long long local = 0;
#pragma unroll
    for (int q = 0; q < kBucketsPerThread; ++q) local += rs.mass[b0 + q];
    unsigned long long incl = local;  // inclusive suffix sum over the lanes of this wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long v = __shfl_down(incl, o);
      if (lane + o < 64) incl += v;
    }
    if (lane == 0) rs.part[wv] = incl;
    __syncthreads();
    unsigned long long run = above + (incl - local);
    for (int w = wv + 1; w < kWaves; ++w) run += rs.part[w];
    // Walk down my range: the lowest non-empty bucket whose top key is kept.
    int cand = kBuckets;
    unsigned long long cand_cum = 0;
#pragma unroll
    for (int q = kBucketsPerThread - 1; q >= 0; --q) {
      const int b = b0 + q;
      if (rs.cnt[b] > 0 && run < thr_fx) {
        cand = b;
        cand_cum = run;
      }
      run += rs.mass[b];
    }
    rs.cand_cum[t] = cand_cum;
    if (cand < kBuckets) atomicMin(&rs.bsel, cand);
    __syncthreads();
    const int bs = rs.bsel;
    above = rs.cand_cum[bs / kBucketsPerThread];
    const unsigned int n_in = rs.cnt[bs];
    pmask |= dmask << shift;
    pval |= (unsigned long long)bs << shift;
    if (t == 0) rs.ncand = 0;
    __syncthreads();  // the next pass clears the histogram
    // Every bit fixed: the bucket is one key value held by n_in tied blocks.
    if (shift == 0) return Cut{pval, tie_kept(above, mass_fx(pval), n_in, thr_fx), n_in};
    if (n_in == 1) break;
    if constexpr (NT * NPT <= 1024) {  // (the larger rows keep their occupancy: no extra registers)
      if (n_in <= kDirect) {
        // Few keys left in the bucket: K is the smallest among them whose mass above (the
        // bucket's `above` plus the larger keys of the bucket) is < thr_fx; the bucket's
        // largest key always qualifies. Then the blocks tied at K. Same answer as further passes.
#pragma unroll
        for (int k = 0; k < NPT; ++k)
          if (t + NT * k < nb && (key[k] & pmask) == pval) rs.cand[atomicAdd(&rs.ncand, 1)] = key[k];
        if (t == 0) rs.found = ~0ull;
        __syncthreads();
        if (t < (int)n_in) {
          const unsigned long long kk = rs.cand[t];
          unsigned long long m = above;
          for (int u = 0; u < (int)n_in; ++u)
            if (rs.cand[u] > kk) m += mass_fx(rs.cand[u]);
          if (m < thr_fx) atomicMin(&rs.found, kk);
        }
        __syncthreads();
        if (t == 0) {
          const unsigned long long kk = rs.found;
          unsigned long long m = above;
          unsigned int n = 0;
          for (int u = 0; u < (int)n_in; ++u) {
            if (rs.cand[u] > kk) m += mass_fx(rs.cand[u]);
            n += rs.cand[u] == kk;
          }
          rs.n_tie = n;
          rs.n_keep = tie_kept(m, mass_fx(kk), n, thr_fx);
        }
        __syncthreads();
        return Cut{rs.found, rs.n_keep, rs.n_tie};
      }
    }
  }
  // The single key in the selected bucket.
#pragma unroll
  for (int k = 0; k < NPT; ++k)
    if (t + NT * k < nb && (key[k] & pmask) == pval) rs.found = key[k];
  __syncthreads();
  return Cut{rs.found, 1u, 1u};
}

// Exclusive prefix of the popcounts of W bit words (W <= 128) in pre[]: wave 0, two words per
// lane. Returns the total (in wave 0). No barrier.
__device__ __forceinline__ int words_prefix(const uint32_t* bits, int* pre, int W, int t) {
  const int lane = t & 63;
  int total = 0;
  if (t < 64) {
    const int w0 = 2 * lane;
    const int c0 = w0 < W ? __popc(bits[w0]) : 0;
    const int c1 = w0 + 1 < W ? __popc(bits[w0 + 1]) : 0;
    int incl = c0 + c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    const int excl = incl - c0 - c1;
    if (w0 < W) pre[w0] = excl;
    if (w0 + 1 < W) pre[w0 + 1] = excl + c0;
    total = __shfl(incl, 63);
  }
  return total;
}

// Rank of block j among the set blocks, in index order, from the words and their prefix.
__device__ __forceinline__ int bit_rank(const uint32_t* bits, const int* pre, int j) {
  return pre[j >> 5] + __popc(bits[j >> 5] & ((1u << (j & 31)) - 1u));
}

template <int NT, int NPT, bool BITONIC>
__global__ __launch_bounds__(NT) void k_select(const double* __restrict__ S, uint32_t* __restrict__ words,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ lists,
                                                        KGeom g, SelArgs a) {
  constexpr int kWaves = NT / 64;
  constexpr int CAP = NT * NPT;
  constexpr int KEYS_WORDS = (sizeof(RadixScratch<NT>) + 7) / 8 > CAP ? (sizeof(RadixScratch<NT>) + 7) / 8 : CAP;
  __shared__ unsigned long long keys[KEYS_WORDS];  // bitonic keys, or the radix-select scratch
  __shared__ uint16_t idx[BITONIC ? CAP : 1];      // bitonic: the block index of each key
  __shared__ uint32_t wbits[CAP / 32];
  __shared__ int wpre[CAP / 32];
  __shared__ double redf[kWaves];
  __shared__ unsigned long long redu[kWaves];
  __shared__ unsigned long long kstar_s;
  __shared__ int jstar_s;

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const long long row = a.row0 + blockIdx.x;
  const int nb = g.nb;
  const int i = (int)(row % nb);
  const double* Srow = S + row * nb;
  const int W = a.W;

  const bool scored = a.mode != ABLA_MASK_STATIC;
  double s[NPT];
  double mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int j = t + NT * k;
    s[k] = (scored && j < nb) ? Srow[j] : -INFINITY;
    mx = fmax(mx, s[k]);
  }
  mx = wave_max(mx);
  if (lane == 0) redf[wv] = mx;
  __syncthreads();
  mx = redf[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) mx = fmax(mx, redf[w]);
  __syncthreads();

  bool keep[NPT];
  if (a.mode == ABLA_MASK_STATIC) {
    // DynamicRad Static-Ratio: per frame position p, its rank around block i's position
    // (squared block distance, then index), and k(dt) per frame distance; keep j iff its
    // position's rank is below k(|t_j - t_i|). Both tables live in the key scratch
    // (F + T <= 2 nb ints).
    const int F = g.nbh * g.nbw;
    int* rank_s = reinterpret_cast<int*>(keys);
    int* kc_s = rank_s + F;
    const int ti = i / F, pi = i - ti * F;
    const int hi = pi / g.nbw, wi = pi - hi * g.nbw;
    for (int p = t; p < F; p += NT) {
      const int hp = p / g.nbw, wp = p - hp * g.nbw;
      const int d2p = (hp - hi) * (hp - hi) + (wp - wi) * (wp - wi);
      int r = 0;
      for (int q = 0; q < F; ++q) {
        const int hq = q / g.nbw, wq = q - hq * g.nbw;
        const int d2q = (hq - hi) * (hq - hi) + (wq - wi) * (wq - wi);
        r += (d2q < d2p) || (d2q == d2p && q < p);
      }
      rank_s[p] = r;
    }
    for (int dt = t; dt < g.T; dt += NT) {
      double ratio = 1.0;
      for (int k = 0; k < dt; ++k) ratio = ratio * a.gamma;  // the float64 products of the definition
      kc_s[dt] = min(F, max(a.floor_k, (int)ceil((double)F * ratio)));
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int j = t + NT * k;
      if (j < nb) {
        const int tj = j / F;
        keep[k] = rank_s[j - tj * F] < kc_s[abs(tj - ti)];
      } else {
        keep[k] = false;
      }
    }
  } else if (a.mode == ABLA_MASK_DYN) {
    const double edge = mx - a.tau;
#pragma unroll
    for (int k = 0; k < NPT; ++k) keep[k] = (t + NT * k < nb) && s[k] >= edge;
  } else if (a.cdf_all || a.cdf_none) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) keep[k] = a.cdf_all && (t + NT * k < nb);
  } else {
    // Softmax of the row (max-shifted exponentials, fixed-order sum).
    double e[NPT];
    double z = 0.0;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      e[k] = (t + NT * k < nb) ? exp(s[k] - mx) : 0.0;
      z += e[k];
    }
    z = wave_sum(z);
    if (lane == 0) redf[wv] = z;
    __syncthreads();
    z = redf[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) z += redf[w];

    unsigned long long key[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int j = t + NT * k;
      key[k] = j < nb ? make_key(e[k] / z) : 0ull;
    }
    if constexpr (!BITONIC) {
      const Cut c = radix_cut<NT, NPT>(key, t, nb, a.thr_fx, *reinterpret_cast<RadixScratch<NT>*>(keys));
      if (c.n_keep >= c.n_tie) {
#pragma unroll
        for (int k = 0; k < NPT; ++k) keep[k] = (t + NT * k < nb) && key[k] >= c.key;
      } else {
        // Only some of the blocks tied at the cut's key are kept: the lowest indices. Rank the
        // tied blocks by index with a ballot per 64 consecutive blocks and a prefix of the
        // words' popcounts (the same layout as the packed mask below).
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
          const unsigned long long b = __ballot((t + NT * k < nb) && key[k] == c.key);
          if (lane == 0) {
            const int w0 = (NT * k + 64 * wv) >> 5;
            wbits[w0] = (uint32_t)b;
            wbits[w0 + 1] = (uint32_t)(b >> 32);
          }
        }
        __syncthreads();
        words_prefix(wbits, wpre, W, t);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
          const int j = t + NT * k;
          keep[k] = j < nb && (key[k] > c.key || (key[k] == c.key && bit_rank(wbits, wpre, j) < (int)c.n_keep));
        }
        __syncthreads();  // the packing below reuses the words
      }
    } else {
      // Bitonic sort of (key, index) pairs in ranking order: key descending, index ascending.
      // Padding entries (key 0, index 0xffff) rank after every block.
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int j = t + NT * k;
        if (j < a.np) {
          keys[j] = key[k];
          idx[j] = (uint16_t)(j < nb ? j : 0xffff);
        }
      }
      if (t == 0) {
        kstar_s = ~0ull;
        jstar_s = -1;
      }
      __syncthreads();
      const int np = a.np;
      for (int size = 2; size <= np; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int pidx = t; pidx < (np >> 1); pidx += NT) {
            const int lo = ((pidx & ~(stride - 1)) << 1) | (pidx & (stride - 1));
            const int hi = lo + stride;
            const unsigned long long x = keys[lo], y = keys[hi];
            const int xi = idx[lo], yi = idx[hi];
            const bool y_first = y > x || (y == x && yi < xi);  // y ranks before x
            const bool ranked = (lo & size) == 0;               // this run in ranking order
            if (ranked ? y_first : !y_first) {
              keys[lo] = y;
              keys[hi] = x;
              idx[lo] = (uint16_t)yi;
              idx[hi] = (uint16_t)xi;
            }
          }
          __syncthreads();
        }
      }

      // Exclusive prefix sum of the sorted masses; thread t owns a contiguous segment.
      const int seg = (np + NT - 1) / NT;
      const int p0 = t * seg;
      unsigned long long local = 0;
      for (int q = 0; q < seg; ++q)
        if (p0 + q < nb) local += mass_fx(keys[p0 + q]);
      // Inclusive wave scan, then across waves.
      unsigned long long incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      if (lane == 63) redu[wv] = incl;
      __syncthreads();
      unsigned long long before = incl - local;
      for (int w = 0; w < wv; ++w) before += redu[w];
      // Walk the segment: rank r is kept iff the mass before it is < thr; record the last kept.
      unsigned long long c = before;
      for (int q = 0; q < seg; ++q) {
        const int pos = p0 + q;
        if (pos >= nb) break;
        const bool kp = c < a.thr_fx;
        const unsigned long long mq = mass_fx(keys[pos]);
        const bool next_kept = (pos + 1 < nb) && (c + mq < a.thr_fx);
        if (kp && !next_kept) {
          kstar_s = keys[pos];
          jstar_s = idx[pos];
        }
        c += mq;
      }
      __syncthreads();
      const unsigned long long kstar = kstar_s;
      const int jstar = jstar_s;
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int j = t + NT * k;
        keep[k] = j < nb && (key[k] > kstar || (key[k] == kstar && j <= jstar));
      }
    }
  }

  // Sliding-tile window around block i.
  if (a.sta_on) {
    const int per_frame = g.nbh * g.nbw;
    const int ti = i / per_frame, hi = (i % per_frame) / g.nbw, wi = i % g.nbw;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int j = t + NT * k;
      const int tj = j / per_frame, hj = (j % per_frame) / g.nbw, wj = j % g.nbw;
      keep[k] = keep[k] || (j < nb && abs(tj - ti) <= a.rt && abs(hj - hi) <= a.rh && abs(wj - wi) <= a.rw);
    }
  }

  // Pack: a wave's ballot covers 64 consecutive blocks = two words.
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const unsigned long long b = __ballot(keep[k]);
    if (lane == 0) {
      const int w0 = (NT * k + 64 * wv) >> 5;
      wbits[w0] = (uint32_t)b;
      wbits[w0 + 1] = (uint32_t)(b >> 32);
    }
  }
  __syncthreads();
  const int total = words_prefix(wbits, wpre, W, t);
  if (t == 0) counts[row] = total;
  for (int w = t; w < W; w += NT) words[row * W + w] = wbits[w];
  __syncthreads();
  if (lists) {
    // Each kept block j goes to its rank among the kept blocks: the kept count before its
    // word plus the kept bits below it in the word (consecutive threads, consecutive slots).
    int32_t* lrow = lists + row * nb;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int j = t + NT * k;
      if (keep[k]) lrow[bit_rank(wbits, wpre, j)] = j;
    }
  }
}

template <int NT, int NPT>
void launch_select(const KGeom& g, const double* S, uint32_t* words, int32_t* counts, int32_t* lists,
                   const SelArgs& args, hipStream_t s) {
  // One workgroup per row, in launches of at most 2^22 rows (a grid dimension holds at most
  // 2^32 work-items).
  const long long rows = (long long)g.B * g.H * g.nb;
  constexpr long long kChunk = 1ll << 22;
  for (long long r0 = 0; r0 < rows; r0 += kChunk) {
    SelArgs a = args;
    a.row0 = r0;
    const dim3 grid((unsigned)(rows - r0 < kChunk ? rows - r0 : kChunk));
    if constexpr (NT == kSelThreads) {  // the bitonic sort needs np <= NT * NPT keys of LDS
      if (a.mode == ABLA_MASK_CDF && a.cut == ABLA_CUT_BITONIC) {
        k_select<NT, NPT, true><<<grid, NT, 0, s>>>(S, words, counts, lists, g, a);
        continue;
      }
    }
    k_select<NT, NPT, false><<<grid, NT, 0, s>>>(S, words, counts, lists, g, a);
  }
}

}  // namespace

hipError_t launch_build_mask(const KGeom& g, const abla_mask_params& p, const double* qbar, const double* kbar,
                             uint32_t* words, int32_t* counts, int32_t* lists, double* scores, hipStream_t s) {
  if (p.mode != ABLA_MASK_STATIC) {
    const double scale = p.pool_scale > 0.0 ? p.pool_scale : 1.0 / sqrt((double)g.d);
    // 128 x 128 tiles when they fill the GPU several times over, else 32 x 32 (one wave each).
    // The tile count B*H*tpr^2 fits an int: B*H*nb < 2^31 and nb <= 4096 are checked on
    // entry, ceil(nb / 128)^2 <= nb for such nb, and the 32-tile form runs only below 32768
    // tiles. Launches of at most 2^22 workgroups keep each grid inside the 2^32 work-items of
    // a dimension.
    const int t128 = (g.nb + 127) / 128;
    const bool big = (long long)t128 * t128 * g.B * g.H >= 2048;
    const int tpr = big ? t128 : (g.nb + 31) / 32;
    const int total = (int)((long long)tpr * tpr * g.B * g.H);
    constexpr int kChunk = 1 << 22;
    for (int base = 0; base < total; base += kChunk) {
      const int n = min(kChunk, total - base);
      if (big && g.d == 128)
        k_scores<128, 128><<<n, 256, 0, s>>>(qbar, kbar, scores, g.nb, scale, tpr, base);
      else if (big)
        k_scores<128, 64><<<n, 256, 0, s>>>(qbar, kbar, scores, g.nb, scale, tpr, base);
      else if (g.d == 128)
        k_scores<32, 128><<<n, 64, 0, s>>>(qbar, kbar, scores, g.nb, scale, tpr, base);
      else
        k_scores<32, 64><<<n, 64, 0, s>>>(qbar, kbar, scores, g.nb, scale, tpr, base);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  SelArgs a{};
  a.mode = p.mode;
  a.cut = p.cut;
  a.cdf_all = p.thr >= 1.0;
  a.cdf_none = p.thr <= 0.0;
  if (!a.cdf_all && !a.cdf_none) {
    unsigned long long fx = (unsigned long long)(p.thr * 4611686018427387904.0);
    a.thr_fx = fx ? fx : 1ull;
  }
  a.tau = p.tau;
  a.sta_on = (p.sta_t | p.sta_h | p.sta_w) != 0;
  a.rt = (p.sta_t - 1) / 2;
  a.rh = (p.sta_h - 1) / 2;
  a.rw = (p.sta_w - 1) / 2;
  int np = 2;
  while (np < g.nb) np <<= 1;
  a.np = np;
  a.W = (g.nb + 31) / 32;
  a.gamma = p.gamma;
  a.floor_k = (int)ceil((double)(g.nbh * g.nbw) * p.lambda);
  // Rows of up to 640 blocks (radix cut or no sort): one wave per row, so the row's steps
  // synchronise within the wave and more rows are in flight per CU; up to 1280 blocks two
  // waves. At most 10-12 keys per thread keeps the registers low enough for that occupancy
  // (the 16-key rows of up to 4096 blocks run at 3 waves per SIMD). The bitonic cross-check
  // sorts np >= nb keys in LDS and keeps the four-wave rows of np / 256 keys per thread; the
  // wide radix form takes those four-wave rows too.
  const bool bitonic = p.mode == ABLA_MASK_CDF && p.cut == ABLA_CUT_BITONIC;
  const bool narrow = !bitonic && p.cut != ABLA_CUT_RADIX_WIDE;
  if (narrow && g.nb <= 256)
    launch_select<64, 4>(g, scores, words, counts, lists, a, s);
  else if (narrow && g.nb <= 640)
    launch_select<64, 10>(g, scores, words, counts, lists, a, s);
  else if (narrow && g.nb <= 1280)
    launch_select<128, 10>(g, scores, words, counts, lists, a, s);
  else if (narrow && g.nb > 2048 && g.nb <= 3072)
    launch_select<kSelThreads, 12>(g, scores, words, counts, lists, a, s);
  else if (np <= 256)
    launch_select<kSelThreads, 1>(g, scores, words, counts, lists, a, s);
  else if (np <= 512)
    launch_select<kSelThreads, 2>(g, scores, words, counts, lists, a, s);
  else if (np <= 1024)
    launch_select<kSelThreads, 4>(g, scores, words, counts, lists, a, s);
  else if (np <= 2048)
    launch_select<kSelThreads, 8>(g, scores, words, counts, lists, a, s);
  else
    launch_select<kSelThreads, 16>(g, scores, words, counts, lists, a, s);
  return hipGetLastError();
}

}  // namespace abla
