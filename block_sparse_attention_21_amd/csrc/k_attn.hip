// Block-sparse attention forward over the kept 64 x 64 blocks.
//
// NABLA, Method: "expansion" -- the block mask names which N x N attention
// blocks are computed; everything else is skipped. For query block i the
// kernel walks the ascending list of kept key blocks with an online softmax.
//
// bf16 path (k_attn_bf16): one workgroup of four waves per pair of query blocks
// (i, i + nbh*nbw), i.e. the same patch in two consecutive frames, whose kept lists
// overlap heavily; waves 0-1 hold block i, waves 2-3 block i + nbh*nbw, 32 query rows
// per wave. The pair walks the union of its two lists once (a schedule built in LDS
// at start), so a key/value tile is fetched once for both blocks; each wave skips the
// tiles its own block does not keep. gfx950 MFMA v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T   A = K rows from LDS, B = Q rows held in registers. The
//                 result puts one query per lane (lanes l and l^32 share it),
//                 so the row max / sum stay in-lane plus one permlane swap.
//   O^T += V^T P^T  A = V^T rows from LDS (V is stored channel-major per
//                 block by the reorder pass), B = the probabilities exactly as
//                 the S^T registers hold them, rounded to bf16. The key order
//                 of the S^T result (keys 0-3,8-11 in lanes 0-31, 4-7,12-15 in
//                 lanes 32-63 of each 16-key step) is matched by loading K rows
//                 4-7 and 8-11 of every 16 swapped, so each V^T read is one chunk.
// Software pipeline: K tiles run one step ahead of V^T tiles (two LDS slots each),
// so while a wave turns the scores of tile u into probabilities it already runs
// the score MFMAs of tile u+1 (an explicit MFMA / LDS-read / VALU interleave). The
// probabilities use the running maximum of the earlier tiles; only when a lane's sum
// of them exceeds 256 is the tile's own maximum taken and the row rebased. One barrier
// per step. Tiles move global -> LDS directly (buffer_load ... lds), with a per-row
// XOR swizzle of 16-byte chunks so the MFMA operand reads are free of bank
// conflicts. The visiting order of the pairs (k_pair_order) depends on the list
// lengths: with short lists, runs of spatially adjacent temporal columns per XCD
// (neighbouring workgroups then share key blocks in L2); with long lists, longest-first
// per head so the long rows of the kept-count distribution do not form the tail.
//
// float32 path (k_attn_f32): float32 matrix cores, four waves per query block.
#include <math.h>

#include <mutex>

#include "common.h"
#include "mfma_tiles.h"

namespace abla {
namespace {

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;
  const int32_t* counts;
  const int32_t* lists;
  const int32_t* order;  // pair ids per (b, h) in visiting order (see k_pair_order)
  const int32_t* walk_mode;  // one int written by k_pair_order: 1 = column order
  uint16_t* out;
  float* lse;
  KGeom g;
  int pairs;    // query-block pairs per (b, h): ceil(T/2) * nbh * nbw
  int grid;     // work items (query-block pairs over all heads)
  int main_col, main_long;  // items 0 .. main-1 belong to workgroups 0 .. main-1, per walk mode (claim_item)
  int32_t* tail_cnt;  // items claimed by the tail workgroups (zeroed by k_pair_order)
  float c2;     // scale * log2(e)
  float scale;
  int orig;
  // Q and K in the original token order (else fractal order): exact division of block
  // indices (< 2^16) by F = nbh*nbw and by nbw as (j * magic) >> 32, magic = 2^32 / x + 1.
  int qk_orig;
  unsigned long long magic_f, magic_w;
};

// Byte offset of key block j's first token (its top-left corner) inside one head, and the
// offsets that walk a tile: a tile load of 256 threads covers 256 / (D/8) LDS rows, i.e. 2
// (d = 128) or 4 (d = 64) rows of the 8 x 8 patch, so consecutive loads of a thread are
// 512 * Ws bytes apart in the original order (4096 bytes, 16 or 32 whole rows, in fractal
// order).
template <int D, bool ORIG>
__device__ __forceinline__ uint32_t k_tile_base(int j, const AttnArgs& a) {
  if constexpr (!ORIG) {
    return (uint32_t)j * Tile<D>::KBYTES;
  } else {
    const KGeom& g = a.g;
    const uint32_t uj = (uint32_t)j;
    const uint32_t t = (uint32_t)(((unsigned long long)uj * a.magic_f) >> 32);
    const uint32_t rem = uj - t * (uint32_t)(g.nbh * g.nbw);
    const uint32_t hp = (uint32_t)(((unsigned long long)rem * a.magic_w) >> 32);
    const uint32_t wp = rem - hp * (uint32_t)g.nbw;
    return ((t * (uint32_t)g.Hs + hp * kP) * (uint32_t)g.Ws + wp * kP) * (uint32_t)(D * 2);
  }
}
template <bool ORIG>
__device__ __forceinline__ uint32_t k_tile_stride(const KGeom& g) {
  return ORIG ? 512u * (uint32_t)g.Ws : 4096u;
}

// Probabilities are formed against the running maximum of the tiles before (no per-tile
// maximum). A tile is accepted as long as each lane's sum of its 32 probabilities stays
// <= 256, which bounds every probability by 256 (fp32 and bf16 hold that without loss of
// relative precision, and 256 * 64 keys * #tiles stays far from overflow); otherwise (the
// first tile, or a maximum that grew by about 2^5 or more) the tile's maximum is taken, the
// running state rescaled and the probabilities formed again.
constexpr float kProbSumBound = 256.0f;

// Attention workgroups resident on one XCD at a time: 32 CUs (MI355X: 256 CUs in 8 XCDs),
// two 4-wave workgroups per CU.
constexpr int kXcdSlots = 64;
constexpr int kQueueTail = 2 * kXcdSlots;

// Column order (short lists): runs of G adjacent temporal columns of one head, G*C close to
// the workgroups one XCD holds at once.
__device__ __forceinline__ int column_run_width(int C) { return max(1, (kXcdSlots + C / 2) / C); }

// LDS map of the bf16 kernel: two K slots, two V^T slots, then the pair's schedule.
template <int D>
struct Lds {
  static constexpr int K0 = 0;
  static constexpr int V0 = 2 * Tile<D>::KBYTES;
  static constexpr int SCHED = V0 + 2 * Tile<D>::VBYTES;  // uint16 entries, kMaxBlocks of them
  static constexpr int BYTES = SCHED + kMaxBlocks * 2;
  __device__ static constexpr int kslot(int s) { return K0 + s * Tile<D>::KBYTES; }
  __device__ static constexpr int vslot(int s) { return V0 + s * Tile<D>::VBYTES; }
};

// Schedule entry: key block j in bits 0-11, bit 12 = block A keeps it, bit 13 = block B keeps it.
constexpr int kSchedJ = 0xfff;
constexpr int kSchedA = 1 << 12;
constexpr int kSchedB = 1 << 13;

// Query blocks of pair p (F = nbh*nbw blocks per frame, nb = T*F): pair tp*F + s covers patch
// s in frames 2*tp and 2*tp + 1. With T odd the last frame has no temporal partner: there
// pair (T-1)/2 * F + s joins the horizontally adjacent patches s and s+1 for even s (s + 1 < F;
// for s = F-1 with F odd, block a alone), and the odd s are empty items (a = -1), so those
// blocks do not run with half of their workgroup idle.
__device__ __forceinline__ void pair_blocks(int p, int F, int nb, int& a, int& b) {
  a = (p / F) * 2 * F + p % F;
  if (a + F < nb) {
    b = a + F;
  } else if ((p % F) & 1) {
    a = b = -1;
  } else {
    b = p % F + 1 < F ? a + 1 : -1;
  }
}

// Merge the two ascending kept lists of the pair into one ascending schedule in LDS
// (the union of the two sets, each entry flagged with the blocks that keep it), through
// two bitmaps and a prefix count of their OR. Returns the schedule length. Uses the
// K/V staging area as scratch; ends with a barrier.
__device__ int build_schedule(char* smem_stage, uint16_t* sched, const int32_t* la, int ca, const int32_t* lb, int cb,
                              int nb) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int nw = (nb + 31) >> 5;  // <= 128 words
  uint32_t* bma = reinterpret_cast<uint32_t*>(smem_stage);
  uint32_t* bmb = bma + 128;
  int* part = reinterpret_cast<int*>(bmb + 128);  // 4 wave totals + the length
  if (t < 128) {
    bma[t] = 0;
    bmb[t] = 0;
  }
  __syncthreads();
  for (int p = t; p < ca; p += 256) {
    const int j = min(max(la[p], 0), nb - 1);
    atomicOr(&bma[j >> 5], 1u << (j & 31));
  }
  for (int p = t; p < cb; p += 256) {
    const int j = min(max(lb[p], 0), nb - 1);
    atomicOr(&bmb[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  const uint32_t wa = t < nw ? bma[t] : 0u, wb = t < nw ? bmb[t] : 0u;
  const uint32_t wu = wa | wb;
  const int c = __builtin_popcount(wu);
  int incl = c;  // inclusive prefix count over the lanes of this wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(incl, o);
    if (lane >= o) incl += x;
  }
  if (lane == 63) part[wv] = incl;
  __syncthreads();
  int base = incl - c;
  for (int v = 0; v < wv; ++v) base += part[v];
  if (t == 0) part[4] = part[0] + part[1] + part[2] + part[3];
  uint32_t bits = wu;
  while (bits) {
    const int b = __builtin_ctz(bits);
    bits &= bits - 1;
    const int j = t * 32 + b;
    sched[base++] = (uint16_t)(j | (((wa >> b) & 1u) ? kSchedA : 0) | (((wb >> b) & 1u) ? kSchedB : 0));
  }
  __syncthreads();
  const int n = part[4];
  __syncthreads();  // the staging area is reused by the first tile loads
  return n;
}

// The next tiles' loads of one step: K(u+2) into K slot `kdst`, V^T(u+1) into V slot
// `vdst`. load(i) issues this thread's i-th 16-byte load (K first, then V^T), so a caller
// can spread the step's loads between its MFMAs instead of issuing them as one burst
// (a burst of 1 KB loads from every wave stalls the issuing waves in the address unit).
template <int D>
struct StepLoads {
  char* kdst;
  char* vdst;
  i32x4_t krs, vrs;
  uint32_t ktile, vtile, koff, voff, kstride, vstride;
  static constexpr int NK = Tile<D>::KBYTES / 16 / 256;
  static constexpr int NV = Tile<D>::VBYTES / 16 / 256;
  __device__ __forceinline__ void load(int i) const {
    if (i < NK)
      raw_buffer_load_lds(krs, (__attribute__((address_space(3))) uint32_t*)(kdst + i * 256 * 16), 16, (int)koff,
                          (int)(ktile + i * kstride), 0, 0);
    else
      raw_buffer_load_lds(vrs, (__attribute__((address_space(3))) uint32_t*)(vdst + (i - NK) * 256 * 16), 16,
                          (int)voff, (int)(vtile + (i - NK) * vstride), 0, 0);
  }
  __device__ __forceinline__ void load_all() const {
#pragma unroll
    for (int i = 0; i < NK + NV; ++i) load(i);
  }
};

// S^T for one staged K tile: s[kh] holds keys kh*32 .. kh*32+31 (in the kperm row order)
// against this wave's 32 queries. klds[ks]: this lane's byte offset of its K chunk for
// k-step ks inside a slot; the two key halves are 32 rows apart. With a StepLoads, one
// of the step's loads goes out after each k-step (D/16 k-steps, D/16 loads).
template <int D, int SLOT, bool LOADS>
__device__ __forceinline__ void tile_scores(const char* smem, const uint32_t* klds, const bf16x8_t* qv,
                                            f32x16_t (&s)[2], const StepLoads<D>* ld) {
  static_assert(StepLoads<D>::NK + StepLoads<D>::NV == D / 16, "one load per k-step");
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kh][r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const bf16x8_t kv =
          *reinterpret_cast<const bf16x8_t*>(smem + Lds<D>::kslot(SLOT) + kh * 32 * D * 2 + klds[ks]);
      s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qv[ks], s[kh], 0, 0, 0);
    }
    if constexpr (LOADS) ld->load(ks);
  }
}

// Largest raw score of this lane's query over the tile (both lanes of the query agree).
__device__ __forceinline__ float tile_max(const f32x16_t (&s)[2]) {
  float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
  return swap_max(mx);
}

// Probabilities exp2(c2*s - m) rounded to bf16 in the V^T-operand order; returns their
// float32 sum over this lane's 32 keys (four partial sums, no long dependency chain).
// (Summing the bf16-rounded values instead, with bf16 pair dot products, saves 16 adds
// per tile but moves the log-sum-exp by up to 2^-8; it measured within the run-to-run
// spread, so the float32 sum stays.)
__device__ __forceinline__ float tile_probs(const f32x16_t (&s)[2], float c2, float m, bf16x8_t (&pb)[4]) {
  float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = exp2_fast(fmaf(s[kh][r], c2, -m));
      ps[r & 3] += pv;
      pb[kh * 2 + (r >> 3)][r & 7] = (__bf16)pv;
    }
  return (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

// O^T += V^T P^T for one staged V^T tile. vlds[kk]: this lane's byte offset of its 8-key
// chunk kk of channel row (lane & 31) inside a slot; channel tile dt is 32 rows further.
// With VT the slot holds a token-major V tile laid out like a K tile (key rows in kperm
// order, chunk-swizzled with kt_swz) and the V^T operand comes from two LDS transpose loads
// per channel tile: vlds[2*dt], vlds[2*dt + 1] are their LDS addresses for keys 0..15 of V
// slot 0, and keys 16*kk of slot SLOT sit a constant offset further. The transpose loads go
// through tr_chunks_at (the wait inside the asm block), so they do not make the compiler wait
// for the next tiles' loads, which fill the other slots.
template <int D, int SLOT, bool VT>
__device__ __forceinline__ void tile_values(const char* smem, const uint32_t* vlds, const bf16x8_t (&pb)[4],
                                            f32x16_t* o) {
  if constexpr (VT) {
    constexpr int DT = D / 32;
    constexpr int S = Lds<D>::vslot(SLOT) - Lds<D>::vslot(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t vv[DT];
      switch (kk) {  // the offset is an immediate of the transpose loads
        case 0: tr_chunks_at<DT, S>(vlds, vv); break;
        case 1: tr_chunks_at<DT, S + 16 * D * 2>(vlds, vv); break;
        case 2: tr_chunks_at<DT, S + 32 * D * 2>(vlds, vv); break;
        default: tr_chunks_at<DT, S + 48 * D * 2>(vlds, vv); break;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[dt], pb[kk], o[dt], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8_t vv =
            *reinterpret_cast<const bf16x8_t*>(smem + Lds<D>::vslot(SLOT) + dt * 32 * kBlock * 2 + vlds[kk]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[kk], o[dt], 0, 0, 0);
      }
  }
}

// Rebase on tile s: the running maximum becomes max(m_run, tile maximum), the running sum
// and output are rescaled to it and the probabilities formed again (all <= 1 now); returns
// their sum. Wave-uniform (called under a ballot).
template <int D>
__device__ __forceinline__ float rebase_tile(const f32x16_t (&s)[2], float c2, float& m_run, float& l_run, f32x16_t* o,
                                          bf16x8_t (&pb)[4]) {
  const float m_new = fmaxf(m_run, tile_max(s) * c2);
  const float alpha = exp2_fast(m_run - m_new);  // 0 on the first tile (m_run = -inf)
  m_run = m_new;
  l_run *= alpha;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
  return tile_probs(s, c2, m_run, pb);
}

// Instruction interleave of the steady state, in two scheduling regions. Phase A: the
// next tile's score MFMAs run under this tile's exp/convert/sum work and the step's tile
// loads. Phase B: the value MFMAs and their LDS reads. Masks: 0x008 MFMA, 0x100 LDS read,
// 0x402 VALU or transcendental, 0x010 vector memory.
template <int D>
__device__ __forceinline__ void schedule_phase_a() {
  constexpr int NS = 2 * (D / 16);
  constexpr int VA = 112 / NS;
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, VA, 0);
    if (i & 1) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  }
}
template <int D, bool VT>
__device__ __forceinline__ void schedule_phase_b() {
  constexpr int NPV = 4 * (D / 32);
  constexpr int RD = VT ? 0 : 1;  // LDS reads per value MFMA (the transpose loads are asm blocks)
  if constexpr (RD) __builtin_amdgcn_sched_group_barrier(0x100, 4 * RD, 0);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (RD) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
  }
}

// Items main .. grid-1 (the last positions of every XCD's queue: its shortest pairs,
// longest-first) are not tied to a workgroup; main depends on the walk mode (a longer dynamic
// tail for long lists, where the XCDs also differ in speed). Workgroups are dealt to the XCDs round-robin and
// each XCD runs its share in order, so an XCD whose share of the static items took less time
// reaches its tail workgroups earlier; each of those takes the next unclaimed item from one
// counter, and the XCDs that finish first take more of the tail. There are kTailOversub tail
// workgroups per tail item (an XCD can take up to a quarter of the tail; the surplus exit at
// once): 2 measured better than 4 (fewer empty workgroups) at 480p, 480p-dyn and on the long
// clip. `slot` is one int of LDS. Returns the item, or -1 when none is left.
constexpr int kTailOversub = 2;
__device__ __forceinline__ int claim_item(const AttnArgs& a, int* slot) {
  const int main = ld_const(a.walk_mode, 0) ? a.main_col : a.main_long;
  if ((int)blockIdx.x < main) return (int)blockIdx.x;
  if (threadIdx.x == 0) *slot = atomicAdd(a.tail_cnt, 1);  // a vector-memory atomic, one lane
  __syncthreads();
  const int it = main + *slot;
  __syncthreads();  // the slot is LDS the schedule reuses
  return it < a.grid ? it : -1;
}

struct Walk {
  int u, n;        // position in the schedule and its length
  int ec, en, ef;  // entries u, u+1, u+2 (0 past the end)
};

// One step of the schedule at position u, whose K/V^T slots have parity P:
//   K(u) in K slot P (already consumed), K(u+1) in K slot P^1, V(u) in V slot P.
// Issues K(u+2) into K slot P and V(u+1) into V slot P^1, then, for this wave's block,
// finishes tile u (probabilities, values) and starts tile u+1 (scores).
// sc holds S(u) if the block keeps u; sn receives S(u+1).
template <int D, int P, bool QKO, bool VT>
__device__ __forceinline__ void walk_step(const AttnArgs& a, char* smem, const uint16_t* sched, Walk& wk, int mine,
                                          int w,
                                          i32x4_t krs, i32x4_t vrs, uint32_t koff,
                                          uint32_t voff, const uint32_t* klds, const uint32_t* vlds,
                                          const bf16x8_t* qv, float c2, f32x16_t (&sc)[2], f32x16_t (&sn)[2],
                                          f32x16_t* o, float& m_run, float& l_run) {
  using TT = Tile<D>;
  wait_vm_lgkm_barrier();  // K(u+1), V(u) landed; every wave is done with step u-1
  // Past the end of the schedule the loads fetch block 0 into the free slot (never read):
  // that keeps the step free of branches around its loads.
  StepLoads<D> ld;
  ld.kdst = smem + Lds<D>::kslot(P) + w * 64 * 16;
  ld.vdst = smem + Lds<D>::vslot(P ^ 1) + w * 64 * 16;
  ld.krs = krs;
  ld.vrs = vrs;
  ld.ktile = k_tile_base<D, QKO>(wk.ef & kSchedJ, a);  // ef, en are 0 past the end
  ld.kstride = k_tile_stride<QKO>(a.g);
  ld.vtile = VT ? k_tile_base<D, true>(wk.en & kSchedJ, a) : (uint32_t)(wk.en & kSchedJ) * TT::VBYTES;
  ld.vstride = k_tile_stride<VT>(a.g);
  ld.koff = koff;
  ld.voff = voff;
  const int look = min(wk.u + 3, wk.n - 1);
  const int raw = sched[look];  // entry u+3, read now and used next step

  const bool mc = (wk.ec & mine) != 0;
  const bool mn = (wk.en & mine) != 0;  // en is 0 past the end
  if (mc && mn) {
    bf16x8_t pb[4];
    // Phase A (exp-heavy) runs at raised wave priority and phase B (MFMA-dense) at the
    // default: the two waves sharing a SIMD then tend to sit in opposite phases, which
    // measured 3-8% faster than equal priorities.
    __builtin_amdgcn_s_setprio(1);
    tile_scores<D, P ^ 1, true>(smem, klds, qv, sn, &ld);
    float psum = tile_probs(sc, c2, m_run, pb);
    schedule_phase_a<D>();
    __builtin_amdgcn_s_setprio(0);
    if (__builtin_amdgcn_ballot_w64(!(psum <= kProbSumBound))) psum = rebase_tile<D>(sc, c2, m_run, l_run, o, pb);
    tile_values<D, P, VT>(smem, vlds, pb, o);
    schedule_phase_b<D, VT>();
    __builtin_amdgcn_s_setprio(0);  // no-op for priority; closes phase B's scheduling region
    l_run += psum;
  } else if (mc) {
    ld.load_all();
    bf16x8_t pb[4];
    float psum = tile_probs(sc, c2, m_run, pb);
    if (__builtin_amdgcn_ballot_w64(!(psum <= kProbSumBound))) psum = rebase_tile<D>(sc, c2, m_run, l_run, o, pb);
    tile_values<D, P, VT>(smem, vlds, pb, o);
    l_run += psum;
  } else if (mn) {
    tile_scores<D, P ^ 1, true>(smem, klds, qv, sn, &ld);
  } else {
    ld.load_all();
  }
  wk.u += 1;
  wk.ec = wk.en;
  wk.en = wk.ef;
  wk.ef = wk.u + 2 < wk.n ? __builtin_amdgcn_readfirstlane(raw) : 0;
}

template <int D, bool QKO, bool VT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bf16(AttnArgs a) {
  using TT = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char smem[Lds<D>::BYTES];
  uint16_t* sched = reinterpret_cast<uint16_t*>(smem + Lds<D>::SCHED);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;          // waves 0,1: block A; waves 2,3: block B
  const int hi = lane >> 5;
  const KGeom& g = a.g;
  const int nb = g.nb;
  const int F = g.nbh * g.nbw;

  // Work item: item blockIdx.x, or for the tail workgroups the next unclaimed item (claim_item).
  const int item = claim_item(a, reinterpret_cast<int*>(sched));
  if (item < 0) return;  // every item is taken (uniform across the workgroup)
  // Visiting order: entry `item` of the table xcd_queue wrote (column order, short lists),
  // else position `item` of the per-head longest-first order (long lists), in plain dispatch
  // order: the resident workgroups of all eight XCDs then work on the same one or two heads
  // at a time, whose K/V (tens of MB) stay in the shared last-level cache.
  int bh, pair;
  if (ld_const(a.walk_mode, 0)) {
    const int gi = ld_const(a.order, (long long)item);
    bh = gi / a.pairs;
    pair = gi - bh * a.pairs;
  } else {
    bh = item / a.pairs;
    const int pos = item - bh * a.pairs;
    pair = ld_const(a.order, (long long)bh * a.pairs + pos);
  }
  int blk_a, blk_b;
  pair_blocks(pair, F, nb, blk_a, blk_b);
  if (blk_a < 0) return;  // an empty item (the odd patch of a last-frame pair)
  const int my_blk = (w < 2) ? blk_a : blk_b;
  const bool active = my_blk >= 0;

  const long long row_a = (long long)bh * nb + blk_a;
  const long long row_b = (long long)bh * nb + (blk_b >= 0 ? blk_b : blk_a);
  const int ca = min(max(ld_const(a.counts, row_a), 0), nb);
  const int cb = blk_b >= 0 ? min(max(ld_const(a.counts, row_b), 0), nb) : 0;

  const int q_local = (w & 1) * 32 + (lane & 31);

  // Q operand: lane holds Q[q_local][ks*16 + 8*hi .. +7] for every k-step.
  bf16x8_t qv[D / 16];
  if (active) {
    const long long qn = QKO ? token_of(g, my_blk, q_local) : (long long)my_blk * kBlock + q_local;
    const uint16_t* qrow = a.q + ((long long)bh * g.N + qn) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qv[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
  }

  Walk wk;
  wk.n = build_schedule(smem, sched, a.lists + row_a * nb, ca, a.lists + row_b * nb, cb, nb);

  // Per-thread global byte offsets of its 16-byte tile loads, and per-lane LDS byte
  // offsets of its MFMA operand chunks (both the same for every tile).
  uint32_t klds[D / 16], vlds[VT ? 2 * (D / 32) : 4];
  // K: LDS row r of a tile holds key kperm(r) of the block; in the original order that key
  // sits (kperm(r) / 8) rows of Ws tokens and kperm(r) % 8 tokens past the block's corner.
  const int kr = kperm(t / TT::KCH);
  const uint32_t krow = QKO ? (uint32_t)((kr >> 3) * g.Ws + (kr & 7)) : (uint32_t)kr;
  const uint32_t koff = krow * (uint32_t)(D * 2) + (uint32_t)(((t % TT::KCH) ^ k_swz<D>(t / TT::KCH)) * 16);
  const uint32_t kstride = k_tile_stride<QKO>(g);
  // V: channel-major V^T blocks, or with VT a token-major tile of the original-order V loaded
  // exactly like a K tile in the original order.
  const uint32_t voff = VT ? (uint32_t)((kr >> 3) * g.Ws + (kr & 7)) * (uint32_t)(D * 2) +
                                 (uint32_t)(((t % TT::KCH) ^ kt_swz<D>(t / TT::KCH)) * 16)
                           : (uint32_t)((t >> 3) * kBlock * 2 + (((t & 7) ^ v_swz(t >> 3)) * 16));
  {
    const int r0 = lane & 31;  // rows r0 and r0 + 32 share the swizzle
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) klds[ks] = (uint32_t)(r0 * D * 2 + (((ks * 2 + hi) ^ k_swz<D>(r0)) * 16));
    if constexpr (VT) {
      const uint32_t vbase = lds_offset(smem + Lds<D>::vslot(0));
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        tr_rel<D>(dt, 0, lane, vlds[2 * dt], vlds[2 * dt + 1]);
        vlds[2 * dt] += vbase;
        vlds[2 * dt + 1] += vbase;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) vlds[kk] = (uint32_t)(r0 * kBlock * 2 + (((2 * kk + hi) ^ v_swz(r0)) * 16));
    }
  }
  // One resource per head: K and V^T of head bh are each N*D*2 bytes, at most 64 MiB
  // (nb <= 4096 blocks of 64 tokens, d <= 128), so 32-bit offsets cover them.
  const uint32_t head_bytes = (uint32_t)(g.N * D * 2);
  const i32x4_t krs = make_rsrc(a.k + (long long)bh * g.N * D, head_bytes);
  const i32x4_t vrs = make_rsrc(a.vt + (long long)bh * nb * D * kBlock, head_bytes);  // = N*D per head
  const uint32_t vstride = k_tile_stride<VT>(g);
  const int mine = (w < 2) ? kSchedA : kSchedB;

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;  // in log2 units (scores * c2)
  float l_run = 0.f;

  wk.u = 0;
  wk.ec = wk.n > 0 ? __builtin_amdgcn_readfirstlane((int)sched[0]) : 0;
  wk.en = wk.n > 1 ? __builtin_amdgcn_readfirstlane((int)sched[1]) : 0;
  wk.ef = wk.n > 2 ? __builtin_amdgcn_readfirstlane((int)sched[2]) : 0;
  f32x16_t s0[2], s1[2];
  if (wk.n > 0) {
    issue_rows<TT::KBYTES>(smem + Lds<D>::kslot(0), w, krs, k_tile_base<D, QKO>(wk.ec & kSchedJ, a), koff,
                           kstride);
    issue_rows<TT::VBYTES>(smem + Lds<D>::vslot(0), w, vrs,
                           VT ? k_tile_base<D, true>(wk.ec & kSchedJ, a) : (uint32_t)(wk.ec & kSchedJ) * TT::VBYTES,
                           voff, vstride);
    if (wk.n > 1)
      issue_rows<TT::KBYTES>(smem + Lds<D>::kslot(1), w, krs, k_tile_base<D, QKO>(wk.en & kSchedJ, a), koff,
                             kstride);
    wait_vm_lgkm_barrier();
    if (wk.ec & mine) {
      tile_scores<D, 0, false>(smem, klds, qv, s0, nullptr);
      m_run = tile_max(s0) * a.c2;  // the first tile's maximum, so its probabilities need no rebase
    }
    while (true) {
      walk_step<D, 0, QKO, VT>(a, smem, sched, wk, mine, w, krs, vrs, koff, voff, klds, vlds, qv, a.c2, s0, s1, o,
                           m_run, l_run);
      if (wk.u >= wk.n) break;
      walk_step<D, 1, QKO, VT>(a, smem, sched, wk, mine, w, krs, vrs, koff, voff, klds, vlds, qv, a.c2, s1, s0, o,
                           m_run, l_run);
      if (wk.u >= wk.n) break;
    }
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

// float32 path on the float32 matrix cores (v_mfma_f32_32x32x2_f32). One workgroup of four waves
// per query block; wave (qh, kh) = (w & 1, w >> 1) takes queries qh*32 .. +31 against keys
// kh*32 .. +31 of every kept tile, with its own online softmax; the two key halves are merged
// through LDS at the end. Operand layout of one 32x32x2 product: lane l supplies A[l % 32][l / 32]
// and B[l / 32][l % 32]; accumulator register r of lane l is D[8(r/4) + 4(l/32) + r%4][l % 32].
//   S^T = K Q^T: lane l supplies channel (l/32)*d/2 + s of its key and of its query at step s
//     (the two lane halves reduce over the two channel halves; d/2 products in all).
//   O^T += V^T P^T: A = V^T with channel row i of tile ct = channel (d/32)*i + ct, so that a lane
//     reads the d/32 channels of all tiles as one vector; B = P^T at step r is register r of the
//     probabilities (keys 8(r/4) + r%4 in lanes 0-31, that + 4 in lanes 32-63), no data movement.
// K and V tiles are staged token-major in LDS (16-byte chunk c of row r at c ^ (r & 7)), double
// buffered through registers: the next tile's global loads are issued before this tile's products
// and stored to the other slot after them, one barrier per tile. The softmax works in log2 units
// (exp2 of scale * log2(e) * s minus the running maximum) and rescales whenever the maximum grows.
struct AttnArgsF32 {
  const float* q;
  const float* k;
  const float* v;  // token-major in the original order (v_orig), else channel-major blocks [nb, d, 64]
  const int32_t* counts;
  const int32_t* lists;
  const int32_t* order;
  float* out;
  float* lse;
  KGeom g;
  float c2;  // scale * log2(e)
  int orig;
};

template <int D>
struct F32Tile {
  static constexpr int CH = D / 4;          // 16-byte chunks per token row
  static constexpr int BYTES = 64 * D * 4;  // one K or V tile
  static constexpr int NLD = 64 * CH / 256; // 16-byte loads per thread per tile (each of K, V)
  static constexpr int CPL = D / 32;        // output channel tiles; channels per lane read of V
};

__device__ __forceinline__ uint32_t f32_swz(int row, int chunk, int D) {
  return (uint32_t)(row * D * 4 + ((chunk ^ (row & 7)) << 4));
}

// Token offset of tile row r from its block's first token: r in fractal order, or (r / 8) rows
// of Ws tokens and r % 8 tokens past the block's corner in the original order.
__device__ __forceinline__ long long f32_row_off(const KGeom& g, int r, bool orig) {
  return orig ? (long long)(r >> 3) * g.Ws + (r & 7) : (long long)r;
}
__device__ __forceinline__ long long f32_block_base(const KGeom& g, int j, bool orig) {
  if (!orig) return (long long)j * kBlock;
  const int F = g.nbh * g.nbw;
  const int tj = j / F, rem = j - tj * F, hp = rem / g.nbw, wp = rem - hp * g.nbw;
  return ((long long)tj * g.Hs + hp * kP) * g.Ws + wp * kP;
}

// This thread's 16-byte chunks of K tile j and V tile j into registers (K first).
template <int D, bool QKO, bool VORIG>
__device__ __forceinline__ void f32_load_tile(const KGeom& g, const float* kbase, const float* vbase, int j, int t,
                                              float4 (&stg)[2 * F32Tile<D>::NLD]) {
  constexpr int CH = F32Tile<D>::CH, NLD = F32Tile<D>::NLD;
  const long long kb = f32_block_base(g, j, QKO), vb = f32_block_base(g, j, true);
#pragma unroll
  for (int it = 0; it < NLD; ++it) {
    const int u = t + 256 * it;
    const int r = u / CH, c = u % CH;
    stg[it] = *reinterpret_cast<const float4*>(kbase + (kb + f32_row_off(g, r, QKO)) * D + 4 * c);
    if constexpr (VORIG)
      stg[NLD + it] = *reinterpret_cast<const float4*>(vbase + (vb + f32_row_off(g, r, true)) * D + 4 * c);
    else  // chunk u of the channel-major block: channel u / 16, keys 4*(u % 16) .. +3
      stg[NLD + it] = *reinterpret_cast<const float4*>(vbase + (long long)j * D * kBlock + 4 * u);
  }
}

// The staged chunks into LDS slot `slot`, both tiles token-major and swizzled.
template <int D, bool VORIG>
__device__ __forceinline__ void f32_store_tile(char* smem, int slot, int t, const float4 (&stg)[2 * F32Tile<D>::NLD]) {
  constexpr int CH = F32Tile<D>::CH, NLD = F32Tile<D>::NLD;
  char* kd = smem + slot * 2 * F32Tile<D>::BYTES;
  char* vd = kd + F32Tile<D>::BYTES;
#pragma unroll
  for (int it = 0; it < NLD; ++it) {
    const int u = t + 256 * it;
    const int r = u / CH, c = u % CH;
    *reinterpret_cast<float4*>(kd + f32_swz(r, c, D)) = stg[it];
    if constexpr (VORIG) {
      *reinterpret_cast<float4*>(vd + f32_swz(r, c, D)) = stg[NLD + it];
    } else {
      const int ch = u >> 4, k0 = (u & 15) * 4;
      *reinterpret_cast<float*>(vd + f32_swz(k0, ch >> 2, D) + (ch & 3) * 4) = stg[NLD + it].x;
      *reinterpret_cast<float*>(vd + f32_swz(k0 + 1, ch >> 2, D) + (ch & 3) * 4) = stg[NLD + it].y;
      *reinterpret_cast<float*>(vd + f32_swz(k0 + 2, ch >> 2, D) + (ch & 3) * 4) = stg[NLD + it].z;
      *reinterpret_cast<float*>(vd + f32_swz(k0 + 3, ch >> 2, D) + (ch & 3) * 4) = stg[NLD + it].w;
    }
  }
}

template <int D, bool QKO, bool VORIG>
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgsF32 a) {
  using TT = F32Tile<D>;
  constexpr int NLD = TT::NLD, CPL = TT::CPL;
  __shared__ __attribute__((aligned(16))) char smem[4 * TT::BYTES];  // K0, V0, K1, V1
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int qh = w & 1, kh = w >> 1, hf = lane >> 5, m = lane & 31;
  const KGeom& g = a.g;
  const int nb = g.nb;
  const int bh = blockIdx.x / nb;
  const int pos = blockIdx.x - bh * nb;
  const int i = a.order[(long long)bh * nb + pos];
  const long long row = (long long)bh * nb + i;
  const int cnt = min(max(a.counts[row], 0), nb);
  const int32_t* lst = a.lists + row * nb;

  // Q operand: Q[query qh*32 + m][hf*D/2 + s] for s = 0 .. D/2 - 1.
  float qv[D / 2];
  {
    const int qr = qh * 32 + m;
    const long long qn = QKO ? token_of(g, i, qr) : (long long)i * kBlock + qr;
    const float4* src = reinterpret_cast<const float4*>(a.q + ((long long)bh * g.N + qn) * D + hf * (D / 2));
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const float4 x = src[c];
      qv[4 * c] = x.x;
      qv[4 * c + 1] = x.y;
      qv[4 * c + 2] = x.z;
      qv[4 * c + 3] = x.w;
    }
  }
  const float* kbase = a.k + (long long)bh * g.N * D;
  const float* vbase = a.v + (long long)bh * g.N * D;  // both V layouts hold N*D floats per head
  float4 stg[2 * NLD];  // the next tile: NLD chunks of K, then NLD of V

  f32x16_t o[CPL];
#pragma unroll
  for (int ct = 0; ct < CPL; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[ct][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.c2;
  const int krow = kh * 32 + m;  // this lane's key row of a tile in S^T

  // List entries are read one step before their tile's loads are issued; past the end of the
  // list the loads fetch tile 0 into the slot that is not read again (no branches around them).
  auto entry = [&](int u) { return u < cnt ? min(max(lst[u], 0), nb - 1) : 0; };
  int j_next = entry(1);
  if (cnt > 0) {
    f32_load_tile<D, QKO, VORIG>(g, kbase, vbase, entry(0), t, stg);
    f32_store_tile<D, VORIG>(smem, 0, t, stg);
    __syncthreads();
  }
  for (int u = 0; u < cnt; ++u) {
    const int j_after = entry(u + 2);
    f32_load_tile<D, QKO, VORIG>(g, kbase, vbase, j_next, t, stg);
    j_next = j_after;
    const char* ks = smem + (u & 1) * 2 * TT::BYTES;
    const char* vs = ks + TT::BYTES;
    // S^T for keys kh*32 + (0..31) x queries qh*32 + (0..31): four accumulators (one per channel
    // step of a chunk) so that consecutive products are independent; added at the end.
    f32x16_t sa[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[e][r] = 0.f;
#pragma unroll
    for (int c4 = 0; c4 < D / 8; ++c4) {
      const float4 kk = *reinterpret_cast<const float4*>(ks + f32_swz(krow, hf * (D / 8) + c4, D));
      sa[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(kk.x, qv[4 * c4], sa[0], 0, 0, 0);
      sa[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(kk.y, qv[4 * c4 + 1], sa[1], 0, 0, 0);
      sa[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(kk.z, qv[4 * c4 + 2], sa[2], 0, 0, 0);
      sa[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(kk.w, qv[4 * c4 + 3], sa[3], 0, 0, 0);
    }
    f32x16_t s0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = (sa[0][r] + sa[1][r]) + (sa[2][r] + sa[3][r]);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s0[r]);
    const float m_new = fmaxf(m_run, swap_max(mx) * c2);
    const float alpha = exp2_fast(m_run - m_new);  // 0 on the first tile (m_run = -inf)
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = exp2_fast(fmaf(s0[r], c2, -m_new));
      ps += s0[r];
    }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
    // O^T += V^T P^T, 16 steps of two keys each.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kh * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
      if constexpr (CPL == 4) {
        const float4 vv = *reinterpret_cast<const float4*>(vs + f32_swz(key, m, D));
        o[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.x, s0[r], o[0], 0, 0, 0);
        o[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.y, s0[r], o[1], 0, 0, 0);
        o[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.z, s0[r], o[2], 0, 0, 0);
        o[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.w, s0[r], o[3], 0, 0, 0);
      } else {
        const float2 vv = *reinterpret_cast<const float2*>(vs + f32_swz(key, m >> 1, D) + (m & 1) * 8);
        o[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.x, s0[r], o[0], 0, 0, 0);
        o[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.y, s0[r], o[1], 0, 0, 0);
      }
    }
    f32_store_tile<D, VORIG>(smem, (u + 1) & 1, t, stg);
    __syncthreads();
  }

  // Merge the two key halves: wave (qh, 1) hands its running maximum, sum and output to (qh, 0).
  const float l_tot = swap_sum(l_run);
  float* xo = reinterpret_cast<float*>(smem) + qh * (CPL * 16 * 64 + 128);  // [CPL][16][64], m, l
  if (cnt > 0 && kh == 1) {
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(ct * 16 + r) * 64 + lane] = o[ct][r];
    xo[CPL * 16 * 64 + lane] = m_run;
    xo[CPL * 16 * 64 + 64 + lane] = l_tot;
  }
  __syncthreads();
  if (kh == 1) return;
  float inv = 0.f, lse2 = -INFINITY;
  if (cnt > 0) {
    const float m1 = xo[CPL * 16 * 64 + lane], l1 = xo[CPL * 16 * 64 + 64 + lane];
    const float mm = fmaxf(m_run, m1);
    const float a0 = exp2_fast(m_run - mm), a1 = exp2_fast(m1 - mm);
    const float l = l_tot * a0 + l1 * a1;
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[ct][r] = o[ct][r] * a0 + xo[(ct * 16 + r) * 64 + lane] * a1;
    inv = 1.0f / l;
    lse2 = mm + log2f(l);
  }
  // Output row of query qh*32 + m: register r holds channels CPL*i .. CPL*i + CPL-1 (one per
  // tile), i = 8(r/4) + 4*hf + r%4.
  const int qr = qh * 32 + m;
  const long long n = a.orig ? token_of(g, i, qr) : (long long)i * kBlock + qr;
  float* orow = a.out + ((long long)bh * g.N + n) * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ci = 8 * (r >> 2) + 4 * hf + (r & 3);
    if constexpr (CPL == 4)
      *reinterpret_cast<float4*>(orow + 4 * ci) =
          make_float4(o[0][r] * inv, o[1][r] * inv, o[2][r] * inv, o[3][r] * inv);
    else
      *reinterpret_cast<float2*>(orow + 2 * ci) = make_float2(o[0][r] * inv, o[1][r] * inv);
  }
  if (a.lse && hf == 0)
    a.lse[(long long)bh * g.N + (long long)i * kBlock + qr] = cnt > 0 ? lse2 * 0.6931471805599453f : -INFINITY;
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

// Column order for the whole launch (short lists). Workgroup b runs on XCD b % 8 (round-robin
// dispatch), so the table lists, for every XCD, the queue of pairs it will run:
//  1. Runs: G adjacent temporal columns (patches in raster order) of one head, each
//     column's frame pairs in time order, dealt round-robin to the 8 XCDs: on XCD x queue
//     rank k holds column 8G*(k / (G*C)) + G*x + (k / C) % G, frame pair k % C (columns
//     that do not fill a last cycle over the 8 XCDs keep the plain mapping). The workgroups an XCD holds at
//     once then come from one run: temporally adjacent pairs of neighbouring patches, whose
//     kept key blocks largely coincide, so their tiles hit in that XCD's L2.
//  2. Long pairs first: within each XCD's queue, the pairs whose kept count exceeds 1.25x
//     the mean move to the front (both parts keep their queue order). Started late, the
//     longest pairs formed a tail in which most of an XCD's slots sat idle (72% slot use at
//     480p, 59% with the dynamic threshold).
//  3. Short pairs last: the final 2 x 64 positions of each queue are written longest-first.
// Workgroup x of k_pair_order writes the queue of XCD x; `total` is the sum of all kept
// counts (each row belongs to exactly one pair); `wpart` (16 ints), `tail_gi` and `tail_cost`
// (kQueueTail ints each) are LDS scratch.
// Queue rank k of XCD x in the column order (workgroup 8k + x): the pair index (b, h, pair)
// flattened, before the long-first and tail reorderings.
__device__ __forceinline__ int column_item(int k, int x, int F, int pairs, int bhs) {
  const int C = pairs / F;
  const int G = column_run_width(C);
  const int full = (bhs * pairs / (8 * G * C)) * 8 * G * C;
  const int b = 8 * k + x;
  int logical = b;
  if (b < full) {
    const int col = (k / (G * C)) * 8 * G + x * G + (k / C) % G;
    logical = col * C + k % C;
  }
  const int h = logical / pairs, pos = logical - h * pairs;
  return h * pairs + (pos % C) * F + pos / C;  // column pos / C, frame pair pos % C
}
// Kept count of pair gi (the sum of its blocks' list lengths).
__device__ __forceinline__ int pair_cost(const int32_t* __restrict__ counts, int gi, int nb, int F, int pairs) {
  const int h = gi / pairs, pair = gi - h * pairs;
  int ba, bb;
  pair_blocks(pair, F, nb, ba, bb);
  const int32_t* c = counts + (long long)h * nb;
  int k = ba >= 0 ? min(max(c[ba], 0), nb) : 0;
  if (bb >= 0) k += min(max(c[bb], 0), nb);
  return k;
}

// pre_gi / pre_cost: this thread's queue item k = t and its cost, already fetched by the
// caller when the queue has at most 1024 items (else ignored and fetched here).
__device__ void xcd_queue(const int32_t* __restrict__ counts, int32_t* __restrict__ order, int nb, int F, int pairs,
                          int bhs, int x, long long total, int* wpart, int* tail_gi, int* tail_cost, int pre_gi,
                          int pre_cost) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int grid = bhs * pairs;
  auto long_cost = [&](int cost) { return 4ll * cost * grid > 5ll * total; };  // above 1.25x the mean
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
  const bool one = n_x <= 1024;  // one item per thread: its gi and cost stay in registers
  int cnt = 0;
  if (one)
    cnt = t < n_x && long_cost(pre_cost) ? 1 : 0;
  else
    for (int k = t; k < n_x; k += 1024)
      cnt += long_cost(pair_cost(counts, column_item(k, x, F, pairs, bhs), nb, F, pairs));
  int nlong;
  block_scan(cnt, nlong);
  // The last kQueueTail positions (two generations of the XCD's resident workgroups) are
  // collected in LDS and then written longest-first, so the queue ends with its shortest
  // pairs and the XCD's slots drain together.
  const int tail0 = max(n_x - kQueueTail, 0);
  int base_l = 0, base_s = nlong;
  for (int c0 = 0; c0 < n_x; c0 += 1024) {
    const int k = c0 + t;
    const bool valid = k < n_x;
    const int gi = !valid ? 0 : one ? pre_gi : column_item(k, x, F, pairs, bhs);
    const int cost = !valid ? 0 : one ? pre_cost : pair_cost(counts, gi, nb, F, pairs);
    const bool lg = valid && long_cost(cost);
    int both;
    const int v = (lg ? 1 : 0) | ((valid && !lg) ? 1 << 16 : 0);  // two counts <= 1024, packed
    const int ex = block_scan(v, both);
    if (valid) {
      const int p = lg ? base_l + (ex & 0xffff) : base_s + (ex >> 16);
      if (p >= tail0) {
        tail_gi[p - tail0] = gi;
        tail_cost[p - tail0] = cost;
      } else {
        order[8 * p + x] = gi;
      }
    }
    base_l += both & 0xffff;
    base_s += both >> 16;
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

// Visiting order of the query-block pairs (i, i + F) of each (b, h), F = nbh*nbw; pair p covers
// blocks a = (p / F)*2F + p % F and a + F, so pair tp*F + s is frame pair tp of patch s (the
// last frame of an odd T pairs neighbouring patches instead: pair_blocks).
// Two orders, chosen once per launch from the mean kept count per row over all heads:
//  - short lists (mean <= kColumnMaxCount): column order for the whole launch, the queues of
//    the 8 XCDs written by workgroups 0-7 (xcd_queue above).
//  - otherwise: pairs longest-first by their kept count (counting sort), so the long rows
//    do not form the tail; with long lists neighbouring workgroups start too far apart
//    for L2 reuse and the balance matters more.
// Every workgroup computes the same mean (a fixed-order sum over all rows, or, beyond
// kMeanSample rows, over kMeanSample evenly spaced ones scaled to the row count, so that the
// work per workgroup stays bounded); workgroup 0 stores the mode. The grid is
// min(max(B*H, 8), kOrderGrid) workgroups; in the longest-first mode each takes the heads
// blockIdx.x, blockIdx.x + gridDim.x, ...
constexpr int kColumnMaxCount = 96;
constexpr long long kMeanSample = 1 << 16;
constexpr int kOrderGrid = 4096;

__global__ __launch_bounds__(1024) void k_pair_order(const int32_t* __restrict__ counts, int32_t* __restrict__ order,
                                                     int32_t* __restrict__ mode_out, int nb, int F, int pairs,
                                                     long long rows) {
  __shared__ int hist[2 * kMaxBlocks + 1];
  __shared__ int scan_part[16];
  __shared__ long long wsum[16];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int bhs = (int)(rows / nb);

  // Workgroups 0-7 write the XCD queues if the lists are short: with one queue item per thread
  // they fetch its kept count now, while the mean is summed (both loads in flight at once).
  int pre_gi = 0, pre_cost = 0;
  if (blockIdx.x < 8) {
    const int x = (int)blockIdx.x;
    const int n_x = (bhs * pairs - x + 7) / 8;
    if (n_x <= 1024 && t < n_x) {
      pre_gi = column_item(t, x, F, pairs, bhs);
      pre_cost = pair_cost(counts, pre_gi, nb, F, pairs);
    }
  }

  const long long nsum = rows < kMeanSample ? rows : kMeanSample;
  long long part = 0;
  for (long long k = t; k < nsum; k += 1024) {
    const long long r = nsum == rows ? k : k * rows / kMeanSample;
    part += min(max(counts[r], 0), nb);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
  if (lane == 0) wsum[wv] = part;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < 16; ++w) total += wsum[w];
  if (nsum != rows) total = total * rows / kMeanSample;
  const bool column = total <= (long long)kColumnMaxCount * rows;
  if (blockIdx.x == 0 && t == 0) {
    mode_out[0] = column ? 1 : 0;
    mode_out[1] = 0;  // the attention's tail counter (claim_item)
  }
  if (column) {
    if (blockIdx.x < 8)
      xcd_queue(counts, order, nb, F, pairs, bhs, (int)blockIdx.x, total, scan_part, hist, hist + kQueueTail, pre_gi,
                pre_cost);
    return;
  }

  const int kmax = 2 * nb;
  for (long long bh = blockIdx.x; bh < bhs; bh += gridDim.x) {
    const int32_t* c = counts + bh * nb;
    auto blk_count = [&](int blk) { return min(max(c[blk], 0), nb); };
    auto key = [&](int pr) {
      int ba, bb;
      pair_blocks(pr, F, nb, ba, bb);
      int k = ba >= 0 ? blk_count(ba) : 0;
      if (bb >= 0) k += blk_count(bb);
      return k;
    };
    __syncthreads();  // the previous head's placement is done with hist
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
}

// Longest-first order of the query blocks of each (b, h), for the float32 path; workgroup
// blockIdx.x takes the heads blockIdx.x, blockIdx.x + gridDim.x, ...
__global__ __launch_bounds__(1024) void k_row_order(const int32_t* __restrict__ counts, int32_t* __restrict__ order,
                                                    int nb, int bhs) {
  __shared__ int hist[kMaxBlocks + 1];
  __shared__ int scan_part[16];
  const int t = threadIdx.x;
  for (long long bh = blockIdx.x; bh < bhs; bh += gridDim.x) {
    const int32_t* c = counts + bh * nb;
    __syncthreads();  // the previous head's placement is done with hist
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
}

}  // namespace

hipError_t launch_sparse_attn(const KGeom& g, int dtype, float scale, const void* q, const void* k,
                              const void* vt, const int32_t* counts, const int32_t* lists, void* out,
                              int out_original_order, int qk_original_order, int v_original_order, float* lse,
                              int32_t* row_order, hipStream_t s) {
  const unsigned bhs = (unsigned)(g.B * g.H);
  if (dtype == ABLA_BF16) {
    const int F = g.nbh * g.nbw;
    const int pairs = ((g.T + 1) / 2) * F;
    int32_t* mode = row_order + (long long)bhs * g.nb;  // after the order array (pairs <= nb per head)
    k_pair_order<<<dim3(bhs < 8 ? 8 : bhs > kOrderGrid ? kOrderGrid : bhs), 1024, 0, s>>>(
        counts, row_order, mode, g.nb, F, pairs, (long long)bhs * g.nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.vt = static_cast<const uint16_t*>(vt);
    a.counts = counts;
    a.lists = lists;
    a.order = row_order;
    a.walk_mode = mode;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.g = g;
    a.pairs = pairs;
    a.grid = (int)((long long)bhs * pairs);
    // The last kQueueTail positions of each XCD's queue (its shortest pairs) form the tail in
    // column order, 1.5 kQueueTail positions for long lists (720p: -1.1% against 128 positions;
    // 480p and 480p-dyn lose 0.7-2% with the longer tail).
    a.main_col = max(0, a.grid / 8 - kQueueTail) * 8;
    a.main_long = max(0, a.grid / 8 - 3 * kQueueTail / 2) * 8;
    a.tail_cnt = mode + 1;
    a.scale = scale;
    a.c2 = scale * 1.4426950408889634f;
    a.orig = out_original_order;
    a.qk_orig = qk_original_order;
    a.magic_f = (1ull << 32) / (unsigned long long)F + 1;
    a.magic_w = (1ull << 32) / (unsigned long long)g.nbw + 1;
    // Enough tail workgroups for either mode (the column mode's extra ones exit at once).
    const dim3 grid((unsigned)(a.main_long + kTailOversub * (a.grid - a.main_long)));
    const int variant = (g.d == 128 ? 4 : 0) | (qk_original_order ? 2 : 0) | (v_original_order ? 1 : 0);
    switch (variant) {
      case 7: k_attn_bf16<128, true, true><<<grid, 256, 0, s>>>(a); break;
      case 6: k_attn_bf16<128, true, false><<<grid, 256, 0, s>>>(a); break;
      case 5: k_attn_bf16<128, false, true><<<grid, 256, 0, s>>>(a); break;
      case 4: k_attn_bf16<128, false, false><<<grid, 256, 0, s>>>(a); break;
      case 3: k_attn_bf16<64, true, true><<<grid, 256, 0, s>>>(a); break;
      case 2: k_attn_bf16<64, true, false><<<grid, 256, 0, s>>>(a); break;
      case 1: k_attn_bf16<64, false, true><<<grid, 256, 0, s>>>(a); break;
      default: k_attn_bf16<64, false, false><<<grid, 256, 0, s>>>(a); break;
    }
  } else {
    k_row_order<<<dim3(bhs > kOrderGrid ? kOrderGrid : bhs), 1024, 0, s>>>(counts, row_order, g.nb, (int)bhs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    AttnArgsF32 a;
    a.q = static_cast<const float*>(q);
    a.k = static_cast<const float*>(k);
    a.v = static_cast<const float*>(vt);
    a.counts = counts;
    a.lists = lists;
    a.order = row_order;
    a.out = static_cast<float*>(out);
    a.lse = lse;
    a.g = g;
    a.c2 = scale * 1.4426950408889634f;
    a.orig = out_original_order;
    const dim3 grid((unsigned)((long long)bhs * g.nb));
    const int variant = (g.d == 128 ? 4 : 0) | (qk_original_order ? 2 : 0) | (v_original_order ? 1 : 0);
    switch (variant) {
      case 7: k_attn_f32<128, true, true><<<grid, 256, 0, s>>>(a); break;
      case 6: k_attn_f32<128, true, false><<<grid, 256, 0, s>>>(a); break;
      case 5: k_attn_f32<128, false, true><<<grid, 256, 0, s>>>(a); break;
      case 4: k_attn_f32<128, false, false><<<grid, 256, 0, s>>>(a); break;
      case 3: k_attn_f32<64, true, true><<<grid, 256, 0, s>>>(a); break;
      case 2: k_attn_f32<64, true, false><<<grid, 256, 0, s>>>(a); break;
      case 1: k_attn_f32<64, false, true><<<grid, 256, 0, s>>>(a); break;
      default: k_attn_f32<64, false, false><<<grid, 256, 0, s>>>(a); break;
    }
  }
  return hipGetLastError();
}

// Scratch of the allocation-free forward (abla_sparse_attn_fwd_noalloc): the visiting order
// and walk-mode word that launch_sparse_attn otherwise keeps in the caller's workspace. Each
// GPU the library runs on holds its own copy until the process ends; every call on that GPU
// shares it (k_pair_order or k_row_order rewrite all of it before the attention reads it, so
// nothing needs clearing), and calls that overlap on one GPU race.
static __device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device. The array's name in host code is only a
// host-side handle; its address on each device comes from hipGetSymbolAddress, once per device.
hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

}  // namespace abla
