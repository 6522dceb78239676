// Shared device helpers of the attention kernels (forward and backward): LDS tile
// geometry and swizzles for the gfx950 32x32x16 bf16 MFMA operands, the key-row
// permutation that makes a score tile's accumulators reusable as the next MFMA's
// operand, global->LDS tile loads and wait/barrier primitives.
#pragma once

#include "common.h"

namespace abla {
namespace {

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

// 16-byte chunk swizzles (bank-conflict-free MFMA operand reads): row r's chunk c of a
// token-major tile sits at position c ^ k_swz(r). Spreads the row operand reads (each lane a
// 16-byte chunk, consecutive rows at one logical chunk) over all banks.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// Swizzle of the tiles that are also read with transpose loads (the backward's): besides the
// row reads, each half-wave of a transpose load reads 4 rows x 4 consecutive chunks, which
// k_swz maps onto the same banks. For d = 128 (16 chunks per row) the table A[r%4] ^ (r/4)%4
// with A = {0, 6, 10, 12} is a bijection on 16 rows and gives the 4 rows of a transpose load
// distinct chunk groups in both a 32- and a 64-bank LDS model (checked by enumeration on the
// host); for d = 64 (8 chunks) 2*(r%4) + (r/4)%2 does so except for a few two-way collisions of
// row reads 8 rows apart. Both repeat every 16 rows.
template <int D>
__device__ __forceinline__ int kt_swz(int r) {
  if constexpr (D == 128)
    return (((r & 1) ? 6 : 0) ^ ((r & 2) ? 10 : 0)) ^ ((r >> 2) & 3);
  else
    return ((r & 3) << 1) | ((r >> 2) & 1);
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

__device__ __forceinline__ void wait_vm_lgkm_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer resource (gfx9 V#) over `bytes` bytes at `base`: raw addressing, no stride.
// Tile loads go through buffer_load ... lds rather than global_load_lds: the compiler's
// wait-count pass tracks the buffer form on the vector-memory counter only, so the LDS
// operand reads of the current tile keep partial lgkmcnt waits while the next tile's
// loads are in flight.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ void raw_buffer_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) uint32_t* lds, int size,
                                    int voffset, int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");

// Plain 16-byte buffer load into registers (bounds-checked against the resource's size).
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
__device__ f32x4v_t raw_buffer_load_f32x4(i32x4_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4f32");

__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));  // stride 0
  r.z = (int)bytes;                                                 // num_records (bytes)
  r.w = 0x00020000;                                                 // 32-bit data format
  return r;
}

// Issue this thread's 16-byte global->LDS loads of one K tile (or one V^T tile) that
// starts `tile` bytes into the resource. Load `it` of thread t fills LDS unit it*256 + t
// of the slot; its source is `off` + it*stride bytes into the tile (for both tile kinds and
// both head dims the swizzled source of unit it*256 + t is 4096 bytes past that of unit
// t in fractal order: 16 K rows of 256 bytes, 32 K rows of 128 bytes, 32 V^T rows of 128
// bytes, all with a swizzle that repeats every 16 or 32 rows; a K tile read in the
// original token order passes its own stride). `w` is the wave index (uniform).
template <int BYTES>
__device__ __forceinline__ void issue_rows(char* dst_slot, int w, i32x4_t rsrc, uint32_t tile, uint32_t off,
                                           uint32_t stride = 4096) {
  constexpr int LOADS = BYTES / 16 / 256;
  char* dst = dst_slot + w * 64 * 16;
#pragma unroll
  for (int it = 0; it < LOADS; ++it)
    raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) uint32_t*)(dst + it * 256 * 16), 16, (int)off,
                        (int)(tile + it * stride), 0, 0);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_ptr;

// Transposed operands. The A operand of a product over the TRANSPOSE of a token-major tile X
// (channel rows, token columns) is read with the gfx950 LDS transpose load: lane l needs
// X^T[dt*32 + l%32][tb + 8*(l/32) + e], e = 0..7, i.e. 8 consecutive tokens of one channel.
// ds_read_b64_tr_b16 works on groups of 16 lanes: each lane names 8 bytes (4 bf16) and lane i
// of the group receives element i%4 of the read named by lane 4e + i/4 as its element e. So
// lane m of a group names token tb + 8*hi + 4*half + m/4, channels c0 + 4*(m%4) .. +3
// (c0 = dt*32 + 16*(group&1)), and lane i then holds channel c0 + i of four consecutive
// tokens; two such reads give the 8 tokens (established with an in-bounds probe). Tiles read
// this way are laid out with kt_swz.
//
// The transpose reads go through inline asm, with the wait inside the block. The compiler's
// wait-count pass does not prove that a ds_read_b64_tr_b16 builtin misses the LDS slot that
// the next tile's buffer_load ... lds is filling, so before the first builtin transpose load
// of a step it waits for every load in flight (vmcnt(0)), which stalls the next tile's
// prefetch. The tiles read here were completed by the step's barrier and the prefetch fills
// the other slot, so no such wait is needed; each block ends with lgkmcnt(0), so its results
// are complete when it returns.
__device__ __forceinline__ uint32_t lds_offset(const char* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}
// Byte offsets, relative to a token-major tile laid out with kt_swz, of the two 8-byte
// transpose reads that give lane `lane` its operand for channel tile dt and tokens
// tb + 8*(lane/32) + 0..7 (the layout above).
template <int D>
__device__ __forceinline__ void tr_rel(int dt, int tb, int lane, uint32_t& a0, uint32_t& a1) {
  const int g = lane >> 4, m = lane & 15;
  const int ch = dt * 32 + 16 * (g & 1) + 4 * (m & 3);
  const int tok = tb + 8 * (g >> 1) + (m >> 2);
  const int r0 = kperm(tok), r1 = kperm(tok + 4);
  a0 = (uint32_t)(r0 * D * 2 + (((ch >> 3) ^ kt_swz<D>(r0)) << 4) + (ch & 7) * 2);
  a1 = (uint32_t)(r1 * D * 2 + (((ch >> 3) ^ kt_swz<D>(r1)) << 4) + (ch & 7) * 2);
}
// out[k] = the transposed operand of channel tile k (tokens tb .. of the tile), for the NT = D/32
// channel tiles, where a[2k], a[2k+1] are the LDS addresses of tile + tr_rel(k, tb0, lane) and the
// tile / token block differs from
// (tile, tb0) by the constant byte offset OFF. Tokens tb0 + 16*n keep the same swizzle (it
// repeats every 16 rows), so OFF = 16*n*D*2 (plus a slot distance) is exact.
template <int NT, int OFF>
__device__ __forceinline__ void tr_chunks_at(const uint32_t* a, bf16x8_t (&out)[NT]);
template <int OFF>
__device__ __forceinline__ void tr_chunks_at_4(const uint32_t* a, bf16x8_t (&out)[4]) {
  i16x4_t r[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
      "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
      "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const i16x4_t both[2] = {r[2 * k], r[2 * k + 1]};
    __builtin_memcpy(&out[k], both, 16);
  }
}
template <int OFF>
__device__ __forceinline__ void tr_chunks_at_2(const uint32_t* a, bf16x8_t (&out)[2]) {
  i16x4_t r[4];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
      "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
      "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
      "ds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF));
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const i16x4_t both[2] = {r[2 * k], r[2 * k + 1]};
    __builtin_memcpy(&out[k], both, 16);
  }
}
template <int NT, int OFF>
__device__ __forceinline__ void tr_chunks_at(const uint32_t* a, bf16x8_t (&out)[NT]) {
  if constexpr (NT == 4)
    tr_chunks_at_4<OFF>(a, out);
  else
    tr_chunks_at_2<OFF>(a, out);
}

}  // namespace
}  // namespace abla
