// The sparse-attention kernels' latent-row tile (forward and backward): layout constants,
// the global-to-LDS gather of 64 selected rows, and the barriers around it.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace dsa {
namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int MT = 64;            // selected rows per tile
constexpr int MROW = 576;         // latent row (Dc + Dr)
constexpr int MDC = 512;          // value dims
constexpr int MRB = MROW * 2;     // bytes per latent row
constexpr int MCH = MRB / 16;     // 16-byte chunks per row (72)
constexpr int MHG = 64;           // heads per workgroup
constexpr int SEG = 128;                         // bytes of a row segment (8 chunks, one cache line)
constexpr int GROUP_BYTES = MT * SEG;            // one segment of all 64 rows (8 KiB)
constexpr int NGROUP = MRB / SEG;                // 9 segments per row
constexpr int TILE_BYTES = NGROUP * GROUP_BYTES; // 73728

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// LDS tile layout: chunk c (16 B) of row r sits at byte
//   (c / 8) * 8192 + r * 128 + 16 * ((c % 8) ^ perm(r)),   perm(r) = bit-reverse of ((r >> 1) & 7).
// Sixteen consecutive rows read at one chunk (K fragments) then cover 16 distinct
// 16-byte bank groups, and so do the 4 rows x 4 chunks of a half-wave of
// transposing V reads (rows r and r + 2 differ in bit 2 of perm).
__device__ __forceinline__ int perm(int r) {
  const int j = (r >> 1) & 7;
  return ((j & 1) << 2) | (j & 2) | ((j >> 2) & 1);
}

// two floats -> packed bf16 pair (round to nearest even, hardware conversion)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// every global load of this wave has landed, the asm global-to-LDS copies included
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Global-to-LDS copies issued as inline asm.  Written with the compiler's builtin, the
// copies are LDS stores it cannot tell apart from the tile being read, so it makes
// every later LDS access wait for all of them (vmcnt(0)) and the next tile's gather
// could no longer overlap the current tile's math.  Issued here, they are ordered by
// the memory clobber and waited for explicitly at the tile barrier (vmcnt).  Each copy
// sets M0 one wait state before the load reads it; the lane's data lands at
// M0 + instruction offset + size * lane (the immediate offset moves the LDS address
// as well as the global one, so M0 takes the LDS offset minus the global one).  The
// compiler issues no other global-to-LDS copy in these kernels and nothing else uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int GOFF, int LOFF>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  static_assert(LOFF >= GOFF && GOFF >= 0 && GOFF < 4096, "offset outside the immediate field");
  asm volatile("s_add_i32 m0, %1, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
               ::"v"(src), "s"(lds_base), "i"(GOFF), "i"(LOFF - GOFF)
               : "memory", "m0", "scc");  // s_add_i32 writes the scalar condition code
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barriers that order LDS traffic only.  __syncthreads() also waits for every
// outstanding global load of the wave (vmcnt(0)), which would stall on the next tile's
// gather that is meant to fly across the barrier.  The memory clobber keeps the
// compiler from moving memory operations across either barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// ... and the tile barrier: this wave's gather of the current tile has landed (all but
// the newest global load, the entry load issued after it) before the barrier.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Per-lane sources of a tile's gather: wave w loads rows [16w, 16w + 16) as 2 row octets x
// the row's segments; in each load lane i fills row 8q + i/8 at stored chunk i%8, which holds
// the row's logical chunk (i%8) ^ perm(row).  Lane l passes the source row number of tile
// row l; rows sit row_bytes apart from `base` (32-bit offsets).
struct GatherSrc {
  const unsigned char* a[2];
};
__device__ __forceinline__ GatherSrc gather_src(const unsigned char* base, uint32_t row_bytes, int32_t lane_row,
                                                int wave, int lane) {
  GatherSrc g;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * wave + 8 * q + (lane >> 3);
    const int32_t ri = __shfl(lane_row, row, 64);
    g.a[q] = base + (uint32_t)ri * row_bytes + 16 * ((lane & 7) ^ perm(row));
  }
  return g;
}

// Part k (0..5) of a tile's gather into the wave's share of the tile at LDS byte `dst`
// (= tile base + wave * 16 * SEG): three of its 18 copies (segment m of row octet q is copy
// 2m + q: global byte m * 128 of each row, LDS group m).  NSEG = 8 leaves out segment 8 (rows
// of 1024 bytes).
template <int NSEG = NGROUP>
__device__ __forceinline__ void gather_part(int k, uint32_t dst, const GatherSrc& g) {
  switch (k) {
    case 0:
      dma16<0 * SEG, 0 * GROUP_BYTES>(g.a[0], dst);
      dma16<0 * SEG, 0 * GROUP_BYTES + 1024>(g.a[1], dst);
      dma16<1 * SEG, 1 * GROUP_BYTES>(g.a[0], dst);
      break;
    case 1:
      dma16<1 * SEG, 1 * GROUP_BYTES + 1024>(g.a[1], dst);
      dma16<2 * SEG, 2 * GROUP_BYTES>(g.a[0], dst);
      dma16<2 * SEG, 2 * GROUP_BYTES + 1024>(g.a[1], dst);
      break;
    case 2:
      dma16<3 * SEG, 3 * GROUP_BYTES>(g.a[0], dst);
      dma16<3 * SEG, 3 * GROUP_BYTES + 1024>(g.a[1], dst);
      dma16<4 * SEG, 4 * GROUP_BYTES>(g.a[0], dst);
      break;
    case 3:
      dma16<4 * SEG, 4 * GROUP_BYTES + 1024>(g.a[1], dst);
      dma16<5 * SEG, 5 * GROUP_BYTES>(g.a[0], dst);
      dma16<5 * SEG, 5 * GROUP_BYTES + 1024>(g.a[1], dst);
      break;
    case 4:
      dma16<6 * SEG, 6 * GROUP_BYTES>(g.a[0], dst);
      dma16<6 * SEG, 6 * GROUP_BYTES + 1024>(g.a[1], dst);
      dma16<7 * SEG, 7 * GROUP_BYTES>(g.a[0], dst);
      break;
    default:
      dma16<7 * SEG, 7 * GROUP_BYTES + 1024>(g.a[1], dst);
      if constexpr (NSEG > 8) {
        dma16<8 * SEG, 8 * GROUP_BYTES>(g.a[0], dst);
        dma16<8 * SEG, 8 * GROUP_BYTES + 1024>(g.a[1], dst);
      }
      break;
  }
}
template <int NSEG = NGROUP>
__device__ __forceinline__ void gather_tile(uint32_t dst, const GatherSrc& g) {
#pragma unroll
  for (int k = 0; k < 6; ++k) gather_part<NSEG>(k, dst, g);
}

}  // namespace mla
}  // namespace dsa
