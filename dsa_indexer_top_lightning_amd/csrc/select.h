// Device helpers of the radix selects (top-k and the fused indexer -> top-k): wave
// prefix counts, the digit search in a 2048-bin histogram, a workgroup prefix sum.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace dsa {

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask, int lane) {
  return (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
}

// Wave 0: in the 2048-bin histogram `hist` (digits of the candidates that match the
// prefix so far), find the digit holding the rem-th largest candidate and that
// candidate's rank among the keys with this digit (written to *digit, *rank).  The total
// count must be >= rem.  Callers synchronise before and after.
__device__ __forceinline__ void hist_find(const uint32_t* hist, uint32_t rem, uint32_t* digit, uint32_t* rank) {
  const int lane = threadIdx.x & 63;
  // lane L owns digits [32L, 32L+32) and sums them starting at bin L % 32 of its range, so
  // that the 64 lanes of each read hit different LDS banks; then suffix sums over lanes
  uint32_t c = 0;
  for (int d = 0; d < 32; ++d) c += hist[32 * lane + ((d + lane) & 31)];
  uint32_t x = c;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_down(x, off, 64);
    if (lane + off < 64) x += v;
  }
  // x = number of candidates with digit >= 32*lane; non-increasing in lane
  const uint64_t ge = __ballot(x >= rem);
  const int L = __popcll(ge) - 1;  // last lane whose suffix reaches rem (>= 0: total >= rem)
  const uint32_t above = __shfl(x - c, L, 64);  // candidates with a digit above lane L's range
  // inside lane L's range: lane i < 32 takes digit 32L + i; s = candidates with a digit in
  // [32L + i, 32L + 32); the digit is the highest i with above + s >= rem
  const uint32_t h = lane < 32 ? hist[32 * L + lane] : 0u;
  uint32_t sfx = h;
  for (int off = 1; off < 32; off <<= 1) {
    const uint32_t v = __shfl_down(sfx, off, 64);
    if (lane + off < 32) sfx += v;
  }
  const uint64_t hit = __ballot(lane < 32 && above + sfx >= rem);
  const int i = hit ? 63 - __clzll(hit) : 0;
  if (lane == i) {
    *digit = (uint32_t)(32 * L + i);
    *rank = rem - (above + sfx - h);
  }
}

// exclusive prefix sum of v over the workgroup (wsum: one LDS word per wave)
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = x - v;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();
  return before;
}

// digit layout of the three radix passes over a 32-bit key: 11, 11, then 10 bits
__host__ __device__ constexpr int radix_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__host__ __device__ constexpr uint32_t radix_mask(int pass) { return pass < 2 ? 2047u : 1023u; }

}  // namespace dsa
