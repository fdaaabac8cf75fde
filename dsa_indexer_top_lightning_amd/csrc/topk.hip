// Per-query top-k selection on gfx950.
//
// For each query row, keep the `topk` candidates with the largest index score
// (GLM-5.2 IndexShare page, section 1: top-k token indices are selected from the
// indexer scores; index_topk = 2048 in the page's verified facts).  Equal scores
// go to the lower position; the kept positions are written in ascending order.
// A row with fewer candidates than topk keeps them all and pads with -1 (the
// Megatron-Bridge pull request's fix for packed sequences shorter than
// index_topk).
//
// Method (one workgroup of 1024 threads per row):
//  1. scores -> uint32 keys that order like the floats (-0.0 folded onto +0.0);
//     rows that fit are cached in LDS so HBM is read once;
//  2. radix select of the k-th largest key tau in three passes over 11/11/10-bit
//     digits, each an LDS histogram built with LDS atomics, and a one-wave
//     suffix scan that finds the digit holding the k-th key;
//  3. an ordered pass that keeps every key > tau and the first (in position
//     order) `rem` keys == tau, writing each kept position to its slot found by
//     wavefront ballots + popcount prefix sums and a cross-wave prefix in LDS.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int64_t TK_CACHE_KEYS = 32768;  // 128 KiB of LDS

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask, int lane) {
  return (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
}

template <bool CACHE>
__global__ __launch_bounds__(TK_THREADS) void topk_rows(TopkParams p) {
  extern __shared__ uint32_t kcache[];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wcnt[2][TK_WAVES];
  __shared__ uint32_t sh_digit, sh_rem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  int64_t ks, ke;
  clamp_range(p.key_start, p.key_end, row, p.s_cap, ks, ke);
  const int64_t n = ke - ks;
  const int K = p.topk;
  int32_t* out = p.out + row * (int64_t)K;

  if (n <= K) {
    for (int i = tid; i < K; i += TK_THREADS) out[i] = (i < n) ? (int32_t)(ks + i) : -1;
    return;
  }
  const float* src = p.scores + row * p.ld + ks;
  if constexpr (CACHE) {
    for (int64_t i = tid; i < n; i += TK_THREADS) kcache[i] = order_key(src[i]);
    __syncthreads();
  }
  auto key_at = [&](int64_t i) -> uint32_t {
    if constexpr (CACHE) return kcache[i];
    else return order_key(src[i]);
  };

  uint32_t prefix = 0, pmask = 0, rem = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass < 2 ? 2047u : 1023u;
    for (int i = tid; i < 2048; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += TK_THREADS) {
      const uint32_t key = key_at(i);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane L owns digits [32L, 32L+32); suffix sums over lanes
      uint32_t c = 0;
      for (int d = 0; d < 32; ++d) c += hist[32 * lane + d];
      uint32_t x = c;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(x, off, 64);
        if (lane + off < 64) x += v;
      }
      // x = number of candidates with digit >= 32*lane; non-increasing in lane
      const uint64_t ge = __ballot(x >= rem);
      const int L = __popcll(ge) - 1;  // last lane whose suffix reaches rem (>= 0: total >= rem)
      if (lane == L) {
        uint32_t above = x - c;
        int d = 32 * lane + 31;
        for (; d > 32 * lane; --d) {
          const uint32_t h = hist[d];
          if (above + h >= rem) break;
          above += h;
        }
        sh_digit = (uint32_t)d;
        sh_rem = rem - above;
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= dmask << shift;
    rem = sh_rem;
    __syncthreads();
  }
  const uint32_t tau = prefix;  // the k-th largest key; `rem` keys equal to it are kept

  uint32_t base_eq = 0, base_sel = 0;
  for (int64_t c0 = 0; c0 < n && base_sel < (uint32_t)K; c0 += TK_THREADS) {
    const int64_t i = c0 + tid;
    const bool in = i < n;
    const uint32_t key = in ? key_at(i) : 0u;
    const bool gt = in && key > tau;
    const bool eq = in && key == tau;
    const uint64_t meq = __ballot(eq);
    if (lane == 0) wcnt[0][wave] = (uint32_t)__popcll(meq);
    __syncthreads();
    uint32_t eq_before = base_eq, eq_total = 0;
    for (int w = 0; w < TK_WAVES; ++w) {
      const uint32_t v = wcnt[0][w];
      eq_total += v;
      if (w < wave) eq_before += v;
    }
    eq_before += lane_prefix(meq, lane);
    const bool sel = gt || (eq && eq_before < rem);
    const uint64_t msel = __ballot(sel);
    if (lane == 0) wcnt[1][wave] = (uint32_t)__popcll(msel);
    __syncthreads();
    uint32_t sel_before = base_sel, sel_total = 0;
    for (int w = 0; w < TK_WAVES; ++w) {
      const uint32_t v = wcnt[1][w];
      sel_total += v;
      if (w < wave) sel_before += v;
    }
    sel_before += lane_prefix(msel, lane);
    if (sel && sel_before < (uint32_t)K) out[sel_before] = (int32_t)(ks + i);
    base_eq += eq_total;
    base_sel += sel_total;
    __syncthreads();
  }
}

}  // namespace

size_t topk_workspace_bytes(int, int, int, int64_t) { return 0; }

hipError_t launch_topk(const TopkParams& p, void*, size_t, hipStream_t st, int* n_launches) {
  const int64_t rows = (int64_t)p.B * p.T;
  if (rows == 0) return hipSuccess;
  if (p.s_cap <= TK_CACHE_KEYS) {
    const size_t lds = (size_t)(p.s_cap > 0 ? p.s_cap : 1) * 4;
    static std::atomic<size_t> high{0};
    const hipError_t attr = allow_dynamic_lds(reinterpret_cast<const void*>(topk_rows<true>), lds, high);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(topk_rows<true>, dim3((unsigned)rows), dim3(TK_THREADS), lds, st, p);
  } else {
    hipLaunchKernelGGL(topk_rows<false>, dim3((unsigned)rows), dim3(TK_THREADS), 0, st, p);
  }
  if (n_launches) ++*n_launches;
  return hipGetLastError();
}

}  // namespace dsa
