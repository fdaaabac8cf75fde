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
// Method (one workgroup of 512 threads per row, several rows per compute unit):
//  1. scores -> uint32 keys that order like the floats (-0.0 folded onto +0.0);
//     rows that fit are cached in LDS so HBM is read once;
//  2. radix select of the k-th largest key tau in three passes over 11/11/10-bit
//     digits, each an LDS histogram built with LDS atomics, and a one-wave
//     suffix scan that finds the digit holding the k-th key;
//  3. an ordered pass that keeps every key > tau and the first (in position
//     order) `rem` keys == tau, writing each kept position to its slot found by
//     wavefront ballots + popcount prefix sums and a cross-wave prefix in LDS.
//
// Many rows longer than that cache (a long-context prefill chunk) read each row twice:
// a histogram of the top digit, then a pass that marks every position above the k-th
// key's digit in an LDS bitmap and keeps the keys sharing that digit in LDS, where the
// select finishes; the output is written in order from the bitmaps.
//
// Few long rows (decode over a long prefix) would leave most compute units idle
// with one workgroup per row, so there each row is cut into chunks of 2048 keys,
// one 256-thread workgroup per chunk, and the same radix select runs as a chain
// of launches on the stream: the three digit histograms are summed per row in a
// workspace with device-scope atomics, every later launch re-derives the digit
// prefix by scanning the finished histograms, a counting launch stores each
// chunk's number of keys > tau and == tau, and the emitting launch writes each
// chunk's kept positions after those of the chunks before it.
#include "dsa_internal.h"
#include "select.h"

namespace dsa {
namespace {

constexpr int TK_THREADS = 512;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int64_t TK_CACHE_KEYS = 32768;  // 128 KiB of LDS

struct SelectLds {
  uint32_t* hist;                  // [2048]
  uint32_t (*wcnt)[TK_WAVES];      // [2][TK_WAVES]
  uint32_t* sh;                    // [2]: digit, rank
};

// Radix passes `first`..2 over key_at(i), i in [0, n) (prefix / pmask / rem carry the
// digits fixed by earlier passes), then the ordered pass that writes every key > tau and
// the first `rem` keys == tau, in position order, to out[0..K).
template <class KeyAt>
__device__ void finish_select(KeyAt key_at, int64_t n, int64_t ks, int K, int32_t* out, int first, uint32_t prefix,
                              uint32_t pmask, uint32_t rem, const SelectLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll 1
  for (int pass = first; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass < 2 ? 2047u : 1023u;
    for (int i = tid; i < 2048; i += TK_THREADS) L.hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += TK_THREADS) {
      const uint32_t key = key_at(i);
      if ((key & pmask) == prefix) atomicAdd(&L.hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) hist_find(L.hist, rem, &L.sh[0], &L.sh[1]);
    __syncthreads();
    prefix |= L.sh[0] << shift;
    pmask |= dmask << shift;
    rem = L.sh[1];
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
    if (lane == 0) L.wcnt[0][wave] = (uint32_t)__popcll(meq);
    __syncthreads();
    uint32_t eq_before = base_eq, eq_total = 0;
    for (int w = 0; w < TK_WAVES; ++w) {
      const uint32_t v = L.wcnt[0][w];
      eq_total += v;
      if (w < wave) eq_before += v;
    }
    eq_before += lane_prefix(meq, lane);
    const bool sel = gt || (eq && eq_before < rem);
    const uint64_t msel = __ballot(sel);
    if (lane == 0) L.wcnt[1][wave] = (uint32_t)__popcll(msel);
    __syncthreads();
    uint32_t sel_before = base_sel, sel_total = 0;
    for (int w = 0; w < TK_WAVES; ++w) {
      const uint32_t v = L.wcnt[1][w];
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

template <bool CACHE>
__global__ __launch_bounds__(TK_THREADS) void topk_rows(TopkParams p) {
  extern __shared__ uint32_t kcache[];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wcnt[2][TK_WAVES];
  __shared__ uint32_t sh[2];

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  if (p.row_mask && !p.row_mask[row]) return;
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
  const SelectLds L{hist, wcnt, sh};
  if constexpr (CACHE) {
    // eight loads per thread in flight before any is waited for
    for (int64_t i0 = tid; i0 < n; i0 += 8 * TK_THREADS) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = i0 + u * TK_THREADS < n ? src[i0 + u * TK_THREADS] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * TK_THREADS < n) kcache[i0 + u * TK_THREADS] = order_key(v[u]);
    }
    __syncthreads();
    finish_select([&](int64_t i) { return kcache[i]; }, n, ks, K, out, 0, 0u, 0u, (uint32_t)K, L);
  } else {
    finish_select([&](int64_t i) { return order_key(src[i]); }, n, ks, K, out, 0, 0u, 0u, (uint32_t)K, L);
  }
}

// ----------------------------------------------------------------- long rows, many of them
// Rows longer than the LDS key cache (and enough of them to fill the chip).  A 512-thread
// workgroup per row, two per compute unit, so that one row's scans overlap the other's
// reads.  Histogram passes over the row fix its top digits (11 bits, then 11, then 10)
// until the digit holding the k-th key has at most LG_CAP keys (one pass on smooth
// score distributions).  One more pass then marks in an LDS bitmap every position whose
// fixed digits lie above that bin and copies the keys inside the bin, with their
// positions, into LDS, where the remaining digits are resolved.  Keys > tau are marked,
// keys == tau go to a second bitmap, and the kept positions are written in ascending
// order by a block scan over the bitmap words (the first `rem` of the == tau keys).
constexpr int LG_THREADS = 512;
constexpr int LG_WAVES = LG_THREADS / 64;
constexpr int64_t LG_MAX_KEYS = 262144;  // bitmap capacity: 2 x 32 KiB
constexpr int LG_CAP = 4096;             // keys of the k-th key's bin held in LDS
constexpr int LG_REP = 4;                // copies of a histogram (2048 * LG_REP <= 2 * LG_CAP)

size_t long_lds_bytes(int64_t s_cap) {
  const int64_t words = (s_cap + 31) / 32;
  return (size_t)(2 * words + 2 * LG_CAP) * 4;
}

__host__ __device__ constexpr int lg_shift(int level) { return level == 0 ? 21 : (level == 1 ? 10 : 0); }
__host__ __device__ constexpr uint32_t lg_mask(int level) { return level < 2 ? 2047u : 1023u; }

// f(i, key) for every i in [0, n), key = order_key(src[i]); the aligned body of the row
// is read with 16-byte loads, U per thread in flight.  REVERSE walks the body from its
// end, so that a pass that follows another starts on the part of the row read last
// (the part most likely still in L2).
template <bool REVERSE, class F>
__device__ __forceinline__ void for_each_key(const float* src, int64_t n, F&& f) {
  const int tid = threadIdx.x;
  const int64_t head = min<int64_t>(n, (int64_t)(((16u - ((uint32_t)(uintptr_t)src & 15u)) & 15u) >> 2));
  if (tid < head) f((int64_t)tid, order_key(src[tid]));
  const float4* body = reinterpret_cast<const float4*>(src + head);
  const int64_t nv = (n - head) >> 2;
  constexpr int U = 8;
  constexpr int64_t STEP = (int64_t)U * LG_THREADS;
  const int64_t full = nv / STEP;  // whole steps of U loads per thread
  for (int64_t c = 0; c < full; ++c) {
    const int64_t v = (REVERSE ? (full - 1 - c) : c) * STEP + tid;
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = body[v + u * LG_THREADS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = head + 4 * (v + u * LG_THREADS);
      f(i, order_key(x[u].x));
      f(i + 1, order_key(x[u].y));
      f(i + 2, order_key(x[u].z));
      f(i + 3, order_key(x[u].w));
    }
  }
  for (int64_t v = full * STEP + tid; v < nv; v += LG_THREADS) {
    const float4 x = body[v];
    const int64_t i = head + 4 * v;
    f(i, order_key(x.x));
    f(i + 1, order_key(x.y));
    f(i + 2, order_key(x.z));
    f(i + 3, order_key(x.w));
  }
  const int64_t t = head + 4 * nv + tid;  // at most 3 tail keys
  if (t < n) f(t, order_key(src[t]));
}

// the == tau positions of bitmap word x that are kept, given e_before of them earlier in the row
__device__ __forceinline__ uint32_t take_equal(uint32_t x, uint32_t e_before, uint32_t rem) {
  if (e_before >= rem) return 0u;
  uint32_t need = rem - e_before;
  if ((uint32_t)__popc(x) <= need) return x;
  uint32_t t = 0u;
  for (; need > 0; --need) {
    const uint32_t low = x & (0u - x);
    t |= low;
    x ^= low;
  }
  return t;
}

__global__ __launch_bounds__(LG_THREADS) void topk_long(TopkParams p, int map_words) {
  extern __shared__ uint32_t lds[];
  uint32_t* selmap = lds;
  uint32_t* eqmap = lds + map_words;
  uint32_t* ckey = lds + 2 * map_words;
  uint32_t* cpos = ckey + LG_CAP;
  uint32_t* rhist = ckey;  // the candidate area holds the replicated histograms until the marking pass
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[2][LG_WAVES];
  __shared__ uint32_t sh[3];

  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  if (p.row_mask && !p.row_mask[row]) return;
  int64_t ks, ke;
  clamp_range(p.key_start, p.key_end, row, p.s_cap, ks, ke);
  const int64_t n = ke - ks;
  const int K = p.topk;
  int32_t* out = p.out + row * (int64_t)K;
  if (n <= K) {
    for (int i = tid; i < K; i += LG_THREADS) out[i] = (i < n) ? (int32_t)(ks + i) : -1;
    return;
  }
  const float* src = p.scores + row * p.ld + ks;

  // histogram passes over the row until the k-th key's bin is small enough; lanes add to
  // copy tid % LG_REP so that lanes with one digit mostly hit different LDS banks
  uint32_t prefix = 0, pmask = 0, rem = (uint32_t)K, binc = 0;
  int level = 0;
  const uint32_t rep = (uint32_t)(tid % LG_REP);
#pragma unroll 1
  do {
    const int shift = lg_shift(level);
    const uint32_t dmask = lg_mask(level);
    for (int i = tid; i < 2048 * LG_REP; i += LG_THREADS) rhist[i] = 0;
    __syncthreads();
    auto add = [&](int64_t, uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&rhist[((key >> shift) & dmask) * LG_REP + rep], 1u);
    };
    if (level & 1) for_each_key<true>(src, n, add);
    else for_each_key<false>(src, n, add);
    __syncthreads();
    for (int i = tid; i < 2048; i += LG_THREADS) {
      uint32_t c = 0;
#pragma unroll
      for (int r = 0; r < LG_REP; ++r) c += rhist[i * LG_REP + r];
      hist[i] = c;
    }
    __syncthreads();
    if (wave == 0) hist_find(hist, rem, &sh[0], &sh[1]);
    __syncthreads();
    prefix |= sh[0] << shift;
    pmask |= dmask << shift;
    rem = sh[1];
    binc = hist[sh[0]];
    ++level;
    __syncthreads();
  } while (binc > (uint32_t)LG_CAP && level < 3);

  // marking pass: keys above the bin into the bitmap, keys inside it into LDS (or, with
  // every digit fixed, straight into the == tau bitmap)
  const int W = (int)((n + 31) >> 5);
  for (int w = tid; w < W; w += LG_THREADS) {
    selmap[w] = 0u;
    eqmap[w] = 0u;
  }
  if (tid == 0) sh[2] = 0u;
  __syncthreads();
  const bool collect = level < 3;
  auto mark = [&](int64_t i, uint32_t key) {
    const uint32_t kp = key & pmask;
    if (kp > prefix) {
      atomicOr(&selmap[i >> 5], 1u << (i & 31));
    } else if (kp == prefix) {
      if (collect) {
        const uint32_t j = atomicAdd(&sh[2], 1u);
        if (j < (uint32_t)LG_CAP) {
          ckey[j] = key;
          cpos[j] = (uint32_t)i;
        }
      } else {
        atomicOr(&eqmap[i >> 5], 1u << (i & 31));
      }
    }
  };
  if (level & 1) for_each_key<true>(src, n, mark);
  else for_each_key<false>(src, n, mark);
  __syncthreads();

  if (collect) {
    // the remaining digits among the binc collected keys
#pragma unroll 1
    for (int lv = level; lv < 3; ++lv) {
      const int shift = lg_shift(lv);
      const uint32_t dmask = lg_mask(lv);
      for (int i = tid; i < 2048; i += LG_THREADS) hist[i] = 0;
      __syncthreads();
      for (uint32_t j = tid; j < binc; j += LG_THREADS) {
        const uint32_t key = ckey[j];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      }
      __syncthreads();
      if (wave == 0) hist_find(hist, rem, &sh[0], &sh[1]);
      __syncthreads();
      prefix |= sh[0] << shift;
      pmask |= dmask << shift;
      rem = sh[1];
      __syncthreads();
    }
    const uint32_t tau = prefix;
    for (uint32_t j = tid; j < binc; j += LG_THREADS) {
      const uint32_t key = ckey[j], i = cpos[j];
      if (key > tau) atomicOr(&selmap[i >> 5], 1u << (i & 31));
      else if (key == tau) atomicOr(&eqmap[i >> 5], 1u << (i & 31));
    }
    __syncthreads();
  }

  // emit: thread t owns bitmap words [t*wpt, (t+1)*wpt)
  const int wpt = (W + LG_THREADS - 1) / LG_THREADS;
  const int w0 = min(W, tid * wpt), w1 = min(W, w0 + wpt);
  uint32_t e = 0;
  for (int w = w0; w < w1; ++w) e += (uint32_t)__popc(eqmap[w]);
  const uint32_t e_first = block_excl_scan(e, wsum[0]);
  uint32_t cnt = 0, er = e_first;
  for (int w = w0; w < w1; ++w) {
    const uint32_t x = eqmap[w];
    cnt += (uint32_t)__popc(selmap[w] | take_equal(x, er, rem));
    er += (uint32_t)__popc(x);
  }
  uint32_t slot = block_excl_scan(cnt, wsum[1]);
  er = e_first;
  for (int w = w0; w < w1; ++w) {
    const uint32_t x = eqmap[w];
    uint32_t m = selmap[w] | take_equal(x, er, rem);
    er += (uint32_t)__popc(x);
    while (m) {
      const int bit = __ffs(m) - 1;
      if (slot < (uint32_t)K) out[slot] = (int32_t)(ks + 32 * (int64_t)w + bit);
      ++slot;
      m &= m - 1u;
    }
  }
}

// ----------------------------------------------------------------- split rows
constexpr int SP_THREADS = 256;
constexpr int SP_PER = 8;                         // keys per thread
constexpr int SP_CHUNK = SP_THREADS * SP_PER;     // keys per workgroup
constexpr int SP_BINS = 2048;
constexpr int64_t SP_MIN_KEYS = 8192;             // shorter rows stay on one workgroup (one launch)
constexpr int64_t SP_MAX_ROWS = 512;              // more rows fill the chip by themselves

__host__ __device__ constexpr int sp_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__host__ __device__ constexpr uint32_t sp_mask(int pass) { return pass < 2 ? 2047u : 1023u; }

int64_t split_chunks(int64_t rows, int64_t s_cap) {
  if (rows >= SP_MAX_ROWS || s_cap <= SP_MIN_KEYS) return 0;
  return (s_cap + SP_CHUNK - 1) / SP_CHUNK;
}

struct SplitArgs {
  uint32_t* hist;  // [rows][3][SP_BINS]
  uint32_t* cnt;   // [rows][nchunk][2]: keys > tau, keys == tau
  int64_t nchunk;
};

// Finds, in the summed histogram gh of one digit, the digit value d that holds the
// rem-th largest candidate and the rank of that candidate among the keys with digit
// d.  Thread t owns bins 8t..8t+7; suffix sums over threads locate the owner.
__device__ void sp_scan(const uint32_t (&h)[8], uint32_t& rem, uint32_t& digit, uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) c += h[i];
  uint32_t x = c;  // suffix sum inside the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_down(x, off, 64);
    if (lane + off < 64) x += v;
  }
  if (lane == 0) sh[wave] = x;
  __syncthreads();
  for (int w = wave + 1; w < SP_THREADS / 64; ++w) x += sh[w];
  // x = candidates with digit >= 8*tid; exactly one thread has x >= rem > x - c
  if (x >= rem && x - c < rem) {
    uint32_t above = x - c;
    int i = 7;
    for (; i > 0; --i) {
      if (above + h[i] >= rem) break;
      above += h[i];
    }
    sh[4] = (uint32_t)(8 * tid + i);
    sh[5] = rem - above;
  }
  __syncthreads();
  digit = sh[4];
  rem = sh[5];
  __syncthreads();
}

// prefix / mask of the digits fixed by the first PASSES finished histograms (the bins of
// every pass are loaded at once; the scans then run one after another)
template <int PASSES>
__device__ void sp_prefix(const uint32_t* gh, uint32_t K, uint32_t& prefix, uint32_t& pmask, uint32_t& rem,
                          uint32_t* sh) {
  prefix = 0;
  pmask = 0;
  rem = K;
  if constexpr (PASSES > 0) {
    uint32_t h[PASSES][8];
#pragma unroll
    for (int q = 0; q < PASSES; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) h[q][i] = gh[q * SP_BINS + 8 * threadIdx.x + i];
#pragma unroll
    for (int q = 0; q < PASSES; ++q) {
      uint32_t d;
      sp_scan(h[q], rem, d, sh);
      prefix |= d << sp_shift(q);
      pmask |= sp_mask(q) << sp_shift(q);
    }
  }
}



struct SpRow {
  int64_t ks, ke, lo, hi;
  bool masked, skip;
};

__device__ __forceinline__ SpRow sp_row(const TopkParams& p) {
  SpRow r;
  clamp_range(p.key_start, p.key_end, blockIdx.y, p.s_cap, r.ks, r.ke);
  r.lo = r.ks + (int64_t)blockIdx.x * SP_CHUNK;
  r.hi = min(r.ke, r.lo + SP_CHUNK);
  r.masked = p.row_mask && !p.row_mask[blockIdx.y];
  r.skip = r.masked || (r.ke - r.ks <= p.topk) || r.lo >= r.ke;
  return r;
}

// the chunk's scores, SP_PER per thread (position lo + tid + SP_THREADS u), all loaded before
// any is used (one loop step per load waited for each in turn); `in` flags those inside it
__device__ __forceinline__ void sp_load(const float* src, const SpRow& r, float (&v)[SP_PER], bool (&in)[SP_PER]) {
#pragma unroll
  for (int u = 0; u < SP_PER; ++u) {
    const int64_t i = r.lo + threadIdx.x + (int64_t)u * SP_THREADS;
    in[u] = i < r.hi;
    v[u] = in[u] ? src[i] : 0.f;
  }
}

__global__ __launch_bounds__(256) void topk_split_clear(uint32_t* hist, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    hist[i] = 0u;
}

template <int PASS>
__global__ __launch_bounds__(SP_THREADS) void topk_split_hist(TopkParams p, SplitArgs a) {
  __shared__ uint32_t lh[SP_BINS];
  __shared__ uint32_t sh[8];
  const SpRow r = sp_row(p);
  if (r.skip) return;
  const int64_t row = blockIdx.y;
  uint32_t* gh = a.hist + row * 3 * SP_BINS;
  const float* src = p.scores + row * p.ld;
  float v[SP_PER];
  bool in[SP_PER];
  sp_load(src, r, v, in);
  uint32_t prefix, pmask, rem;
  sp_prefix<PASS>(gh, (uint32_t)p.topk, prefix, pmask, rem, sh);
  for (int i = threadIdx.x; i < SP_BINS; i += SP_THREADS) lh[i] = 0u;
  __syncthreads();
  constexpr int shift = sp_shift(PASS);
  constexpr uint32_t dmask = sp_mask(PASS);
#pragma unroll
  for (int u = 0; u < SP_PER; ++u) {
    const uint32_t key = order_key(v[u]);
    if (in[u] && (key & pmask) == prefix) atomicAdd(&lh[(key >> shift) & dmask], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < SP_BINS; i += SP_THREADS) {
    const uint32_t v = lh[i];
    if (v) atomicAdd(&gh[PASS * SP_BINS + i], v);
  }
}

__device__ __forceinline__ void sp_block_sum2(uint32_t& a, uint32_t& b, uint32_t* sh) {
  // inclusive block sums of (a, b); returns totals in a, b for every thread
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sh[wave] = a;
    sh[4 + wave] = b;
  }
  __syncthreads();
  a = sh[0] + sh[1] + sh[2] + sh[3];
  b = sh[4] + sh[5] + sh[6] + sh[7];
  __syncthreads();
}

__global__ __launch_bounds__(SP_THREADS) void topk_split_count(TopkParams p, SplitArgs a) {
  __shared__ uint32_t sh[8];
  const SpRow r = sp_row(p);
  if (r.skip) return;
  const int64_t row = blockIdx.y;
  const float* src = p.scores + row * p.ld;
  float v[SP_PER];
  bool in[SP_PER];
  sp_load(src, r, v, in);
  uint32_t tau, pmask, rem;
  sp_prefix<3>(a.hist + row * 3 * SP_BINS, (uint32_t)p.topk, tau, pmask, rem, sh);
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < SP_PER; ++u) {
    const uint32_t key = order_key(v[u]);
    gt += in[u] && key > tau;
    eq += in[u] && key == tau;
  }
  sp_block_sum2(gt, eq, sh);
  if (threadIdx.x == 0) {
    uint32_t* c = a.cnt + (row * a.nchunk + blockIdx.x) * 2;
    c[0] = gt;
    c[1] = eq;
  }
}

__global__ __launch_bounds__(SP_THREADS) void topk_split_emit(TopkParams p, SplitArgs a) {
  __shared__ uint32_t keys[SP_CHUNK + SP_CHUNK / SP_PER];  // one pad word per thread segment
  __shared__ uint32_t sh[8];
  __shared__ uint32_t scan_g[SP_THREADS / 64], scan_e[SP_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.y;
  const int K = p.topk;
  int32_t* out = p.out + row * (int64_t)K;
  SpRow r = sp_row(p);
  if (r.masked) return;
  if (r.ke - r.ks <= K) {
    if (blockIdx.x == 0)
      for (int i = tid; i < K; i += SP_THREADS) out[i] = (i < r.ke - r.ks) ? (int32_t)(r.ks + i) : -1;
    return;
  }
  if (r.skip) return;
  const float* src = p.scores + row * p.ld;
  float v[SP_PER];
  bool in[SP_PER];
  sp_load(src, r, v, in);
  uint32_t tau, pmask, rem;
  sp_prefix<3>(a.hist + row * 3 * SP_BINS, (uint32_t)K, tau, pmask, rem, sh);

  // keys > tau and == tau in the chunks before this one
  const uint32_t* c = a.cnt + row * a.nchunk * 2;
  uint32_t gtb = 0, eqb = 0;
  for (int64_t j = tid; j < (int64_t)blockIdx.x; j += SP_THREADS) {
    gtb += c[2 * j];
    eqb += c[2 * j + 1];
  }
  sp_block_sum2(gtb, eqb, sh);
  const uint32_t my_gt = c[2 * blockIdx.x], my_eq = c[2 * blockIdx.x + 1];
  if (my_gt == 0 && (my_eq == 0 || eqb >= rem)) return;  // nothing kept here (uniform)

  // stage the chunk's keys; thread t then walks positions lo + SP_PER t .. lo + SP_PER (t + 1) - 1
  const int len = (int)(r.hi - r.lo);
#pragma unroll
  for (int u = 0; u < SP_PER; ++u) {
    const int i = tid + u * SP_THREADS;
    if (in[u]) keys[i + i / SP_PER] = order_key(v[u]);
  }
  __syncthreads();
  const int i0 = tid * SP_PER, i1 = min(len, i0 + SP_PER);
  uint32_t g = 0, e = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i + i / SP_PER];
    g += key > tau;
    e += key == tau;
  }
  // exclusive prefix over threads
  uint32_t gi = g, ei = e;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t vg = __shfl_up(gi, off, 64), ve = __shfl_up(ei, off, 64);
    if (lane >= off) {
      gi += vg;
      ei += ve;
    }
  }
  if (lane == 63) {
    scan_g[wave] = gi;
    scan_e[wave] = ei;
  }
  __syncthreads();
  uint32_t gpos = gtb + gi - g, epos = eqb + ei - e;
  for (int w = 0; w < wave; ++w) {
    gpos += scan_g[w];
    epos += scan_e[w];
  }
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i + i / SP_PER];
    if (key > tau) {
      const uint32_t slot = gpos + min(epos, rem);
      if (slot < (uint32_t)K) out[slot] = (int32_t)(r.lo + i);
      ++gpos;
    } else if (key == tau) {
      if (epos < rem && gpos + epos < (uint32_t)K) out[gpos + epos] = (int32_t)(r.lo + i);
      ++epos;
    }
  }
}

size_t split_ws_bytes(int64_t rows, int64_t nchunk) {
  return (size_t)rows * 3 * SP_BINS * 4 + (size_t)rows * nchunk * 2 * 4;
}

}  // namespace

size_t topk_workspace_bytes(int B, int T, int, int64_t s_cap) {
  const int64_t rows = (int64_t)B * T;
  const int64_t nch = split_chunks(rows, s_cap);
  return nch ? split_ws_bytes(rows, nch) : 0;
}

hipError_t launch_topk(const TopkParams& p, void* ws, size_t ws_bytes, hipStream_t st, int* n_launches) {
  const int64_t rows = (int64_t)p.B * p.T;
  if (rows == 0) return hipSuccess;
  const int64_t nch = split_chunks(rows, p.s_cap);
  if (nch) {
    if (!ws || ws_bytes < split_ws_bytes(rows, nch)) return hipErrorInvalidValue;
    SplitArgs a{static_cast<uint32_t*>(ws), static_cast<uint32_t*>(ws) + rows * 3 * SP_BINS, nch};
    const int64_t words = rows * 3 * SP_BINS;
    hipLaunchKernelGGL(topk_split_clear, dim3((unsigned)std::min<int64_t>((words + 255) / 256, 1024)), dim3(256), 0, st,
                       a.hist, words);
    const dim3 grid((unsigned)nch, (unsigned)rows);
    hipLaunchKernelGGL(topk_split_hist<0>, grid, dim3(SP_THREADS), 0, st, p, a);
    hipLaunchKernelGGL(topk_split_hist<1>, grid, dim3(SP_THREADS), 0, st, p, a);
    hipLaunchKernelGGL(topk_split_hist<2>, grid, dim3(SP_THREADS), 0, st, p, a);
    hipLaunchKernelGGL(topk_split_count, grid, dim3(SP_THREADS), 0, st, p, a);
    hipLaunchKernelGGL(topk_split_emit, grid, dim3(SP_THREADS), 0, st, p, a);
    if (n_launches) *n_launches += 6;
    return hipGetLastError();
  }
  if (p.s_cap <= TK_CACHE_KEYS) {
    const size_t lds = (size_t)(p.s_cap > 0 ? p.s_cap : 1) * 4;
    static std::atomic<size_t> high{0};
    const hipError_t attr = allow_dynamic_lds(reinterpret_cast<const void*>(topk_rows<true>), lds, high);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(topk_rows<true>, dim3((unsigned)rows), dim3(TK_THREADS), lds, st, p);
  } else if (p.s_cap <= LG_MAX_KEYS) {
    const size_t lds = long_lds_bytes(p.s_cap);
    static std::atomic<size_t> high{0};
    const hipError_t attr = allow_dynamic_lds(reinterpret_cast<const void*>(topk_long), lds, high);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(topk_long, dim3((unsigned)rows), dim3(LG_THREADS), lds, st, p, (int)((p.s_cap + 31) / 32));
  } else {
    hipLaunchKernelGGL(topk_rows<false>, dim3((unsigned)rows), dim3(TK_THREADS), 0, st, p);
  }
  if (n_launches) ++*n_launches;
  return hipGetLastError();
}

}  // namespace dsa
