// Fused lightning indexer -> top-k for long rows on gfx950.
//
// The indexer scores every key of a query's prefix and the top-k keeps the index_topk
// best (GLM-5.2 IndexShare page, section 1; the DeepSeek-V3.2 material names the
// indexer and this selection as the long-context cost).  Written plainly, the whole
// [rows, s_cap] fp32 score matrix goes to HBM and is read back by the select.  Here it
// does not, in the common case:
//  1. sample pass: the indexer kernel scores only keys R*i (every R-th key);
//  2. threshold: per row, the order key of the r-th largest sample.  About R*r keys reach
//     it, with a spread of about R*sqrt(r); r = k/R + y with y^2 = 36 (k/R + y) puts the
//     mean six of those spreads above k (r = 89 for k = 2048, R = 64: ~5700 candidates);
//  3. candidate pass: the indexer kernel scores every key again and appends each cell
//     at or above the row's threshold, with its position, to the row's list (cap slots);
//  4. exact select over the list: when it holds c keys with k <= c <= cap it holds every
//     key at or above the row's k-th largest score (ties included), so the radix select
//     over it returns exactly what the full select returns; the kept positions are
//     sorted ascending.  Other rows (c < k: the samples misled the threshold; c > cap:
//     too many keys tie or crowd above it) are flagged;
//  5. fall-back for flagged rows only: the indexer kernel writes their full score rows
//     (row mask) and the plain top-k selects them.
// Every score is computed by the same kernel and arithmetic as the unfused path, so the
// indices are bit-identical to dsa_indexer_scores followed by dsa_topk_select.
#include "dsa_internal.h"
#include "select.h"

namespace dsa {
namespace {


struct FusedArgs {
  int64_t rows, s_cap;
  const int32_t* key_start;
  const int32_t* key_end;
  int K;                 // topk
  int64_t R;             // sample stride
  uint32_t rank;         // the threshold is the rank-th largest sample
  const float* samples;  // [rows, lds]
  int64_t lds;
  uint32_t* lkey;        // [rows] threshold (an order key)
  int32_t* live;         // [rows] 1: the row selects from its candidates (n > K)
  int32_t* fb;           // [rows] 1: the row falls back to the full score row
  int32_t* cnt;          // [rows] candidates appended (may exceed cap)
  const int32_t* pos;    // [rows, cap]
  const float* val;      // [rows, cap]
  int cap;
  int32_t* out;          // [rows, K]
};

// The rem-th largest of n values v_at(i) (those with pred: v_at returns false for the others),
// all below 2^bits: radix passes over digits of at most 11 bits from bit `bits` down (none
// when bits == 0: every value is 0).  *rem_out receives the value's rank among the values
// equal to it, *eq_count (if given) how many values equal it.  NT threads.
template <int NT, class VAt>
__device__ uint32_t radix_kth(VAt v_at, int n, uint32_t rem, int bits, uint32_t* hist, uint32_t* sh,
                              uint32_t* rem_out, uint32_t* eq_count) {
  const int tid = threadIdx.x, wave = tid >> 6;
  uint32_t prefix = 0, pmask = 0, eq = (uint32_t)n;
#pragma unroll 1
  for (int top = bits; top > 0; top -= 11) {
    const int shift = top > 11 ? top - 11 : 0;
    const uint32_t dmask = (1u << (top - shift)) - 1u;
    for (int i = tid; i < 2048; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      uint32_t v;
      if (v_at(i, v) && (v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) hist_find(hist, rem, &sh[0], &sh[1]);
    __syncthreads();
    prefix |= sh[0] << shift;
    pmask |= dmask << shift;
    rem = sh[1];
    eq = hist[sh[0]];
    __syncthreads();
  }
  *rem_out = rem;
  if (eq_count) *eq_count = eq;
  return prefix;
}

__device__ __forceinline__ int bit_length(uint32_t x) { return x ? 32 - __clz((int)x) : 0; }

// One workgroup per row: the threshold from the row's samples (staged in LDS); clears the
// candidate count.
constexpr int TH_THREADS = 256;
constexpr int TH_STAGE = 2048;  // samples staged in LDS (longer sample rows are read from L2)
__global__ __launch_bounds__(TH_THREADS) void fused_threshold(FusedArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sk[TH_STAGE];
  __shared__ uint32_t sh[2];
  const int64_t row = blockIdx.x;
  int64_t ks, ke;
  clamp_range(a.key_start, a.key_end, row, a.s_cap, ks, ke);
  const bool select = ke - ks > a.K;
  if (threadIdx.x == 0) {
    a.cnt[row] = 0;
    a.live[row] = select ? 1 : 0;
    a.lkey[row] = 0u;
  }
  if (!select) return;
  // samples of the row: columns c with key R c in [ks, ke)
  const int64_t c0 = (ks + a.R - 1) / a.R, c1 = (ke + a.R - 1) / a.R;
  const int m = (int)(c1 - c0);
  if (m < (int)a.rank) return;  // too few samples: every key is a candidate
  const float* src = a.samples + row * a.lds + c0;
  uint32_t rem, th;
  if (m <= TH_STAGE) {
    for (int i0 = 0; i0 < m; i0 += 8 * TH_THREADS) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * TH_THREADS + (int)threadIdx.x;
        v[u] = i < m ? src[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * TH_THREADS + (int)threadIdx.x;
        if (i < m) sk[i] = order_key(v[u]);
      }
    }
    __syncthreads();
    th = radix_kth<TH_THREADS>(
        [&](int i, uint32_t& v) {
          v = sk[i];
          return true;
        },
        m, a.rank, 32, hist, sh, &rem, nullptr);
  } else {
    th = radix_kth<TH_THREADS>(
        [&](int i, uint32_t& v) {
          v = order_key(src[i]);
          return true;
        },
        m, a.rank, 32, hist, sh, &rem, nullptr);
  }
  if (threadIdx.x == 0) a.lkey[row] = th;
}

constexpr int FU_SORT = 4096;     // largest topk of the fused path
constexpr int FS_THREADS = 512;
constexpr int FS_MAP_KEYS = 131072;  // rows up to this long are emitted through a bitmap of their range

// One workgroup per row: exact top-k over the row's candidate list, or the fall-back flag.
// The list's keys are held in LDS as offsets above the row's threshold (every candidate's key
// is >= it), so the radix digits start at the top bit the offsets use and the first pass
// spreads over its bins instead of piling into the few that the top bits of close keys share.
// The kept positions are written in ascending order from a bitmap of the row's range (rows
// up to FS_MAP_KEYS keys) or after a bitonic sort.
// Dynamic LDS: cap words of offsets, then FS_MAP_KEYS / 32 words (bitmap or sort buffer).
__global__ __launch_bounds__(FS_THREADS) void fused_select(FusedArgs a) {
  extern __shared__ uint32_t dyn[];
  uint32_t* dk = dyn;                   // [cap]: key - threshold of each candidate
  uint32_t* map = dyn + a.cap;          // [FS_MAP_KEYS / 32] bitmap of kept positions, or
  int32_t* sel = reinterpret_cast<int32_t*>(map);  // [FU_SORT] kept positions to sort
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wsum[FS_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  int64_t ks, ke;
  clamp_range(a.key_start, a.key_end, row, a.s_cap, ks, ke);
  const int64_t n = ke - ks;
  const int K = a.K;
  int32_t* out = a.out + row * (int64_t)K;
  if (n <= K) {
    for (int i = tid; i < K; i += FS_THREADS) out[i] = (i < n) ? (int32_t)(ks + i) : -1;
    if (tid == 0) a.fb[row] = 0;
    return;
  }
  const int32_t c = a.cnt[row];
  if (c < K || c > a.cap) {
    if (tid == 0) a.fb[row] = 1;
    return;
  }
  if (tid == 0) a.fb[row] = 0;
  const float* val = a.val + row * a.cap;
  const int32_t* pos = a.pos + row * a.cap;
  const uint32_t lk = a.lkey[row];
  const bool use_map = n <= FS_MAP_KEYS;
  const int W = (int)((n + 31) >> 5);
  if (use_map)
    for (int w = tid; w < W; w += FS_THREADS) map[w] = 0u;

  uint32_t mx = 0;
  for (int i0 = 0; i0 < c; i0 += 8 * FS_THREADS) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * FS_THREADS + tid;
      v[u] = i < c ? val[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * FS_THREADS + tid;
      if (i < c) {
        const uint32_t d = order_key(v[u]) - lk;
        dk[i] = d;
        mx = max(mx, d);
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
  if (lane == 0) wsum[wave] = mx;
  __syncthreads();
  mx = 0;
#pragma unroll
  for (int w = 0; w < FS_THREADS / 64; ++w) mx = max(mx, wsum[w]);

  // the K-th largest offset tau among the c candidates; rem of those equal to it are kept
  uint32_t rem, eq;
  const uint32_t tau = radix_kth<FS_THREADS>(
      [&](int i, uint32_t& v) {
        v = dk[i];
        return true;
      },
      c, (uint32_t)K, bit_length(mx), hist, sh, &rem, &eq);
  // with more candidates equal to tau than kept, the kept ones are the rem lowest positions:
  // the rem-th largest of (ke - 1 - position) among them bounds them
  uint32_t pmax = 0xffffffffu;
  if (eq > rem) {
    uint32_t r2;
    const uint32_t far = radix_kth<FS_THREADS>(
        [&](int i, uint32_t& v) {
          v = (uint32_t)(ke - 1 - pos[i]);
          return dk[i] == tau;
        },
        c, rem, bit_length((uint32_t)(n - 1)), hist, sh, &r2, nullptr);
    pmax = (uint32_t)(ke - 1) - far;
  }

  // kept: offsets > tau, and offsets == tau at positions <= pmax
  if (tid == 0) sh[2] = 0;
  __syncthreads();
  for (int i0 = 0; i0 < c; i0 += 8 * FS_THREADS) {
    bool cand[8];
    int32_t ps[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * FS_THREADS + tid;
      cand[u] = i < c && dk[i] >= tau;
      ps[u] = cand[u] ? pos[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * FS_THREADS + tid;
      const bool take = cand[u] && (dk[i] > tau || (uint32_t)ps[u] <= pmax);
      if (use_map) {
        if (take) {
          const uint32_t o = (uint32_t)(ps[u] - ks);
          atomicOr(&map[o >> 5], 1u << (o & 31));
        }
      } else {
        const uint64_t m = __ballot(take);
        uint32_t base = 0;
        if (lane == 0 && m) base = atomicAdd(&sh[2], (uint32_t)__popcll(m));
        base = __shfl(base, 0, 64);
        if (take) {
          const uint32_t slot = base + lane_prefix(m, lane);
          if (slot < (uint32_t)K) sel[slot] = ps[u];
        }
      }
    }
  }
  __syncthreads();
  if (use_map) {
    // thread t owns words [t wpt, (t + 1) wpt) of the bitmap; kept positions in order
    const int wpt = (W + FS_THREADS - 1) / FS_THREADS;
    const int w0 = min(W, tid * wpt), w1 = min(W, w0 + wpt);
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += (uint32_t)__popc(map[w]);
    uint32_t slot = block_excl_scan(cnt, wsum);
    for (int w = w0; w < w1; ++w) {
      uint32_t x = map[w];
      while (x) {
        const int bit = __ffs(x) - 1;
        if (slot < (uint32_t)K) out[slot] = (int32_t)(ks + 32 * (int64_t)w + bit);
        ++slot;
        x &= x - 1u;
      }
    }
    return;
  }
  // pad to a power of two with positions past every key, then a bitonic sort (ascending)
  int P = 1;
  while (P < K) P <<= 1;
  for (int i = K + tid; i < P; i += FS_THREADS) sel[i] = INT32_MAX;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += FS_THREADS) {
        const int lo = 2 * t - (t & (stride - 1)), hi = lo + stride;
        const int32_t x = sel[lo], y = sel[hi];
        const bool up = (lo & size) == 0;
        if ((x > y) == up) {
          sel[lo] = y;
          sel[hi] = x;
        }
      }
      __syncthreads();
    }
  for (int i = tid; i < K; i += FS_THREADS) out[i] = sel[i];
}

constexpr int64_t FU_CAP = 12288;         // candidate slots per row (about 11 spreads above the mean)
constexpr int64_t FU_MIN_STRIDE = 16;     // the sample buffer is sized for this stride
constexpr int64_t FU_DEFAULT_STRIDE = 64;

size_t al(size_t x) { return (x + 255) / 256 * 256; }

struct Layout {
  size_t scores, topk_ws, samples, lkey, live, fb, cnt, pos, val, vec, end;
};

Layout layout(int B, int T, int topk, int64_t s_cap, size_t vec_bytes) {
  const size_t rows = (size_t)B * T;
  Layout L;
  L.scores = 0;
  L.topk_ws = al(rows * (size_t)s_cap * 4);
  L.samples = L.topk_ws + al(topk_workspace_bytes(B, T, topk, s_cap));
  L.lkey = L.samples + al(rows * (size_t)((s_cap + FU_MIN_STRIDE - 1) / FU_MIN_STRIDE) * 4);
  L.live = L.lkey + al(rows * 4);
  L.fb = L.live + al(rows * 4);
  L.cnt = L.fb + al(rows * 4);
  L.pos = L.cnt + al(rows * 4);
  L.val = L.pos + al(rows * (size_t)FU_CAP * 4);
  L.vec = L.val + al(rows * (size_t)FU_CAP * 4);
  L.end = L.vec + al(vec_bytes);
  return L;
}

}  // namespace

int64_t indexer_topk_stride(int64_t requested) { return requested == 0 ? FU_DEFAULT_STRIDE : requested; }
bool indexer_topk_stride_ok(int64_t stride) { return stride == 0 || (stride >= FU_MIN_STRIDE && stride <= (1 << 20)); }

bool indexer_topk_fused(const IndexerParams& p, Dtype dt, int topk) {
  if (topk < 1 || topk > FU_SORT || (int64_t)p.B * p.T > INT32_MAX) return false;
  IndexerParams ps = p;
  ps.kstride = FU_MIN_STRIDE;
  return indexer_modes_supported(p, dt) && indexer_modes_supported(ps, dt);
}

size_t indexer_topk_workspace_bytes(int B, int T, int topk, int64_t s_cap, bool fused, size_t vec_bytes) {
  const Layout L = layout(B, T, topk, s_cap, vec_bytes);
  return fused ? L.end : L.samples;
}

hipError_t launch_indexer_topk(const IndexerParams& p, Dtype dt, int topk, int64_t stride, int32_t* out, void* ws,
                               size_t ws_bytes, hipStream_t st, int* n_launches) {
  const int64_t rows = (int64_t)p.B * p.T;
  if (rows == 0) return hipSuccess;
  const bool fused = indexer_topk_fused(p, dt, topk) && p.s_cap > 0;
  const size_t vec_bytes = fused ? indexer_vectors_bytes(p.B, p.T, p.H, p.D, p.Hk, p.s_cap, dt) : 0;
  const Layout L = layout(p.B, p.T, topk, p.s_cap, vec_bytes);
  const size_t need = fused ? L.end : L.samples;
  if (ws_bytes < need || (need && !ws)) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + L.scores);
  void* tws = base + L.topk_ws;
  const size_t tws_bytes = L.samples - L.topk_ws;
  TopkParams tp{p.B, p.T, topk, p.s_cap, p.key_start, p.key_end, scores, p.s_cap, out};
  hipError_t e;
  if (!fused) {
    IndexerParams pf = p;
    pf.scores = scores;
    pf.ld = p.s_cap;
    if ((e = launch_indexer(pf, dt, st, n_launches)) != hipSuccess) return e;
    return launch_topk(tp, tws, tws_bytes, st, n_launches);
  }
  const int64_t R = indexer_topk_stride(stride);
  const double kr = (double)topk / (double)R;
  const double y = 0.5 * (36.0 + std::sqrt(36.0 * 36.0 + 4.0 * 36.0 * kr));
  FusedArgs a;
  a.rows = rows;
  a.s_cap = p.s_cap;
  a.key_start = p.key_start;
  a.key_end = p.key_end;
  a.K = topk;
  a.R = R;
  a.rank = (uint32_t)std::ceil(kr + y);
  a.samples = reinterpret_cast<const float*>(base + L.samples);
  a.lds = (p.s_cap + R - 1) / R;
  a.lkey = reinterpret_cast<uint32_t*>(base + L.lkey);
  a.live = reinterpret_cast<int32_t*>(base + L.live);
  a.fb = reinterpret_cast<int32_t*>(base + L.fb);
  a.cnt = reinterpret_cast<int32_t*>(base + L.cnt);
  a.pos = reinterpret_cast<const int32_t*>(base + L.pos);
  a.val = reinterpret_cast<const float*>(base + L.val);
  a.cap = (int)FU_CAP;
  a.out = out;

  // 1. samples
  IndexerParams ps = p;
  ps.kstride = R;
  ps.scores = const_cast<float*>(a.samples);
  ps.ld = a.lds;
  if ((e = launch_indexer(ps, dt, st, n_launches)) != hipSuccess) return e;
  // 2. thresholds (and cleared counts)
  hipLaunchKernelGGL(fused_threshold, dim3((unsigned)rows), dim3(TH_THREADS), 0, st, a);
  if (n_launches) ++*n_launches;
  // 3. candidates (head-major vectors first, where the kernel takes them)
  IndexerParams pv = p;
  if ((e = launch_indexer_vectors(pv, dt, vec_bytes ? base + L.vec : nullptr, st, n_launches)) != hipSuccess) return e;
  IndexerParams pc = pv;
  pc.scores = nullptr;
  pc.ld = 0;
  pc.row_mask = a.live;
  pc.lkey = a.lkey;
  pc.cand_cnt = a.cnt;
  pc.cand_pos = const_cast<int32_t*>(a.pos);
  pc.cand_val = const_cast<float*>(a.val);
  pc.cap = a.cap;
  if ((e = launch_indexer(pc, dt, st, n_launches)) != hipSuccess) return e;
  // 4. exact select over the candidates, fall-back flags
  {
    static std::atomic<size_t> high{0};
    static_assert(FS_MAP_KEYS / 32 >= FU_SORT, "the sort buffer shares the bitmap's words");
    const size_t lds = (size_t)(FU_CAP + FS_MAP_KEYS / 32) * 4;
    if ((e = allow_dynamic_lds(reinterpret_cast<const void*>(&fused_select), lds, high)) != hipSuccess) return e;
    hipLaunchKernelGGL(fused_select, dim3((unsigned)rows), dim3(FS_THREADS), lds, st, a);
  }
  if (n_launches) ++*n_launches;
  // 5. fall-back rows: full score rows, plain select
  IndexerParams pf = pv;
  pf.scores = scores;
  pf.ld = p.s_cap;
  pf.row_mask = a.fb;
  pf.few_rows = 1;
  if ((e = launch_indexer(pf, dt, st, n_launches)) != hipSuccess) return e;
  tp.row_mask = a.fb;
  return launch_topk(tp, tws, tws_bytes, st, n_launches);
}

}  // namespace dsa
