// Index-score backward on the matrix cores, for selections that cover a large share of
// each row's key range (a prefill whose index_topk is comparable to the prefix).
//
// The gradients are those of indexer_bwd.hip (GLM-5.2 IndexShare page, section 1 score,
// ReLU derivative 0 at 0):
//   dw[t,h] = sum_j DI[t,j] max(0, s),   dq[t,h] = sum_j DI[t,j] w[t,h] [s > 0] k~[j,g(h)],
//   dk[j,g] = sum_{t,h: g(h) = g} DI[t,j] w[t,h] [s > 0] q~[t,h],   s = q~[t,h] . k~[j,g(h)],
// where DI[t,j] is the sum of dI over the slots of row t that name key j.  Here DI is
// scattered into a dense [row][key] fp32 matrix in the workspace (with a byte per 64 x 64
// block that holds any selection), and the sums over keys and over queries become tile
// products on v_mfma_f32_32x32x16_bf16:
//   id_dq  per (128 queries, head): for each occupied 64-key tile, S^T = K Q^T, then
//          G^T = DI w [S > 0] (times the key scale for fp8) and dq^T += K^T G^T; dw from
//          the same S on the vector ALU;
//   id_dk  per (64 keys, key head): for each occupied 64-query tile (and each query head of
//          the key head), S = Q K^T, G = DI w [S > 0] (times the query scale for fp8),
//          dk^T += Q^T G.
// Every output row is written once (zero where nothing is selected): no atomics, no clear
// of dk.  The inputs (bf16, or e4m3 codes, which bf16 holds exactly) give exact products
// with fp32 sums; G enters the second product as two bf16 terms (G = hi + lo, |G - hi -
// lo| <= 2^-17 |G|), so dq and dk carry fp32-level rounding.  K and Q tiles go to LDS
// twice: row-major (rows of 128 dims, 16-byte chunks XOR-swizzled by row) for the S
// products and transposed (a row per dim, 8-byte units of 4 rows swizzled by dim) for the
// second products, whose contraction runs over the tile's rows in the order a 32 x 32
// accumulator holds them (rows 8 (i / 4) + 4 lg + i % 4 for lane group lg, i = 0..15).
#include "dsa_internal.h"
#include "mla_tile.h"

namespace dsa {
namespace {
using mla::bf16x8;
using mla::f32x16;
using mla::i32x4;
using mla::pack_bf16x2;

constexpr int ID_D = 128;                  // index head dim
constexpr int ID_T = 64;                   // rows of a tile (keys or queries) and of an occupancy block
constexpr int ID_ROWB = ID_D * 2;          // bytes of a bf16 row
constexpr int ID_R = ID_T * ID_ROWB;       // row-major tile: 16 KiB
constexpr int ID_BUF = 2 * ID_R;           // + transposed copy
constexpr int ID_MAXT = 4096;              // tiles along either axis (list length)
constexpr int ID_DQ_Q = 128;               // queries per id_dq workgroup (4 waves x 32)

struct DenseWs {
  float* DI;        // [B*T][ldi]
  uint8_t* occ;     // [B][nqt][nkt]
  int64_t ldi;
  int nqt, nkt;
};

int64_t id_ldi(int64_t s_cap) { return (s_cap + ID_T - 1) / ID_T * ID_T; }
size_t id_al(size_t x) { return (x + 255) / 256 * 256; }

// four e4m3 codes (OCP e4m3fn) -> four bf16 (exact: bf16 holds every e4m3 value)
__device__ __forceinline__ uint2 id_fp8x4(uint32_t w) {
  const mla::f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const mla::f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]));
}

// ---------------------------------------------------------------- staging of one 64-row tile
// Thread tid stages rows 4 (tid / 16) + m (m = 0..3), dims 8 (tid % 16) .. +8.
template <int DT>
__device__ __forceinline__ void id_load(const unsigned char* base, int64_t row_bytes, int64_t row0, int64_t nvalid,
                                        uint4 (&v)[4]) {
  const int tid = threadIdx.x, kq = tid >> 4, dc = tid & 15;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t r = min<int64_t>(row0 + 4 * kq + m, nvalid - 1);  // rows past the end load a valid row
    if constexpr (DT == BF16) {
      v[m] = *reinterpret_cast<const uint4*>(base + r * row_bytes + 16 * dc);
    } else {
      const uint2 c = *reinterpret_cast<const uint2*>(base + r * row_bytes + 8 * dc);
      v[m] = make_uint4(c.x, c.y, 0u, 0u);  // raw codes: converted by id_store, after the tile's math
    }
  }
}
template <int DT>
__device__ __forceinline__ void id_store(unsigned char* buf, uint4 (&v)[4]) {
  const int tid = threadIdx.x, kq = tid >> 4, dc = tid & 15;
  if constexpr (DT == FP8) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint2 lo = id_fp8x4(v[m].x), hi = id_fp8x4(v[m].y);
      v[m] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = 4 * kq + m;
    *reinterpret_cast<uint4*>(buf + r * ID_ROWB + 16 * (dc ^ (r & 15))) = v[m];
  }
  unsigned char* xt = buf + ID_R;
  const uint32_t w[4][4] = {{v[0].x, v[0].y, v[0].z, v[0].w}, {v[1].x, v[1].y, v[1].z, v[1].w},
                            {v[2].x, v[2].y, v[2].z, v[2].w}, {v[3].x, v[3].y, v[3].z, v[3].w}};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * dc + e;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of two words
    const uint32_t lo = __builtin_amdgcn_perm(w[1][e >> 1], w[0][e >> 1], sel);
    const uint32_t hi = __builtin_amdgcn_perm(w[3][e >> 1], w[2][e >> 1], sel);
    *reinterpret_cast<uint2*>(xt + d * (ID_T * 2) + 8 * (kq ^ (d & 15))) = make_uint2(lo, hi);
  }
}
// 8 dims (16-byte chunk c) of row r of a row-major tile
__device__ __forceinline__ bf16x8 id_row(const unsigned char* buf, int r, int c) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(buf + r * ID_ROWB + 16 * (c ^ (r & 15))));
}
// rows 16 ks + {4 lg .. +3, 8 + 4 lg .. +3} of dim d, from the transposed copy
__device__ __forceinline__ bf16x8 id_col(const unsigned char* buf, int d, int ks, int lg) {
  const unsigned char* xt = buf + ID_R + d * (ID_T * 2);
  const uint2 a = *reinterpret_cast<const uint2*>(xt + 8 * ((4 * ks + lg) ^ (d & 15)));
  const uint2 b = *reinterpret_cast<const uint2*>(xt + 8 * ((4 * ks + 2 + lg) ^ (d & 15)));
  const i32x4 v = {(int)a.x, (int)a.y, (int)b.x, (int)b.y};
  return __builtin_bit_cast(bf16x8, v);
}
// 8 dims of a global row as a bf16 fragment
template <int DT>
__device__ __forceinline__ bf16x8 id_frag(const unsigned char* row, int d0) {
  if constexpr (DT == BF16) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(row + 2 * d0));
  } else {
    const uint2 c = *reinterpret_cast<const uint2*>(row + d0);
    const uint2 lo = id_fp8x4(c.x), hi = id_fp8x4(c.y);
    const i32x4 o = {(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
    return __builtin_bit_cast(bf16x8, o);
  }
}
// G as two bf16 fragments (hi + lo) from accumulator registers [8c, 8c + 8)
__device__ __forceinline__ void id_split(const float (&g)[8], bf16x8& hi, bf16x8& lo) {
  i32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p = pack_bf16x2(g[2 * i], g[2 * i + 1]);
    h[i] = (int)p;
    l[i] = (int)pack_bf16x2(g[2 * i] - __uint_as_float(p << 16), g[2 * i + 1] - __uint_as_float(p & 0xffff0000u));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// The occupied blocks of one row (or column) of the occupancy map, in order, into list[];
// returns their number.  Wave 0 scans 64 entries per step.
__device__ int id_list(const uint8_t* occ, int64_t stride, int n, const uint8_t* occ2, uint16_t* list, int* cnt) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int c = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const bool on = i < n && (occ[(int64_t)i * stride] || (occ2 && occ2[(int64_t)i * stride]));
      const uint64_t m = __ballot(on);
      if (on) list[c + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = (uint16_t)i;
      c += __popcll(m);
    }
    if (lane == 0) *cnt = c;
  }
  __syncthreads();
  const int c = *cnt;
  __syncthreads();
  return c;
}

// ---------------------------------------------------------------- clear and scatter
__global__ __launch_bounds__(256) void id_clear(float* x, int64_t n, uint8_t* occ, int64_t nocc) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) x[i] = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nocc; i += stride) occ[i] = 0;
}

// one workgroup per query row
__global__ __launch_bounds__(256) void id_scatter(IndexBwdParams p, DenseWs ws) {
  const int64_t row = blockIdx.x;
  const int64_t b = row / p.T, t = row % p.T;
  const int32_t* idx = p.idx + row * p.topk;
  const float* dI = p.dI + row * p.topk;
  float* di = ws.DI + row * ws.ldi;
  uint8_t* oc = ws.occ + (b * ws.nqt + t / ID_T) * ws.nkt;
  for (int j = threadIdx.x; j < p.topk; j += 256) {
    const int32_t e = idx[j];
    if (e < 0 || (int64_t)e >= p.s_cap) continue;
    atomicAdd(di + e, dI[j]);
    oc[e / ID_T] = 1;
  }
}

// ---------------------------------------------------------------- dq, dw
// grid (ceil(T / 128), H, B); wave w owns queries 32 w .. +32 of the workgroup's 128.
constexpr int ID_DQ_LDS = 2 * ID_BUF + 2 * ID_T * 4 + ID_MAXT * 2 + 16;

template <int DT>
__global__ __launch_bounds__(256, 2) void id_dq(IndexBwdParams p, DenseWs ws) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* ksv = reinterpret_cast<float*>(smem + 2 * ID_BUF);            // [2][64] key scales
  uint16_t* list = reinterpret_cast<uint16_t*>(smem + 2 * ID_BUF + 2 * ID_T * 4);
  int* cnt = reinterpret_cast<int*>(smem + 2 * ID_BUF + 2 * ID_T * 4 + ID_MAXT * 2);
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const int qx = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = p.H, T = p.T, g = (p.Hk == H) ? h : 0;
  const int64_t S = p.s_cap;
  constexpr int ESZ = DT == BF16 ? 2 : 1;
  const int64_t qrow_bytes = (int64_t)H * ID_D * ESZ, krow_bytes = (int64_t)p.Hk * ID_D * ESZ;
  const unsigned char* kbase = static_cast<const unsigned char*>(p.k) + ((int64_t)b * S * p.Hk + g) * ID_D * ESZ;

  // occupied key tiles of this workgroup's two 64-query blocks
  const int qb0 = 2 * qx;
  const uint8_t* o1 = ws.occ + ((int64_t)b * ws.nqt + qb0) * ws.nkt;
  const uint8_t* o2 = qb0 + 1 < ws.nqt ? o1 + ws.nkt : nullptr;
  const int n = id_list(o1, 1, ws.nkt, o2, list, cnt);

  // this lane's query (clamped for loads), its S^T B fragments, weight and scale
  const int t = ID_DQ_Q * qx + 32 * wv + lr;
  const int tc = min(t, T - 1);
  const int64_t qrow = (int64_t)b * T + tc;
  bf16x8 qf[8];
  {
    const unsigned char* qp = static_cast<const unsigned char*>(p.q) + qrow * qrow_bytes + (int64_t)h * ID_D * ESZ;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = id_frag<DT>(qp, 16 * ks + 8 * lg);
  }
  const float wt = p.w[qrow * H + h];
  const float qs = DT == FP8 ? p.q_scale[qrow * H + h] : 1.f;
  const float* dirow = ws.DI + ((int64_t)b * T + tc) * ws.ldi;
  const bool tin = t < T;

  f32x16 dq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[j][r] = 0.f;
  float dwacc = 0.f;

  uint4 st[4];
  float ksn = 1.f;
  auto fetch = [&](int i) {
    const int64_t j0 = (int64_t)list[i] * ID_T;
    id_load<DT>(kbase, krow_bytes, j0, S, st);
    if (DT == FP8 && tid < ID_T) ksn = p.k_scale[(((int64_t)b * S + min<int64_t>(j0 + tid, S - 1)) * p.Hk) + g];
  };
  auto put = [&](int i) {
    id_store<DT>(smem + (i & 1) * ID_BUF, st);
    if (DT == FP8 && tid < ID_T) ksv[(i & 1) * ID_T + tid] = ksn;
  };
  if (n > 0) {
    fetch(0);
    put(0);
  }
  __syncthreads();
  for (int i = 0; i < n; ++i) {
    const unsigned char* buf = smem + (i & 1) * ID_BUF;
    const int64_t j0 = (int64_t)list[i] * ID_T;
    const float* kv = ksv + (i & 1) * ID_T;
    // DI of this lane's query at key rows 32 kb + 8 q + 4 lg + (0..3), issued before the next
    // tile's loads so that using it does not wait for them (loads complete in issue order)
    float4 dib[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dib[kb][q] = tin ? *reinterpret_cast<const float4*>(dirow + j0 + 32 * kb + 8 * q + 4 * lg) : make_float4(0.f, 0.f, 0.f, 0.f);
    if (i + 1 < n) fetch(i + 1);
    // one 32-key half at a time: S^T = K Q^T (keys 32 kb + rows, this wave's 32 queries as
    // columns), G^T and dw, then dq^T += K^T G^T over its two 16-key steps
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float4 (&di)[4] = dib[kb];
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(id_row(buf, 32 * kb + lr, 2 * ks + lg), qf[ks], s, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float gv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * c + e, q = r >> 2;
          const float d = (&di[q].x)[r & 3];
          const float kk = DT == FP8 ? kv[32 * kb + 8 * q + 4 * lg + (r & 3)] : 1.f;
          const float a = s[r];
          dwacc = fmaf(d * kk, fmaxf(a, 0.f), dwacc);
          gv[e] = a > 0.f ? d * wt * kk : 0.f;
        }
        bf16x8 gh, gl;
        id_split(gv, gh, gl);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 a = id_col(buf, 32 * db + lr, 2 * kb + c, lg);
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gh, dq[db], 0, 0, 0);
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gl, dq[db], 0, 0, 0);
        }
      }
    }
    if (i + 1 < n) put(i + 1);
    __syncthreads();
  }
  // dw: the two lane groups hold different keys of the same query
  dwacc += __shfl_xor(dwacc, 32, 64);
  if (tin && lg == 0) p.dw[((int64_t)b * T + t) * H + h] = dwacc * qs;
  if (tin) {
    float* dqp = p.dq + (((int64_t)b * T + t) * H + h) * ID_D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dqp + 32 * db + 8 * q + 4 * lg) =
            make_float4(dq[db][4 * q], dq[db][4 * q + 1], dq[db][4 * q + 2], dq[db][4 * q + 3]);
  }
}

// ---------------------------------------------------------------- dk
// grid (nkt, Hk, B); wave w: keys 32 (w & 1) .. +32 of the tile, queries 32 (w >> 1) .. +32 of
// each 64-query tile; the two query halves meet in LDS at the end.
constexpr int ID_DK_LDS = 2 * ID_BUF + 4 * ID_T * 4 + ID_MAXT * 2 + 16;

template <int DT>
__global__ __launch_bounds__(256, 2) void id_dk(IndexBwdParams p, DenseWs ws) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* vec = reinterpret_cast<float*>(smem + 2 * ID_BUF);  // [2][w, w qs][64]
  uint16_t* list = reinterpret_cast<uint16_t*>(smem + 2 * ID_BUF + 4 * ID_T * 4);
  int* cnt = reinterpret_cast<int*>(smem + 2 * ID_BUF + 4 * ID_T * 4 + ID_MAXT * 2);
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5, kb = wv & 1, qh = wv >> 1;
  const int kx = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int H = p.H, T = p.T, Hk = p.Hk;
  const int64_t S = p.s_cap;
  constexpr int ESZ = DT == BF16 ? 2 : 1;
  const int64_t qrow_bytes = (int64_t)H * ID_D * ESZ;
  const int64_t j0 = (int64_t)kx * ID_T;

  // occupied 64-query tiles of this key tile
  const int n = id_list(ws.occ + (int64_t)b * ws.nqt * ws.nkt + kx, ws.nkt, ws.nqt, nullptr, list, cnt);
  const int nh = (Hk == H) ? 1 : H;  // query heads of this key head
  const int total = n * nh;

  // this lane's key: S = Q K^T B fragments
  const int64_t jc = min<int64_t>(j0 + 32 * kb + lr, S - 1);
  bf16x8 kf[8];
  {
    const unsigned char* kp = static_cast<const unsigned char*>(p.k) + (((int64_t)b * S + jc) * Hk + g) * ID_D * ESZ;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = id_frag<DT>(kp, 16 * ks + 8 * lg);
  }
  const int64_t jcol = j0 + 32 * kb + lr;  // DI column (zero past s_cap: padded)

  f32x16 dk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[j][r] = 0.f;

  uint4 st[4];
  float wn = 0.f, wqn = 0.f;
  auto fetch = [&](int i) {
    const int hh = (Hk == H) ? g : i / n;
    const int64_t t0 = (int64_t)list[i % n] * ID_T;
    const unsigned char* qb = static_cast<const unsigned char*>(p.q) + ((int64_t)b * T * H + hh) * ID_D * ESZ;
    id_load<DT>(qb, qrow_bytes, t0, T, st);
    if (tid < ID_T) {
      const int64_t r = (int64_t)b * T + min<int64_t>(t0 + tid, T - 1);
      wn = p.w[r * H + hh];
      wqn = DT == FP8 ? wn * p.q_scale[r * H + hh] : wn;
    }
  };
  auto put = [&](int i) {
    id_store<DT>(smem + (i & 1) * ID_BUF, st);
    if (tid < ID_T) {
      vec[(i & 1) * 2 * ID_T + tid] = wn;
      vec[(i & 1) * 2 * ID_T + ID_T + tid] = wqn;
    }
  };
  // DI at the accumulator's query rows 32 qh + 8 q + 4 lg + e of tile i, this lane's key
  // column: loaded one tile ahead and before that tile's query rows, so that using it never
  // waits for the newer loads (loads complete in issue order)
  float dn[16];
  auto fetch_di = [&](int i) {
    const int64_t t0 = (int64_t)list[i % n] * ID_T;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t t = t0 + 32 * qh + 8 * (r >> 2) + 4 * lg + (r & 3);
      const int64_t tc = t < T ? t : T - 1;
      const float dv = ws.DI[((int64_t)b * T + tc) * ws.ldi + jcol];
      dn[r] = t < T ? dv : 0.f;
    }
  };
  if (total > 0) {
    fetch_di(0);
    fetch(0);
    put(0);
  }
  __syncthreads();
  for (int i = 0; i < total; ++i) {
    float di[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) di[r] = dn[r];
    if (i + 1 < total) {
      fetch_di(i + 1);
      fetch(i + 1);
    }
    const unsigned char* buf = smem + (i & 1) * ID_BUF;
    // S = Q K^T: queries 32 qh + rows, this wave's 32 keys as columns
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(id_row(buf, 32 * qh + lr, 2 * ks + lg), kf[ks], s, 0, 0, 0);
    // G (times the query scale for fp8) as bf16 hi + lo per 16-query step
    const float* wq = vec + (i & 1) * 2 * ID_T + ID_T;
    bf16x8 gh[2], gl[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float gv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * c + e;
        const float wqr = wq[32 * qh + 8 * (r >> 2) + 4 * lg + (r & 3)];
        gv[e] = s[r] > 0.f ? di[r] * wqr : 0.f;
      }
      id_split(gv, gh[c], gl[c]);
    }
    // dk^T += Q^T G over this wave's 32 queries (2 steps of 16)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 a = id_col(buf, 32 * db + lr, 2 * qh + c, lg);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gh[c], dk[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gl[c], dk[db], 0, 0, 0);
      }
    if (i + 1 < total) put(i + 1);
    __syncthreads();
  }
  // the query halves meet: waves 2, 3 leave their sums in LDS, waves 0, 1 add and store
  float* red = reinterpret_cast<float*>(smem) + (kb * 64 + lane) * 64;
  if (qh == 1)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(red + 16 * db + 4 * q) = make_float4(dk[db][4 * q], dk[db][4 * q + 1], dk[db][4 * q + 2], dk[db][4 * q + 3]);
  __syncthreads();
  if (qh == 0 && jcol < S) {
    float* dkp = p.dk + (((int64_t)b * S + jcol) * Hk + g) * ID_D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 o = *reinterpret_cast<const float4*>(red + 16 * db + 4 * q);
        *reinterpret_cast<float4*>(dkp + 32 * db + 8 * q + 4 * lg) =
            make_float4(dk[db][4 * q] + o.x, dk[db][4 * q + 1] + o.y, dk[db][4 * q + 2] + o.z, dk[db][4 * q + 3] + o.w);
      }
  }
}

// one high-water mark per kernel (N: which kernel)
template <int N>
hipError_t id_allow(const void* f, int bytes) {
  static std::atomic<size_t> high{0};
  return allow_dynamic_lds(f, (size_t)bytes, high);
}

}  // namespace

bool index_bwd_dense(int B, int T, int H, int D, int Hk, int topk, int64_t s_cap, Dtype dt) {
  if (!(dt == BF16 || dt == FP8) || D != ID_D || H < 1 || H > 64 || !(Hk == H || Hk == 1)) return false;
  if (B < 1 || T < 1 || s_cap < 1 || topk < 1) return false;
  const int64_t nkt = (s_cap + ID_T - 1) / ID_T, nqt = ((int64_t)T + ID_T - 1) / ID_T;
  if (nkt > ID_MAXT || nqt > ID_MAXT || B > 65535) return false;
  if ((int64_t)B * T * id_ldi(s_cap) * 4 > (int64_t(1) << 32)) return false;
  return 8 * (int64_t)topk >= s_cap;  // the selection covers at least 1/8 of the key capacity
}

size_t index_bwd_workspace_bytes(int B, int T, int H, int D, int Hk, int topk, int64_t s_cap, Dtype dt) {
  if (!index_bwd_dense(B, T, H, D, Hk, topk, s_cap, dt)) return 0;
  const size_t nkt = (size_t)((s_cap + ID_T - 1) / ID_T), nqt = (size_t)((T + ID_T - 1) / ID_T);
  return id_al((size_t)B * T * id_ldi(s_cap) * 4) + id_al((size_t)B * nqt * nkt);
}

hipError_t launch_index_bwd_dense(const IndexBwdParams& p, Dtype dt, void* ws_ptr, size_t ws_bytes, hipStream_t st,
                                  int* n_launches) {
  if (ws_bytes < index_bwd_workspace_bytes(p.B, p.T, p.H, p.D, p.Hk, p.topk, p.s_cap, dt) || !ws_ptr)
    return hipErrorInvalidValue;
  DenseWs ws;
  ws.ldi = id_ldi(p.s_cap);
  ws.nkt = (int)((p.s_cap + ID_T - 1) / ID_T);
  ws.nqt = (p.T + ID_T - 1) / ID_T;
  ws.DI = static_cast<float*>(ws_ptr);
  ws.occ = static_cast<uint8_t*>(ws_ptr) + id_al((size_t)p.B * p.T * ws.ldi * 4);
  const int64_t rows = (int64_t)p.B * p.T;
  const int64_t ndi = rows * ws.ldi, nocc = (int64_t)p.B * ws.nqt * ws.nkt;
  hipLaunchKernelGGL(id_clear, dim3((unsigned)std::min<int64_t>((ndi + 255) / 256, 8192)), dim3(256), 0, st, ws.DI, ndi,
                     ws.occ, nocc);
  hipLaunchKernelGGL(id_scatter, dim3((unsigned)rows), dim3(256), 0, st, p, ws);
  hipError_t e;
  const dim3 gq((unsigned)((p.T + ID_DQ_Q - 1) / ID_DQ_Q), (unsigned)p.H, (unsigned)p.B);
  const dim3 gk((unsigned)ws.nkt, (unsigned)p.Hk, (unsigned)p.B);
  if (dt == BF16) {
    if ((e = id_allow<0>(reinterpret_cast<const void*>(id_dq<BF16>), ID_DQ_LDS)) != hipSuccess) return e;
    hipLaunchKernelGGL(id_dq<BF16>, gq, dim3(256), ID_DQ_LDS, st, p, ws);
    if ((e = id_allow<1>(reinterpret_cast<const void*>(id_dk<BF16>), ID_DK_LDS)) != hipSuccess) return e;
    hipLaunchKernelGGL(id_dk<BF16>, gk, dim3(256), ID_DK_LDS, st, p, ws);
  } else {
    if ((e = id_allow<2>(reinterpret_cast<const void*>(id_dq<FP8>), ID_DQ_LDS)) != hipSuccess) return e;
    hipLaunchKernelGGL(id_dq<FP8>, gq, dim3(256), ID_DQ_LDS, st, p, ws);
    if ((e = id_allow<3>(reinterpret_cast<const void*>(id_dk<FP8>), ID_DK_LDS)) != hipSuccess) return e;
    hipLaunchKernelGGL(id_dk<FP8>, gk, dim3(256), ID_DK_LDS, st, p, ws);
  }
  if (n_launches) *n_launches += 4;
  return hipGetLastError();
}

}  // namespace dsa
