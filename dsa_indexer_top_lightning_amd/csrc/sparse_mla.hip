// Sparse MLA attention over the selected latent rows, on gfx950.
//
// For each query (b,t) and head h, attention runs only over the rows whose
// positions topk_indices[b,t,:] lists (GLM-5.2 IndexShare page, section 1: the
// main attention runs on the selected positions instead of the whole prefix; the
// table "What is actually shared?": every layer computes its own attention with
// its own inputs).  Absorbed MLA: a latent row holds kv_lora_rank 512 + rope 64 =
// 576 values (Megatron-Bridge pull request, commit on the rope-dim parse); it is
// the key, and its first 512 values are the value.
//
// mla_mfma (bf16, Dc = 512, Dr = 64, 64 heads per workgroup):
//   * the workgroup's indices are compacted (valid entries, original order) into
//     LDS; tiles of 64 selected rows are gathered from HBM with 16-byte loads
//     (a latent row is 1152 contiguous bytes) into one row-major LDS tile, the
//     next tile being prefetched into registers while the current one is used;
//   * wave (hh, vv) computes S^T = K Q^T for kv rows [32vv, +32) x heads
//     [32hh, +32) on v_mfma_f32_32x32x16_bf16 (Q^T fragments live in registers
//     for the whole kernel), the two vv waves of a head half swap their halves
//     through LDS, and run the online softmax (exp2, fp32) for all 64 rows;
//   * the same wave accumulates O^T[256vv..+256 dims][32 heads] += V^T P^T; the
//     V^T fragments come straight from the row-major tile with ds_read_b64_tr_b16
//     (transposing LDS reads), so K and V share one LDS copy;
//   * with several workgroups per query (decode: few queries), each writes an
//     unnormalised partial (O, running max, sum) and mla_combine merges them in
//     a fixed order (no float atomics: results are run-to-run identical).
// mla_generic: any Dc/Dr/Hm, fp32 or bf16, one wave per head, fp32 FMA.
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int MT = 64;            // selected rows per tile
constexpr int MROW = 576;         // latent row (Dc + Dr)
constexpr int MDC = 512;          // value dims
constexpr int MRS = 1168;         // padded LDS row stride in bytes (1152 + 16)
constexpr int MCH = 72;           // 16-byte chunks per row
constexpr int MHG = 64;           // heads per workgroup
constexpr int MPF = MT * MCH / 256;  // prefetched chunks per thread (18)
constexpr int MAX_CHUNK = 4096;   // selected entries handled by one workgroup
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
  union {
    uint16_t u[8];
    bf16x8 b;
  } r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r.u[e] = f32_to_bf16_bits(v[e]);
  return r.b;
}

// LDS layout of mla_mfma (dynamic): tile [MT][MRS] bytes | xbuf [4 waves][16][64] f32 | idx list [chunk] i32
constexpr int LDS_TILE = MT * MRS;
constexpr int LDS_XBUF = 4 * 16 * 64 * 4;

// grid.x = (query, split) work item, heaviest queries first; grid.y = head group.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_mfma(MlaParams p, int nsplit, int chunk, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* tile = smem;
  float* xbuf = reinterpret_cast<float*>(smem + LDS_TILE);
  int32_t* idxl = reinterpret_cast<int32_t*>(smem + LDS_TILE + LDS_XBUF);
  __shared__ uint32_t wcnt[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = wave & 1, vv = wave >> 1;
  const int lr = lane & 31, lg = lane >> 5;
  const int64_t rows = (int64_t)p.B * p.T;
  const int64_t item = blockIdx.x;
  const int64_t tok = rows - 1 - item / nsplit;  // heaviest (latest) queries first
  const int split = (int)(item % nsplit);
  const int hg = blockIdx.y;
  const int64_t b = tok / p.T;
  const int64_t s_cap = p.s_cap;

  // ---- compact this split's valid indices into LDS (original order)
  const int e0 = split * chunk;
  const int e1 = min(p.topk, e0 + chunk);
  const int32_t* gidx = p.idx + tok * (int64_t)p.topk;
  int nv = 0;
  for (int c0 = e0; c0 < e1; c0 += 256) {
    const int e = c0 + tid;
    int32_t v = -1;
    if (e < e1) v = gidx[e];
    const bool ok = (e < e1) && v >= 0 && (int64_t)v < s_cap;
    const uint64_t m = __ballot(ok);
    if (lane == 0) wcnt[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    int before = nv;
    int total = 0;
    for (int w = 0; w < 4; ++w) {
      total += (int)wcnt[w];
      if (w < wave) before += (int)wcnt[w];
    }
    before += (int)__popcll(m & ((1ull << lane) - 1ull));
    if (ok) idxl[before] = v;
    nv += total;
    __syncthreads();
  }

  const int head0 = hg * MHG + 32 * hh;  // first head of this wave's half
  const int myhead = head0 + lr;
  if (nv == 0) {
    if (nsplit == 1) {
      uint16_t* og = static_cast<uint16_t*>(p.out) + (tok * p.Hm + hg * MHG) * MDC;
      for (int i = tid; i < MHG * MDC; i += 256) og[i] = 0;
      if (p.lse && vv == 0 && lg == 0) p.lse[tok * p.Hm + myhead] = -__builtin_inff();
    } else {
      if (vv == 0 && lg == 0) {
        float* ml = ws_ml + ((tok * nsplit + split) * p.Hm + myhead) * 2;
        ml[0] = -__builtin_inff();
        ml[1] = 0.f;
      }
    }
    return;
  }

  // ---- Q^T fragments for the whole kernel: lane (head lr, group lg) holds
  //      q[head][16*st + 8*lg .. +7] for st = 0..35
  bf16x8 qf[MROW / 16];
  {
    const unsigned char* qg = static_cast<const unsigned char*>(p.q) + ((tok * p.Hm + myhead) * MROW) * 2;
#pragma unroll
    for (int st = 0; st < MROW / 16; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qg + (16 * st + 8 * lg) * 2);
  }

  const unsigned char* kvg = static_cast<const unsigned char*>(p.kv) + (b * s_cap) * (MROW * 2);
  const int ntiles = (nv + MT - 1) / MT;
  i32x4 stage[MPF];
  // Padding rows of the last tile reload a valid row (masked out of the softmax),
  // so the loads need no branch; offsets are 32-bit from the item's uniform base.
  auto prefetch = [&](int t) {
#pragma unroll
    for (int k = 0; k < MPF; ++k) {
      const int c = tid + 256 * k;
      const int r = c / MCH, ch = c % MCH;
      const int e = min(t * MT + r, nv - 1);
      const uint32_t off = (uint32_t)idxl[e] * (uint32_t)(MROW * 2) + (uint32_t)ch * 16u;
      stage[k] = *reinterpret_cast<const i32x4*>(kvg + off);
    }
  };
  prefetch(0);

  const float qk_scale = p.sm_scale * LOG2E;
  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x16 acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int k = 0; k < MPF; ++k) {
      const int c = tid + 256 * k;
      const int r = c / MCH, ch = c % MCH;
      *reinterpret_cast<i32x4*>(tile + r * MRS + ch * 16) = stage[k];
    }
    __syncthreads();
    if (t + 1 < ntiles) prefetch(t + 1);

    // S^T (own 32 kv rows x 32 heads)
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const unsigned char* krow = tile + (32 * vv + lr) * MRS;
#pragma unroll
    for (int st = 0; st < MROW / 16; ++st) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (16 * st + 8 * lg) * 2);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s, 0, 0, 0);
    }
    const int valid_rows = nv - t * MT;  // rows >= valid_rows of this tile are padding
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * vv + 8 * (r >> 2) + 4 * lg + (r & 3);
      s[r] = (m < valid_rows) ? s[r] * qk_scale : -__builtin_inff();
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) xbuf[(wave * 16 + r) * 64 + lane] = s[r];
    __syncthreads();
    float sl[16], sh[16];  // kv rows of half 0 and half 1
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float o = xbuf[((wave ^ 2) * 16 + r) * 64 + lane];
      sl[r] = vv == 0 ? s[r] : o;
      sh[r] = vv == 0 ? o : s[r];
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(sl[r], sh[r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);  // finite: every tile holds a valid row
    const float alpha = exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sl[r] = exp2f(sl[r] - m_new);
      sh[r] = exp2f(sh[r] - m_new);
      rs += sl[r] + sh[r];
    }
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;

    // P^T fragments: step sg covers half sg/2, C-layout values 8*(sg%2) .. +7
    bf16x8 pf[4];
    pf[0] = pack_bf16x8(sl);
    pf[1] = pack_bf16x8(sl + 8);
    pf[2] = pack_bf16x8(sh);
    pf[3] = pack_bf16x8(sh + 8);

    // O^T[256vv + 32dt .. +32][32 heads] += V^T . P^T
    const int blk = lr >> 4, li = lr & 15;
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      const int kvb = 32 * (sg >> 1) + 16 * (sg & 1) + 4 * lg + (li >> 2);  // row of this lane's read #1
      const unsigned char* r1 = tile + kvb * MRS;
      const unsigned char* r2 = r1 + 8 * MRS;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int col = 256 * vv + 32 * dt + 16 * blk + 4 * (li & 3);
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(r1 + col * 2));
        const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(r2 + col * 2));
        union {
          i16x4 h[2];
          bf16x8 b;
        } a;
        a.h[0] = v1;
        a.h[1] = v2;
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.b, pf[sg], acc[dt], 0, 0, 0);
      }
    }
  }

  if (nsplit == 1) {
    // normalise, transpose through LDS, write out[tok][hg*64 .. +64][512] with 16-byte stores
    __syncthreads();
    constexpr int OST = MDC + 8;  // padded bf16 row stride of the staging buffer
    uint16_t* ost = reinterpret_cast<uint16_t*>(smem);
    const float inv = 1.f / l_run;
    const int hl = 32 * hh + lr;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dim = 256 * vv + 32 * dt + 8 * j + 4 * lg;
        uint16_t* dst = ost + hl * OST + dim;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = f32_to_bf16_bits(acc[dt][4 * j + i] * inv);
      }
    __syncthreads();
    unsigned char* og = static_cast<unsigned char*>(p.out) + ((tok * p.Hm + hg * MHG) * MDC) * 2;
    for (int c = tid; c < MHG * (MDC * 2 / 16); c += 256) {
      const int h = c / (MDC * 2 / 16), ch = c % (MDC * 2 / 16);
      *reinterpret_cast<i32x4*>(og + (h * MDC) * 2 + ch * 16) =
          *reinterpret_cast<const i32x4*>(reinterpret_cast<const unsigned char*>(ost + h * OST) + ch * 16);
    }
    if (p.lse && vv == 0 && lg == 0) p.lse[tok * p.Hm + myhead] = (m_run + log2f(l_run)) * LN2;
  } else {
    float* o = ws_o + ((tok * nsplit + split) * p.Hm + myhead) * MDC;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dim = 256 * vv + 32 * dt + 8 * j + 4 * lg;
        float4 v = make_float4(acc[dt][4 * j], acc[dt][4 * j + 1], acc[dt][4 * j + 2], acc[dt][4 * j + 3]);
        *reinterpret_cast<float4*>(o + dim) = v;
      }
    if (vv == 0 && lg == 0) {
      float* ml = ws_ml + ((tok * nsplit + split) * p.Hm + myhead) * 2;
      ml[0] = m_run;
      ml[1] = l_run;
    }
  }
}

// Merge the split partials of one (query, head) in split order.  grid.x = query *
// (Hm / 4); 256 threads = 4 heads x 64 threads x 8 dims.
__global__ __launch_bounds__(256) void mla_combine(MlaParams p, int nsplit, const float* __restrict__ ws_o,
                                                   const float* __restrict__ ws_ml) {
  const int64_t tok = blockIdx.x / (p.Hm / 4);
  const int head = (int)(blockIdx.x % (p.Hm / 4)) * 4 + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  float M = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws_ml[((tok * nsplit + s) * p.Hm + head) * 2]);
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < nsplit; ++s) {
      const float* ml = ws_ml + ((tok * nsplit + s) * p.Hm + head) * 2;
      if (ml[1] == 0.f) continue;
      const float f = exp2f(ml[0] - M);
      L += ml[1] * f;
      const float* src = ws_o + ((tok * nsplit + s) * p.Hm + head) * MDC + d0;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(src[i], f, o[i]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* og = static_cast<uint16_t*>(p.out) + (tok * p.Hm + head) * MDC + d0;
#pragma unroll
  for (int i = 0; i < 8; ++i) og[i] = f32_to_bf16_bits(o[i] * inv);
  if (p.lse && (threadIdx.x & 63) == 0)
    p.lse[tok * p.Hm + head] = L > 0.f ? (M + log2f(L)) * LN2 : -__builtin_inff();
}

// ----------------------------------------------------------------- generic kernel
// grid.x = query row, grid.y = block of 4 heads (one per wave).  Each lane holds
// dims lane + 64*i of q and of the output accumulator.
template <int DT>
__global__ __launch_bounds__(256) void mla_generic(MlaParams p) {
  const int64_t tok = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= p.Hm) return;
  const int R = p.Dc + p.Dr, Dc = p.Dc;
  const int64_t b = tok / p.T;
  auto ld = [&](const void* base, int64_t i) -> float {
    if constexpr (DT == F32) return static_cast<const float*>(base)[i];
    else return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  };
  float q[16], o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int d = lane + 64 * i;
    q[i] = d < R ? ld(p.q, (tok * p.Hm + h) * R + d) : 0.f;
    o[i] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  const int32_t* idx = p.idx + tok * (int64_t)p.topk;
  for (int j = 0; j < p.topk; ++j) {
    const int32_t e = idx[j];
    if (e < 0 || (int64_t)e >= p.s_cap) continue;
    const int64_t rb = (b * p.s_cap + e) * R;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = lane + 64 * i;
      if (d < R) part = fmaf(q[i], ld(p.kv, rb + d), part);
    }
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    const float z = part * p.sm_scale;
    const float mn = fmaxf(m, z);
    const float a = expf(m - mn), pj = expf(z - mn);
    l = l * a + pj;
    m = mn;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = lane + 64 * i;
      if (d < Dc) o[i] = fmaf(pj, ld(p.kv, rb + d), o[i] * a);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int d = lane + 64 * i;
    if (d < Dc) {
      const int64_t oi = (tok * p.Hm + h) * Dc + d;
      if constexpr (DT == F32) static_cast<float*>(p.out)[oi] = o[i] * inv;
      else static_cast<uint16_t*>(p.out)[oi] = f32_to_bf16_bits(o[i] * inv);
    }
  }
  if (p.lse && lane == 0) p.lse[tok * p.Hm + h] = l > 0.f ? m + logf(l) : -__builtin_inff();
}

struct SplitPlan {
  int nsplit, chunk;
};

SplitPlan plan_split(int64_t rows, int Hm, int topk) {
  const int64_t wgs = rows * (Hm / MHG);
  int nsplit = 1;
  const int max_split = (topk + MT - 1) / MT;
  // few queries (decode): split the selection so that >= 512 workgroups run
  if (wgs < 512) nsplit = (int)std::min<int64_t>(max_split, (512 + wgs - 1) / std::max<int64_t>(wgs, 1));
  int chunk = (topk + nsplit - 1) / nsplit;
  chunk = ((chunk + MT - 1) / MT) * MT;
  while (chunk > MAX_CHUNK) {
    ++nsplit;
    chunk = (((topk + nsplit - 1) / nsplit + MT - 1) / MT) * MT;
  }
  nsplit = (topk + chunk - 1) / chunk;
  return {nsplit, chunk};
}

}  // namespace

// The MFMA kernel gathers with 32-bit byte offsets inside one batch item's latent rows.
bool mla_uses_mfma(int Hm, int Dc, int Dr, int64_t s_cap, Dtype dt) {
  return dt == BF16 && Dc == MDC && Dr == MROW - MDC && Hm % MHG == 0 && s_cap * (MROW * 2) < (int64_t(1) << 32);
}

size_t mla_workspace_bytes(int B, int T, int Hm, int Dc, int Dr, int topk, int64_t s_cap, Dtype dt) {
  if (!mla_uses_mfma(Hm, Dc, Dr, s_cap, dt)) return 0;
  const int64_t rows = (int64_t)B * T;
  const SplitPlan sp = plan_split(rows, Hm, topk);
  if (sp.nsplit == 1) return 0;
  return (size_t)rows * sp.nsplit * Hm * (MDC + 2) * sizeof(float) + 256;
}

hipError_t launch_sparse_mla(const MlaParams& p, Dtype dt, void* ws, size_t, hipStream_t st, int* n_launches) {
  const int64_t rows = (int64_t)p.B * p.T;
  if (rows == 0) return hipSuccess;
  if (mla_uses_mfma(p.Hm, p.Dc, p.Dr, p.s_cap, dt)) {
    const SplitPlan sp = plan_split(rows, p.Hm, p.topk);
    const size_t lds = LDS_TILE + LDS_XBUF + (size_t)sp.chunk * 4;
    static std::atomic<size_t> high{0};
    const hipError_t attr = allow_dynamic_lds(reinterpret_cast<const void*>(mla_mfma), lds, high);
    if (attr != hipSuccess) return attr;
    float* ws_o = nullptr;
    float* ws_ml = nullptr;
    if (sp.nsplit > 1) {
      ws_o = static_cast<float*>(ws);
      ws_ml = ws_o + (size_t)rows * sp.nsplit * p.Hm * MDC;
    }
    dim3 grid((unsigned)(rows * sp.nsplit), (unsigned)(p.Hm / MHG));
    hipLaunchKernelGGL(mla_mfma, grid, dim3(256), lds, st, p, sp.nsplit, sp.chunk, ws_o, ws_ml);
    if (n_launches) ++*n_launches;
    if (sp.nsplit > 1) {
      hipLaunchKernelGGL(mla_combine, dim3((unsigned)(rows * (p.Hm / 4))), dim3(256), 0, st, p, sp.nsplit,
                         ws_o, ws_ml);
      if (n_launches) ++*n_launches;
    }
  } else {
    dim3 grid((unsigned)rows, (unsigned)((p.Hm + 3) / 4));
    if (dt == F32) hipLaunchKernelGGL(mla_generic<F32>, grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL(mla_generic<BF16>, grid, dim3(256), 0, st, p);
    if (n_launches) ++*n_launches;
  }
  return hipGetLastError();
}

}  // namespace dsa
