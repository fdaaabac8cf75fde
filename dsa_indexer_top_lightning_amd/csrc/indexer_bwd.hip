// Backward of the lightning-indexer score at the selected positions, on gfx950.
//
// The score (GLM-5.2 IndexShare page, section 1; per-head ReLU and scalar head weight
// as in the forward) I[t,s] = sum_h w[t,h] max(0, q[t,h] . k[s,g(h)]) receives a loss
// gradient dI at the positions the top-k kept; with s = q[t,h] . k[j,g(h)] and the
// ReLU derivative taken as 0 at 0:
//
//   dw[t,h]     = sum_j dI_j max(0, s)
//   dq[t,h]     = sum_j dI_j w[t,h] [s > 0] k[j,g(h)]
//   dk[j,g(h)] += dI_j w[t,h] [s > 0] q[t,h]
//
// Gradients are with respect to the dequantised values (fp8 codes times their scales).
// index_bwd: one workgroup of 8 waves per (query token, split of its slots); wave w
// keeps heads w, w+8, ... of the token's query (decoded) in registers, lanes over the
// head dims (lane + 64 i); per selected key and head a 64-lane sum by DPP moves gives s;
// the key-gradient contributions go to dk with fp32 atomics (summed over the wave's
// heads first when all heads share one key).  For few query tokens the slots are split
// over several workgroups that add their dq and dw shares with atomics.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int IB_THREADS = 512;
constexpr int IB_WAVES = IB_THREADS / 64;
constexpr int IB_HPW = 8;   // heads per wave (H <= 64)
constexpr int IB_DI = 4;    // dims per lane (D <= 256)

template <int CTRL, int ROWS>
__device__ __forceinline__ float ib_dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}
// sum over the 64 lanes (the same DPP sequence as the sparse MLA backward)
__device__ __forceinline__ float ib_wave_sum(float v) {
  v += ib_dpp<0xB1, 0xF>(v);
  v += ib_dpp<0x4E, 0xF>(v);
  v += ib_dpp<0x141, 0xF>(v);
  v += ib_dpp<0x140, 0xF>(v);
  v += ib_dpp<0x142, 0xA>(v);
  v += ib_dpp<0x143, 0xC>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

template <int DT>
__device__ __forceinline__ float ib_ld(const void* base, int64_t i) {
  if constexpr (DT == F32) return static_cast<const float*>(base)[i];
  else if constexpr (DT == BF16) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
  else return __builtin_amdgcn_cvt_f32_fp8((int)static_cast<const uint8_t*>(base)[i], 0);  // OCP e4m3fn
}

template <int DT>
__global__ __launch_bounds__(IB_THREADS) void index_bwd(IndexBwdParams p, int nsplit, int per_split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tok = blockIdx.x / nsplit;
  const int split = (int)(blockIdx.x % nsplit);
  const int64_t b = tok / p.T;
  const int H = p.H, D = p.D, Hk = p.Hk;
  const int jbeg = split * per_split, jend = min(p.topk, jbeg + per_split);

  float q[IB_HPW][IB_DI], dq[IB_HPW][IB_DI], wh[IB_HPW], dw[IB_HPW];
#pragma unroll
  for (int k = 0; k < IB_HPW; ++k) {
    const int h = wave + IB_WAVES * k;
    const bool on = h < H;
    float qs = 1.f;
    if constexpr (DT == FP8) qs = on ? p.q_scale[tok * H + h] : 0.f;
    wh[k] = on ? p.w[tok * H + h] : 0.f;
    dw[k] = 0.f;
#pragma unroll
    for (int i = 0; i < IB_DI; ++i) {
      const int d = lane + 64 * i;
      q[k][i] = (on && d < D) ? ib_ld<DT>(p.q, (tok * H + h) * D + d) * qs : 0.f;
      dq[k][i] = 0.f;
    }
  }

  const int32_t* idx = p.idx + tok * (int64_t)p.topk;
  const float* dI = p.dI + tok * (int64_t)p.topk;
  for (int j = jbeg; j < jend; ++j) {
    const int32_t e = idx[j];
    const float g = dI[j];
    if (e < 0 || (int64_t)e >= p.s_cap || g == 0.f) continue;  // uniform: nothing to add
    const int64_t krow = (b * p.s_cap + e) * Hk;
    float acc[IB_DI] = {0.f, 0.f, 0.f, 0.f};  // shared key head: this wave's heads summed
#pragma unroll
    for (int k = 0; k < IB_HPW; ++k) {
      const int h = wave + IB_WAVES * k;
      if (h >= H) break;  // uniform per wave
      const int gh = (Hk == H) ? h : 0;
      float ks = 1.f;
      if constexpr (DT == FP8) ks = p.k_scale[krow + gh];
      float kv[IB_DI], part = 0.f;
#pragma unroll
      for (int i = 0; i < IB_DI; ++i) {
        const int d = lane + 64 * i;
        kv[i] = d < D ? ib_ld<DT>(p.k, (krow + gh) * D + d) * ks : 0.f;
        part = fmaf(q[k][i], kv[i], part);
      }
      const float s = ib_wave_sum(part);
      if (s > 0.f) {  // uniform
        dw[k] = fmaf(g, s, dw[k]);
        const float c = g * wh[k];
#pragma unroll
        for (int i = 0; i < IB_DI; ++i) {
          dq[k][i] = fmaf(c, kv[i], dq[k][i]);
          const int d = lane + 64 * i;
          if (Hk == H) {
            if (d < D) atomicAdd(&p.dk[(krow + gh) * D + d], c * q[k][i]);
          } else {
            acc[i] = fmaf(c, q[k][i], acc[i]);
          }
        }
      }
    }
    if (Hk != H) {
#pragma unroll
      for (int i = 0; i < IB_DI; ++i) {
        const int d = lane + 64 * i;
        if (d < D && acc[i] != 0.f) atomicAdd(&p.dk[krow * D + d], acc[i]);
      }
    }
  }

#pragma unroll
  for (int k = 0; k < IB_HPW; ++k) {
    const int h = wave + IB_WAVES * k;
    if (h >= H) break;
#pragma unroll
    for (int i = 0; i < IB_DI; ++i) {
      const int d = lane + 64 * i;
      if (d < D) {
        if (nsplit == 1) p.dq[(tok * H + h) * D + d] = dq[k][i];
        else atomicAdd(&p.dq[(tok * H + h) * D + d], dq[k][i]);
      }
    }
    if (lane == 0) {
      if (nsplit == 1) p.dw[tok * H + h] = dw[k];
      else atomicAdd(&p.dw[tok * H + h], dw[k]);
    }
  }
}

__global__ __launch_bounds__(256) void ib_zero(float* x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.f;
}

void ib_clear(float* x, int64_t n, hipStream_t st, int* n_launches) {
  if (n <= 0) return;
  hipLaunchKernelGGL(ib_zero, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0, st, x, n);
  if (n_launches) ++*n_launches;
}

}  // namespace

bool index_bwd_supported(int H, int D, int Hk) {
  return H >= 1 && H <= IB_WAVES * IB_HPW && D >= 1 && D <= 64 * IB_DI && (Hk == H || Hk == 1);
}

hipError_t launch_index_bwd(const IndexBwdParams& p, Dtype dt, void* ws, size_t ws_bytes, hipStream_t st,
                            int* n_launches) {
  if (index_bwd_dense(p.B, p.T, p.H, p.D, p.Hk, p.topk, p.s_cap, dt))
    return launch_index_bwd_dense(p, dt, ws, ws_bytes, st, n_launches);
  const int64_t rows = (int64_t)p.B * p.T;
  int nsplit = 1;
  if (rows > 0 && rows < 1024) nsplit = (int)std::min<int64_t>(p.topk, (1024 + rows - 1) / rows);
  const int per_split = (p.topk + nsplit - 1) / nsplit;
  nsplit = (p.topk + per_split - 1) / per_split;
  ib_clear(p.dk, (int64_t)p.B * p.s_cap * p.Hk * p.D, st, n_launches);
  if (nsplit > 1) {
    ib_clear(p.dq, rows * p.H * p.D, st, n_launches);
    ib_clear(p.dw, rows * p.H, st, n_launches);
  }
  if (rows == 0) return hipGetLastError();
  const dim3 grid((unsigned)(rows * nsplit));
  switch (dt) {
    case F32: hipLaunchKernelGGL(index_bwd<F32>, grid, dim3(IB_THREADS), 0, st, p, nsplit, per_split); break;
    case BF16: hipLaunchKernelGGL(index_bwd<BF16>, grid, dim3(IB_THREADS), 0, st, p, nsplit, per_split); break;
    default: hipLaunchKernelGGL(index_bwd<FP8>, grid, dim3(IB_THREADS), 0, st, p, nsplit, per_split); break;
  }
  if (n_launches) ++*n_launches;
  return hipGetLastError();
}

}  // namespace dsa
