// Backward of the sparse MLA attention on gfx950.
//
// The forward (GLM-5.2 IndexShare page, section 1: attention over the selected
// positions only; absorbed MLA, the latent row of kv_lora_rank 512 + rope 64 values is
// the key and its first 512 values the value) has the selection as a constant, so the
// gradient flows to the queries and to the selected latent rows only:
//
//   P_j  = exp(z_j - lse),  z_j = sm_scale q . c_j      (lse from the forward)
//   dP_j = dout . c_j[:Dc],  D = dout . o              (o from the forward)
//   dz_j = P_j (dP_j - D)
//   dq   = sm_scale sum_j dz_j c_j
//   dc_j = sum_heads (sm_scale dz_j q + [P_j dout, 0])  (scatter-added over queries)
//
// mla_bwd: one workgroup of 8 waves per query token; the token's queries and output
// gradients sit in LDS in their storage type, wave w takes heads w, w+8, ... with its
// lanes over the row's values (lane + 64 i) and sums over lanes by DPP moves.  Selected
// rows are taken two at a time into LDS as fp32; each wave adds its heads' share of the
// two rows' gradients into an LDS sum (ds_add_f32), and the workgroup then adds the sums
// to the latent-row gradient in global memory with one fp32 atomic per value (rows
// shared by several queries, or listed twice, collect every contribution; the order of
// those additions is not fixed, so dkv is reproducible to fp32 rounding only).  dq is
// written whole, except for few query tokens (decode), whose selections are split over
// several workgroups that add their shares of dq with atomics.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int BW_THREADS = 512;
constexpr int BW_WAVES = BW_THREADS / 64;
constexpr int BW_MAX_HPW = 8;   // heads per wave (Hm <= 64)
constexpr int BW_RI = 10;       // row values per lane (R <= 640)
constexpr int BW_DI = 8;        // value dims per lane (Dc <= 512)
constexpr int BW_JB = 2;        // selected rows per step
constexpr float BW_LOG2E = 1.4426950408889634f;

__host__ __device__ constexpr size_t bw_align16(size_t x) { return (x + 15) & ~(size_t)15; }

__device__ __forceinline__ float bw_bf16(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

template <int DT>
__device__ __forceinline__ float bw_ld(const void* base, int64_t i) {
  if constexpr (DT == F32) return static_cast<const float*>(base)[i];
  else return bw_bf16(static_cast<const uint16_t*>(base)[i]);
}

template <int DT>
__device__ __forceinline__ float bw_lds(const unsigned char* base, int i) {
  if constexpr (DT == F32) return reinterpret_cast<const float*>(base)[i];
  else return bw_bf16(reinterpret_cast<const uint16_t*>(base)[i]);
}

// Sum over the 64 lanes with data-parallel-primitive moves (no LDS round trips): swap
// neighbours, swap pairs, mirror within 8 and within 16 lanes (each lane then holds its
// row's sum), add row 0 into row 1 and row 2 into row 3 (broadcast of lane 15), then
// rows 0+1 into rows 2 and 3 (broadcast of lane 31); lane 63 holds the total.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_move<0x140, 0xF>(v);  // row_mirror
  v += dpp_move<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  v += dpp_move<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// grid.x = (query token, split): split s takes the token's selection slots
// [s * per_split, (s + 1) * per_split); with more than one split dq is accumulated with
// atomics too (cleared beforehand).
template <int DT>
__global__ __launch_bounds__(BW_THREADS) void mla_bwd(MlaBwdParams p, int nsplit, int per_split) {
  constexpr int ESZ = (DT == F32) ? 4 : 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int Hm = p.Hm, Dc = p.Dc, R = p.Dc + p.Dr;
  unsigned char* qs = lds;                                   // [Hm][R] storage type
  unsigned char* gs = qs + bw_align16((size_t)Hm * R * ESZ); // [Hm][Dc] storage type
  float* ct = reinterpret_cast<float*>(gs + bw_align16((size_t)Hm * Dc * ESZ));  // [JB][R]
  float* dct = ct + BW_JB * R;                                // [JB][R]
  float* dh = dct + BW_JB * R;                                // [Hm] D per head
  float* l2 = dh + Hm;                                        // [Hm] lse * log2(e)
  __shared__ int32_t rows[BW_JB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tok = blockIdx.x / nsplit;
  const int split = (int)(blockIdx.x % nsplit);
  const int64_t b = tok / p.T;
  const int jbeg = split * per_split, jend = min(p.topk, jbeg + per_split);
  const float s = p.sm_scale, s2 = p.sm_scale * BW_LOG2E;

  // the token's queries and output gradients into LDS
  for (int i = tid; i < Hm * R; i += BW_THREADS) {
    if constexpr (DT == F32) reinterpret_cast<float*>(qs)[i] = static_cast<const float*>(p.q)[tok * Hm * R + i];
    else reinterpret_cast<uint16_t*>(qs)[i] = static_cast<const uint16_t*>(p.q)[tok * Hm * R + i];
  }
  for (int i = tid; i < Hm * Dc; i += BW_THREADS) {
    if constexpr (DT == F32) reinterpret_cast<float*>(gs)[i] = static_cast<const float*>(p.dout)[tok * Hm * Dc + i];
    else reinterpret_cast<uint16_t*>(gs)[i] = static_cast<const uint16_t*>(p.dout)[tok * Hm * Dc + i];
  }
  // D = dout . o and lse per head, one wave per head
  for (int h = wave; h < Hm; h += BW_WAVES) {
    float d = 0.f;
    for (int i = lane; i < Dc; i += 64)
      d = fmaf(bw_ld<DT>(p.dout, (tok * Hm + h) * Dc + i), bw_ld<DT>(p.out, (tok * Hm + h) * Dc + i), d);
    d = wave_sum(d);
    if (lane == 0) {
      dh[h] = d;
      l2[h] = p.lse[tok * Hm + h] * BW_LOG2E;
    }
  }

  float dq[BW_MAX_HPW][BW_RI];
#pragma unroll
  for (int k = 0; k < BW_MAX_HPW; ++k)
#pragma unroll
    for (int i = 0; i < BW_RI; ++i) dq[k][i] = 0.f;

  const int32_t* idx = p.idx + tok * (int64_t)p.topk;
  for (int j0 = jbeg; j0 < jend; j0 += BW_JB) {
    __syncthreads();  // previous step's LDS sums are flushed; the token's data is in place
    if (tid < BW_JB) {
      const int j = j0 + tid;
      const int32_t e = j < jend ? idx[j] : -1;
      rows[tid] = (e >= 0 && (int64_t)e < p.s_cap) ? e : -1;
    }
    __syncthreads();
    for (int i = tid; i < BW_JB * R; i += BW_THREADS) {
      const int jj = i / R, d = i % R;
      const int32_t e = rows[jj];
      ct[i] = e >= 0 ? bw_ld<DT>(p.kv, (b * p.s_cap + e) * R + d) : 0.f;
      dct[i] = 0.f;
    }
    __syncthreads();
    if (rows[0] < 0 && rows[1] < 0) continue;  // uniform

    float dc[BW_JB][BW_RI];
#pragma unroll
    for (int jj = 0; jj < BW_JB; ++jj)
#pragma unroll
      for (int i = 0; i < BW_RI; ++i) dc[jj][i] = 0.f;
#pragma unroll
    for (int k = 0; k < BW_MAX_HPW; ++k) {
      const int h = wave + BW_WAVES * k;
      if (h >= Hm) break;  // uniform per wave
      const unsigned char* qh = qs + (size_t)h * R * ESZ;
      const unsigned char* gh = gs + (size_t)h * Dc * ESZ;
      float qv[BW_RI], gv[BW_DI];
#pragma unroll
      for (int i = 0; i < BW_RI; ++i) {
        const int d = lane + 64 * i;
        qv[i] = d < R ? bw_lds<DT>(qh, d) : 0.f;
      }
#pragma unroll
      for (int i = 0; i < BW_DI; ++i) {
        const int d = lane + 64 * i;
        gv[i] = d < Dc ? bw_lds<DT>(gh, d) : 0.f;
      }
      const float Dh = dh[h], L2 = l2[h];
#pragma unroll
      for (int jj = 0; jj < BW_JB; ++jj) {
        if (rows[jj] < 0) continue;  // uniform
        const float* c = ct + jj * R;
        float zp = 0.f, dp = 0.f;
#pragma unroll
        for (int i = 0; i < BW_RI; ++i) {
          const int d = lane + 64 * i;
          const float cv = d < R ? c[d] : 0.f;
          zp = fmaf(qv[i], cv, zp);
          if (i < BW_DI) dp = fmaf(gv[i], cv, dp);  // gv is 0 past Dc
        }
        zp = wave_sum(zp);
        dp = wave_sum(dp);
        const float P = exp2f(zp * s2 - L2);
        const float dz = P * (dp - Dh);
        const float sdz = s * dz;
#pragma unroll
        for (int i = 0; i < BW_RI; ++i) {
          const int d = lane + 64 * i;
          const float cv = d < R ? c[d] : 0.f;
          dq[k][i] = fmaf(sdz, cv, dq[k][i]);
          float v = sdz * qv[i];
          if (i < BW_DI) v = fmaf(P, gv[i], v);
          dc[jj][i] += v;
        }
      }
    }
    // this wave's share of the rows' gradients into the LDS sums
#pragma unroll
    for (int jj = 0; jj < BW_JB; ++jj) {
      if (rows[jj] < 0) continue;
#pragma unroll
      for (int i = 0; i < BW_RI; ++i) {
        const int d = lane + 64 * i;
        if (d < R) atomicAdd(&dct[jj * R + d], dc[jj][i]);
      }
    }
    __syncthreads();
    for (int i = tid; i < BW_JB * R; i += BW_THREADS) {
      const int jj = i / R, d = i % R;
      const int32_t e = rows[jj];
      if (e >= 0) atomicAdd(&p.dkv[(b * p.s_cap + e) * R + d], dct[i]);
    }
  }

  // dq of this wave's heads
#pragma unroll
  for (int k = 0; k < BW_MAX_HPW; ++k) {
    const int h = wave + BW_WAVES * k;
    if (h >= Hm) break;
#pragma unroll
    for (int i = 0; i < BW_RI; ++i) {
      const int d = lane + 64 * i;
      if (d < R) {
        if (nsplit == 1) p.dq[(tok * Hm + h) * R + d] = dq[k][i];
        else atomicAdd(&p.dq[(tok * Hm + h) * R + d], dq[k][i]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void bw_zero(float* x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.f;
}

}  // namespace

size_t mla_bwd_lds_bytes(int Hm, int Dc, int Dr, Dtype dt) {
  const size_t esz = dt == F32 ? 4 : 2, R = (size_t)Dc + Dr;
  return bw_align16((size_t)Hm * R * esz) + bw_align16((size_t)Hm * Dc * esz) + 2 * BW_JB * R * 4 + 2 * (size_t)Hm * 4;
}

bool mla_bwd_supported(int Hm, int Dc, int Dr, Dtype dt) {
  return Hm >= 1 && Hm <= BW_WAVES * BW_MAX_HPW && Dc >= 1 && Dc <= 64 * BW_DI && Dr >= 0 &&
         Dc + Dr <= 64 * BW_RI && (dt == F32 || dt == BF16) && mla_bwd_lds_bytes(Hm, Dc, Dr, dt) <= 150 * 1024;
}

hipError_t launch_sparse_mla_bwd(const MlaBwdParams& p, Dtype dt, void* ws, size_t ws_bytes, hipStream_t st,
                                 int* n_launches) {
  if (mla_bwd_uses_mfma(p.Hm, p.Dc, p.Dr, p.s_cap, dt)) return launch_sparse_mla_bwd_mfma(p, ws, ws_bytes, st, n_launches);
  const int64_t rows = (int64_t)p.B * p.T;
  const int64_t nkv = (int64_t)p.B * p.s_cap * (p.Dc + p.Dr);
  // few query tokens (decode): split each selection so that >= 1024 workgroups run
  int nsplit = 1;
  if (rows > 0 && rows < 1024) nsplit = (int)std::min<int64_t>((p.topk + BW_JB - 1) / BW_JB, (1024 + rows - 1) / rows);
  int per_split = (p.topk + nsplit - 1) / nsplit;
  per_split = (per_split + BW_JB - 1) / BW_JB * BW_JB;
  nsplit = per_split > 0 ? (p.topk + per_split - 1) / per_split : 1;
  if (nkv > 0) {
    hipLaunchKernelGGL(bw_zero, dim3((unsigned)std::min<int64_t>((nkv + 255) / 256, 4096)), dim3(256), 0, st,
                       p.dkv, nkv);
    if (n_launches) ++*n_launches;
  }
  const int64_t nq = rows * p.Hm * (p.Dc + p.Dr);
  if (nsplit > 1 && nq > 0) {
    hipLaunchKernelGGL(bw_zero, dim3((unsigned)std::min<int64_t>((nq + 255) / 256, 4096)), dim3(256), 0, st,
                       p.dq, nq);
    if (n_launches) ++*n_launches;
  }
  if (rows == 0) return hipGetLastError();
  const size_t lds = mla_bwd_lds_bytes(p.Hm, p.Dc, p.Dr, dt);
  hipError_t e;
  if (dt == F32) {
    static std::atomic<size_t> high{0};
    if ((e = allow_dynamic_lds(reinterpret_cast<const void*>(mla_bwd<F32>), lds, high)) != hipSuccess) return e;
    hipLaunchKernelGGL(mla_bwd<F32>, dim3((unsigned)(rows * nsplit)), dim3(BW_THREADS), lds, st, p, nsplit, per_split);
  } else {
    static std::atomic<size_t> high{0};
    if ((e = allow_dynamic_lds(reinterpret_cast<const void*>(mla_bwd<BF16>), lds, high)) != hipSuccess) return e;
    hipLaunchKernelGGL(mla_bwd<BF16>, dim3((unsigned)(rows * nsplit)), dim3(BW_THREADS), lds, st, p, nsplit, per_split);
  }
  if (n_launches) ++*n_launches;
  return hipGetLastError();
}

}  // namespace dsa
