// Internal launch interface between the C-ABI host layer (dsa_api.cpp) and the
// gfx950 kernels.  Not installed; the public interface is include/dsa.h.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>

namespace dsa {

enum Dtype : int { F32 = 0, BF16 = 1, FP8 = 2 };

struct IndexerParams {
  int B, T, H, D, Hk;
  int64_t s_cap;
  const int32_t* key_start;  // nullable
  const int32_t* key_end;    // nullable
  const void* q;
  const float* q_scale;
  const void* k;
  const float* k_scale;
  const float* w;
  float* scores;
  int64_t ld;
  // Rows with row_mask[row] == 0 are skipped (nothing written).  Nullable.
  const int32_t* row_mask = nullptr;
  // Launch hint: the mask leaves few rows live (the tile kernel then runs one block per key
  // tile that walks the query tiles, instead of one block per tile).
  int few_rows = 0;
  // Sampling (kstride > 1): only keys s = kstride * i are scored, into scores[row * ld + i].
  int64_t kstride = 1;
  // Candidate mode (lkey != nullptr): no scores are written; every cell whose order key
  // (order_key below) is >= lkey[row] is appended to its row's list: slot =
  // atomicAdd(cand_cnt + row, 1), and if slot < cap, cand_pos[row * cap + slot] = key
  // position, cand_val[row * cap + slot] = score.
  const uint32_t* lkey = nullptr;
  int32_t* cand_cnt = nullptr;
  int32_t* cand_pos = nullptr;
  float* cand_val = nullptr;
  int32_t cap = 0;
  // Optional head-major copies of the per-head vectors (written by launch_indexer_vectors):
  // ks_t [B][H][vec_s] = k_scale, wq_t [B][H][vec_t] = w * q_scale (one fp32 product), zero
  // past s_cap and T.  With them the fp8 tile kernel loads a head's vectors of a tile as two
  // contiguous runs instead of one 4-byte word per row and key.  Nullable.
  const float* ks_t = nullptr;
  const float* wq_t = nullptr;
  int64_t vec_s = 0, vec_t = 0;
};

struct TopkParams {
  int B, T, topk;
  int64_t s_cap;
  const int32_t* key_start;
  const int32_t* key_end;
  const float* scores;
  int64_t ld;
  int32_t* out;
  const int32_t* row_mask = nullptr;  // rows with row_mask[row] == 0 are skipped (nullable)
};

struct MlaParams {
  int B, T, Hm, Dc, Dr, topk;
  int64_t s_cap;
  const void* q;
  const void* kv;
  const int32_t* idx;
  float sm_scale;
  void* out;
  float* lse;
};

// Backward of the sparse MLA attention: forward inputs and results, output gradient.
struct MlaBwdParams {
  int B, T, Hm, Dc, Dr, topk;
  int64_t s_cap;
  const void* q;        // [B,T,Hm,Dc+Dr]
  const void* kv;       // [B,S,Dc+Dr]
  const int32_t* idx;   // [B,T,topk]
  float sm_scale;
  const void* out;      // [B,T,Hm,Dc] forward output
  const float* lse;     // [B,T,Hm] forward log-sum-exp
  const void* dout;     // [B,T,Hm,Dc]
  float* dq;            // [B,T,Hm,Dc+Dr]
  float* dkv;           // [B,S,Dc+Dr]
};

// Backward of the index score at the selected positions.
struct IndexBwdParams {
  int B, T, H, D, Hk, topk;
  int64_t s_cap;
  const void* q;          // [B,T,H,D]
  const float* q_scale;   // [B,T,H] (fp8)
  const void* k;          // [B,S,Hk,D]
  const float* k_scale;   // [B,S,Hk] (fp8)
  const float* w;         // [B,T,H]
  const int32_t* idx;     // [B,T,topk]
  const float* dI;        // [B,T,topk]
  float* dq;              // [B,T,H,D]
  float* dk;              // [B,S,Hk,D]
  float* dw;              // [B,T,H]
};

// New index vectors x [n, heads, D] fp32 -> RoPE -> out rows (bf16 or fp8 codes + scales).
struct PrepParams {
  int n, heads, D;
  float theta;
  int out_dtype;            // BF16 or FP8
  const float* x;
  const int32_t* pos;       // [n]
  const int64_t* rows;      // [n] destination rows, or NULL (row = n)
  int64_t n_rows;           // rows of out; destinations outside [0, n_rows) are skipped
  void* out;                // [n_rows, heads, D]
  float* out_scale;         // [n_rows, heads] (fp8)
};

// New latent rows src [n, row_bytes] -> dst rows.
struct LatentAppendParams {
  int64_t n;
  int row_bytes;            // multiple of 16
  const void* src;
  const int64_t* rows;
  int64_t n_rows;
  void* dst;
};

// Each launcher assumes its arguments were validated by the host layer.
hipError_t launch_indexer(const IndexerParams& p, Dtype dt, hipStream_t st, int* n_launches);
// Whether the shape runs on a kernel with row masks, sampling and candidate mode (the fp8
// tile kernel with one key head per query head, or the decode stream kernel).
bool indexer_modes_supported(const IndexerParams& p, Dtype dt);
// Bytes of the head-major vector copies for the shape (0 where the fp8 tile kernel does not
// run it); launch_indexer_vectors writes them into `dst` and points p.ks_t / p.wq_t there.
size_t indexer_vectors_bytes(int B, int T, int H, int D, int Hk, int64_t s_cap, Dtype dt);
hipError_t launch_indexer_vectors(IndexerParams& p, Dtype dt, void* dst, hipStream_t st, int* n_launches);
size_t topk_workspace_bytes(int B, int T, int topk, int64_t s_cap);
hipError_t launch_topk(const TopkParams& p, void* ws, size_t ws_bytes, hipStream_t st, int* n_launches);
// Fused indexer -> top-k.  Workspace: [rows * s_cap fp32 scores][top-k workspace], then,
// when `fused`, the sample, threshold and candidate buffers and `vec_bytes` of head-major
// vectors (indexer_vectors_bytes).  The scores region is only written for rows that fall
// back (or by the unfused path of shapes that cannot fuse).
bool indexer_topk_fused(const IndexerParams& p, Dtype dt, int topk);
bool indexer_topk_stride_ok(int64_t stride);
size_t indexer_topk_workspace_bytes(int B, int T, int topk, int64_t s_cap, bool fused, size_t vec_bytes);
hipError_t launch_indexer_topk(const IndexerParams& p, Dtype dt, int topk, int64_t stride, int32_t* out, void* ws,
                               size_t ws_bytes, hipStream_t st, int* n_launches);
bool mla_uses_mfma(int Hm, int Dc, int Dr, int64_t s_cap, Dtype dt);
size_t mla_workspace_bytes(int B, int T, int Hm, int Dc, int Dr, int topk, int64_t s_cap, Dtype dt);
hipError_t launch_sparse_mla(const MlaParams& p, Dtype dt, void* ws, size_t ws_bytes, hipStream_t st,
                             int* n_launches);
size_t mla_bwd_lds_bytes(int Hm, int Dc, int Dr, Dtype dt);
bool mla_bwd_supported(int Hm, int Dc, int Dr, Dtype dt);
// bf16 with 512 + 64 latent rows and heads in groups of 64 runs on the matrix cores (its
// workspace holds P and sm_scale * dz per selected slot); other shapes on the vector kernel
bool mla_bwd_uses_mfma(int Hm, int Dc, int Dr, int64_t s_cap, Dtype dt);
size_t mla_bwd_workspace_bytes(int B, int T, int Hm, int Dc, int Dr, int topk, int64_t s_cap, Dtype dt);
hipError_t launch_sparse_mla_bwd_mfma(const MlaBwdParams& p, void* ws, size_t ws_bytes, hipStream_t st,
                                      int* n_launches);
hipError_t launch_sparse_mla_bwd(const MlaBwdParams& p, Dtype dt, void* ws, size_t ws_bytes, hipStream_t st,
                                 int* n_launches);
bool index_bwd_supported(int H, int D, int Hk);
// dense-selection path of the index backward (matrix cores; needs a workspace)
bool index_bwd_dense(int B, int T, int H, int D, int Hk, int topk, int64_t s_cap, Dtype dt);
size_t index_bwd_workspace_bytes(int B, int T, int H, int D, int Hk, int topk, int64_t s_cap, Dtype dt);
hipError_t launch_index_bwd_dense(const IndexBwdParams& p, Dtype dt, void* ws, size_t ws_bytes, hipStream_t st,
                                  int* n_launches);
hipError_t launch_index_bwd(const IndexBwdParams& p, Dtype dt, void* ws, size_t ws_bytes, hipStream_t st,
                            int* n_launches);
hipError_t launch_index_prep(const PrepParams& p, hipStream_t st);
hipError_t launch_latent_append(const LatentAppendParams& p, hipStream_t st);

// Dynamic LDS above 64 KiB must be allowed per kernel.  `high` remembers the
// largest size already allowed for that kernel; a failure is returned and the
// runtime's last-error slot is cleared so it does not leak into later calls.
inline hipError_t allow_dynamic_lds(const void* kernel, size_t bytes, std::atomic<size_t>& high) {
  if (bytes <= 65536 || bytes <= high.load()) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return e;
  }
  size_t cur = high.load();
  while (bytes > cur && !high.compare_exchange_weak(cur, bytes)) {
  }
  return hipSuccess;
}

// Scores -> uint32 keys that order like the floats (-0.0 folded onto +0.0).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Clamp a query's candidate range to [0, s_cap].
__device__ __forceinline__ void clamp_range(const int32_t* ks_arr, const int32_t* ke_arr, int64_t row,
                                            int64_t s_cap, int64_t& ks, int64_t& ke) {
  int64_t a = ks_arr ? (int64_t)ks_arr[row] : 0;
  int64_t e = ke_arr ? (int64_t)ke_arr[row] : s_cap;
  a = a < 0 ? 0 : (a > s_cap ? s_cap : a);
  e = e < a ? a : (e > s_cap ? s_cap : e);
  ks = a;
  ke = e;
}

}  // namespace dsa
