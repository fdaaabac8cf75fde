// C-ABI host layer: argument checks (all before any enqueue), dispatch to the
// gfx950 kernels, and the IndexShare group driver.
//
// Group driver (GLM-5.2 IndexShare page, section 2 and the layer-pattern figure:
// full layers run the indexer and cache the top-k indices, shared layers reuse
// the nearest preceding full layer's indices; the page's implementation checklist
// asks to follow indexer_types rather than a fixed pattern).  The handle plays the
// part of the carried indexer state of MaxText's scanned layer loop and of the
// per-microbatch top-k holder of the Megatron-Bridge pull request; that pull
// request's stage-start check and stale-holder guard become DSA_ERR_NO_DONOR and
// DSA_ERR_STALE_CACHE.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status hip_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_dtype(int d) { return d == DSA_F32 || d == DSA_BF16 || d == DSA_FP8_E4M3; }

int64_t rows_of(const dsa_shape* s) { return (int64_t)s->B * s->T; }

dsa_status check_common(const dsa_shape* s) {
  if (!s) return fail(DSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 0 || s->T < 0 || s->s_cap < 0)
    return fail(DSA_ERR_INVALID_ARG, "negative size: B=%d T=%d s_cap=%lld", s->B, s->T, (long long)s->s_cap);
  if (s->s_cap > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "s_cap %lld exceeds int32 positions", (long long)s->s_cap);
  return DSA_OK;
}

dsa_status check_indexer_shape(const dsa_shape* s, dsa_dtype dt) {
  dsa_status st = check_common(s);
  if (st != DSA_OK) return st;
  if (!valid_dtype(dt)) return fail(DSA_ERR_INVALID_ARG, "unknown index dtype %d", (int)dt);
  if (s->H < 1 || s->D < 1 || s->Hk < 1) return fail(DSA_ERR_INVALID_ARG, "H, D, Hk must be >= 1");
  if (s->Hk != 1 && s->Hk != s->H) return fail(DSA_ERR_INVALID_ARG, "Hk must be 1 or H (Hk=%d H=%d)", s->Hk, s->H);
  if (s->H > 128) return fail(DSA_ERR_UNSUPPORTED, "H=%d > 128", s->H);
  if (s->D % 16 != 0 || s->D > 256) return fail(DSA_ERR_UNSUPPORTED, "D=%d: need D %% 16 == 0 and D <= 256", s->D);
  return DSA_OK;
}

dsa_status check_indexer_ptrs(const dsa_shape* s, dsa_dtype dt, const void* q, const float* qs, const void* k,
                              const float* kscale, const float* w) {
  if (rows_of(s) == 0 || s->s_cap == 0) return DSA_OK;
  if (!q || !k || !w) return fail(DSA_ERR_INVALID_ARG, "index q, k and w must be non-NULL");
  if (dt == DSA_FP8_E4M3 && (!qs || !kscale)) return fail(DSA_ERR_INVALID_ARG, "fp8 inputs need q_scale and k_scale");
  return DSA_OK;
}

dsa_status check_scores(const dsa_shape* s, const float* scores, int64_t ld) {
  if (ld < s->s_cap) return fail(DSA_ERR_INVALID_ARG, "ld_scores %lld < s_cap %lld", (long long)ld, (long long)s->s_cap);
  if (rows_of(s) > 0 && s->s_cap > 0 && !scores) return fail(DSA_ERR_INVALID_ARG, "scores must be non-NULL");
  return DSA_OK;
}

dsa_status check_topk_shape(const dsa_shape* s) {
  dsa_status st = check_common(s);
  if (st != DSA_OK) return st;
  if (s->topk < 1) return fail(DSA_ERR_INVALID_ARG, "topk=%d must be >= 1", s->topk);
  return DSA_OK;
}

dsa_status check_mla_shape(const dsa_shape* s, dsa_dtype dt) {
  dsa_status st = check_topk_shape(s);
  if (st != DSA_OK) return st;
  if (dt != DSA_F32 && dt != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "MLA dtype %d: need F32 or BF16", (int)dt);
  if (s->Hm < 1 || s->Dc < 1 || s->Dr < 0) return fail(DSA_ERR_INVALID_ARG, "need Hm >= 1, Dc >= 1, Dr >= 0");
  if (s->Hm > 1024 || s->Dc + s->Dr > 1024 || s->Dc % 8 || s->Dr % 8)
    return fail(DSA_ERR_UNSUPPORTED, "Hm=%d Dc=%d Dr=%d: need Hm <= 1024, Dc+Dr <= 1024, Dc and Dr multiples of 8",
                s->Hm, s->Dc, s->Dr);
  return DSA_OK;
}

dsa_status check_mla_ptrs(const dsa_shape* s, const void* q, const void* kv, const void* out) {
  if (rows_of(s) == 0) return DSA_OK;
  if (!q || !out || (!kv && s->s_cap > 0)) return fail(DSA_ERR_INVALID_ARG, "q, kv and out must be non-NULL");
  return DSA_OK;
}

dsa_status check_sm_scale(float sm_scale) {
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(DSA_ERR_INVALID_ARG, "sm_scale must be a positive finite number (got %g)", (double)sm_scale);
  return DSA_OK;
}

size_t topk_ws(const dsa_shape* s) { return dsa::topk_workspace_bytes(s->B, s->T, s->topk, s->s_cap); }
size_t mla_ws(const dsa_shape* s, dsa_dtype dt) {
  return dsa::mla_workspace_bytes(s->B, s->T, s->Hm, s->Dc, s->Dr, s->topk, s->s_cap, (dsa::Dtype)dt);
}
size_t mla_bwd_ws(const dsa_shape* s, dsa_dtype dt) {
  return dsa::mla_bwd_workspace_bytes(s->B, s->T, s->Hm, s->Dc, s->Dr, s->topk, s->s_cap, (dsa::Dtype)dt);
}
size_t index_bwd_ws(const dsa_shape* s, dsa_dtype dt) {
  return dsa::index_bwd_workspace_bytes(s->B, s->T, s->H, s->D, s->Hk, s->topk, s->s_cap, (dsa::Dtype)dt);
}
size_t scores_bytes(const dsa_shape* s) { return align_up((size_t)rows_of(s) * (size_t)s->s_cap * sizeof(float)); }

// Full layers of a group over rows at least this long run the fused indexer -> top-k.
constexpr int64_t kFuseMinKeys = 65536;

dsa::IndexerParams indexer_params(const dsa_shape* s, const void* q, const float* qs, const void* k,
                                  const float* ksc, const float* w, float* scores, int64_t ld) {
  return dsa::IndexerParams{s->B, s->T, s->H, s->D, s->Hk, s->s_cap, s->key_start, s->key_end, q, qs, k, ksc, w,
                            scores, ld};
}
// Whether dsa_indexer_topk runs the shape without the score matrix (for this dtype / any dtype).
bool fused_shape(const dsa_shape* s, dsa_dtype dt) {
  return dsa::indexer_topk_fused(indexer_params(s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, s->s_cap),
                                 (dsa::Dtype)dt, s->topk);
}
bool fused_any(const dsa_shape* s) { return fused_shape(s, DSA_BF16) || fused_shape(s, DSA_FP8_E4M3); }
size_t indexer_topk_ws(const dsa_shape* s, bool fused) {
  // the head-major vectors exist for fp8 only: sized for it whatever the call's dtype
  const size_t vec = fused ? dsa::indexer_vectors_bytes(s->B, s->T, s->H, s->D, s->Hk, s->s_cap, dsa::FP8) : 0;
  return dsa::indexer_topk_workspace_bytes(s->B, s->T, s->topk, s->s_cap, fused, vec);
}
// Inside a group only prefill chunks fuse (fp8 tile kernel, T >= 64): for decode rows the score
// round trip is small beside the key stream and the fused passes cost more than it.
bool group_fuses(const dsa_shape* s, dsa_dtype dt) {
  return s->s_cap >= kFuseMinKeys && s->T >= 64 && fused_shape(s, dt);
}

dsa::TopkParams topk_params(const dsa_shape* s, const float* scores, int64_t ld, int32_t* out) {
  return dsa::TopkParams{s->B, s->T, s->topk, s->s_cap, s->key_start, s->key_end, scores, ld, out};
}
dsa::MlaParams mla_params(const dsa_shape* s, const void* q, const void* kv, const int32_t* idx, float sm, void* out,
                          float* lse) {
  return dsa::MlaParams{s->B, s->T, s->Hm, s->Dc, s->Dr, s->topk, s->s_cap, q, kv, idx, sm, out, lse};
}

// Analytic counters of a group call from host copies of the key ranges (NULL: 0 and
// s_cap).  Candidate count n = clamped key_end - key_start, selected rows min(n, topk).
void group_counters(const dsa_shape* s, dsa_dtype idx_dtype, dsa_dtype mla_dtype, int32_t n_layers,
                    const dsa_layer_type* types, const int32_t* ks_h, const int32_t* ke_h, dsa_group_stats* out) {
  const int64_t rows = rows_of(s);
  double sum_n = 0, sum_j = 0, prefix = 0;
  for (int b = 0; b < s->B; ++b) {
    int64_t mx = 0;
    for (int t = 0; t < s->T; ++t) {
      const int64_t r = (int64_t)b * s->T + t;
      int64_t a = ks_h ? ks_h[r] : 0, z = ke_h ? ke_h[r] : s->s_cap;
      a = std::min<int64_t>(std::max<int64_t>(a, 0), s->s_cap);
      z = std::min<int64_t>(std::max<int64_t>(z, a), s->s_cap);
      sum_n += (double)(z - a);
      sum_j += (double)std::min<int64_t>(z - a, s->topk);
      mx = std::max(mx, z);
    }
    prefix += (double)mx;
  }
  int n_full = 0;
  for (int l = 0; l < n_layers; ++l) n_full += types[l] == DSA_FULL;
  const double ie = idx_dtype == DSA_F32 ? 4 : (idx_dtype == DSA_BF16 ? 2 : 1);
  const double sc = idx_dtype == DSA_FP8_E4M3 ? 4 : 0;
  const double me = mla_dtype == DSA_F32 ? 4 : 2;
  const double R = s->Dc + s->Dr;
  *out = dsa_group_stats{};
  out->n_full = n_full;
  out->n_shared = n_layers - n_full;
  out->n_fused = group_fuses(s, idx_dtype) ? n_full : 0;
  out->indexer_flops = n_full * 2.0 * s->H * s->D * sum_n;
  out->indexer_bytes =
      n_full * ((double)rows * s->H * (s->D * ie + 4 + sc) + prefix * s->Hk * (s->D * ie + sc) + 4.0 * sum_n);
  out->topk_bytes = n_full * (4.0 * sum_n + 4.0 * (double)rows * s->topk);
  out->attn_flops = n_layers * 2.0 * s->Hm * (2.0 * s->Dc + s->Dr) * sum_j;
  out->attn_bytes = n_layers * (sum_j * R * me + (double)rows * s->Hm * R * me + (double)rows * s->Hm * s->Dc * me);
}

// ---- allocation-free group call
// Scratch of dsa_group_forward_noalloc: a file-scope device array, one copy per GPU,
// held for the life of the process.  In host code `scratch` names a host-side stand-in,
// not device memory, so its device address is looked up once per device (with that
// device current) and only that address is handed to kernels.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of the current device's scratch (looked up on the first call on it).
dsa_status current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a NULL address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_last_error(void) { return g_last_error.c_str(); }

const char* dsa_status_string(dsa_status st) {
  switch (st) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_NO_DONOR: return "DSA_ERR_NO_DONOR";
    case DSA_ERR_STALE_CACHE: return "DSA_ERR_STALE_CACHE";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "DSA_ERR_WORKSPACE_TOO_SMALL";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

size_t dsa_workspace_bytes(const dsa_shape* s, dsa_op op) {
  if (!s || s->B < 0 || s->T < 0 || s->s_cap < 0 || s->topk < 0) return 0;
  switch (op) {
    case DSA_OP_INDEXER: return 0;
    case DSA_OP_TOPK: return topk_ws(s);
    case DSA_OP_SPARSE_MLA: return mla_ws(s, DSA_BF16);
    case DSA_OP_GROUP: {
      const size_t plain = scores_bytes(s) + align_up(std::max(topk_ws(s), mla_ws(s, DSA_BF16)));
      const bool fuse = s->s_cap >= kFuseMinKeys && s->T >= 64 && fused_any(s);
      return fuse ? std::max(plain, indexer_topk_ws(s, true)) : plain;
    }
    case DSA_OP_INDEXER_TOPK: return indexer_topk_ws(s, fused_any(s));
    case DSA_OP_SPARSE_MLA_BWD: return mla_bwd_ws(s, DSA_BF16);
    case DSA_OP_INDEX_BWD: return std::max(index_bwd_ws(s, DSA_BF16), index_bwd_ws(s, DSA_FP8_E4M3));
  }
  return 0;
}

dsa_status dsa_indexer_scores(const dsa_shape* s, dsa_dtype dt, const void* q, const float* qs, const void* k,
                              const float* ksc, const float* w, float* scores, int64_t ld, void* stream) {
  dsa_status st = check_indexer_shape(s, dt);
  if (st == DSA_OK) st = check_indexer_ptrs(s, dt, q, qs, k, ksc, w);
  if (st == DSA_OK) st = check_scores(s, scores, ld);
  if (st != DSA_OK) return st;
  hipError_t e = dsa::launch_indexer(indexer_params(s, q, qs, k, ksc, w, scores, ld), (dsa::Dtype)dt,
                                     (hipStream_t)stream, nullptr);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "indexer launch");
}

dsa_status dsa_topk_select(const dsa_shape* s, const float* scores, int64_t ld, int32_t* out, void* ws,
                           size_t ws_bytes, void* stream) {
  dsa_status st = check_topk_shape(s);
  if (st == DSA_OK) st = check_scores(s, scores, ld);
  if (st != DSA_OK) return st;
  if (rows_of(s) > 0 && !out) return fail(DSA_ERR_INVALID_ARG, "topk_indices must be non-NULL");
  const size_t need = topk_ws(s);
  if (ws_bytes < need || (need && !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "top-k workspace %zu < %zu", ws_bytes, need);
  hipError_t e = dsa::launch_topk(topk_params(s, scores, ld, out), ws, ws_bytes, (hipStream_t)stream, nullptr);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "top-k launch");
}

dsa_status dsa_indexer_topk(const dsa_shape* s, dsa_dtype dt, const void* q, const float* qs, const void* k,
                            const float* ksc, const float* w, int32_t* out, int32_t sample_stride, void* ws,
                            size_t ws_bytes, void* stream) {
  dsa_status st = check_indexer_shape(s, dt);
  if (st == DSA_OK) st = check_topk_shape(s);
  if (st == DSA_OK) st = check_indexer_ptrs(s, dt, q, qs, k, ksc, w);
  if (st != DSA_OK) return st;
  if (rows_of(s) > 0 && !out) return fail(DSA_ERR_INVALID_ARG, "topk_indices must be non-NULL");
  if (!dsa::indexer_topk_stride_ok(sample_stride))
    return fail(DSA_ERR_INVALID_ARG, "sample_stride %d: need 0 or 16 .. 1048576", sample_stride);
  if (rows_of(s) == 0) return DSA_OK;
  const size_t need = indexer_topk_ws(s, fused_shape(s, dt));
  if (ws_bytes < need || (need && !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "indexer top-k workspace %zu < %zu", ws_bytes, need);
  hipError_t e = dsa::launch_indexer_topk(indexer_params(s, q, qs, k, ksc, w, nullptr, s->s_cap), (dsa::Dtype)dt,
                                          s->topk, sample_stride, out, ws, ws_bytes, (hipStream_t)stream, nullptr);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "indexer top-k launch");
}

dsa_status dsa_sparse_mla_attention(const dsa_shape* s, dsa_dtype dt, const void* q, const void* kv,
                                    const int32_t* idx, float sm_scale, void* out, float* lse, void* ws,
                                    size_t ws_bytes, void* stream) {
  dsa_status st = check_mla_shape(s, dt);
  if (st == DSA_OK) st = check_mla_ptrs(s, q, kv, out);
  if (st == DSA_OK) st = check_sm_scale(sm_scale);
  if (st != DSA_OK) return st;
  if (rows_of(s) > 0 && !idx) return fail(DSA_ERR_INVALID_ARG, "topk_indices must be non-NULL");
  const size_t need = mla_ws(s, dt);
  if (ws_bytes < need || (need && !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "sparse MLA workspace %zu < %zu", ws_bytes, need);
  hipError_t e = dsa::launch_sparse_mla(mla_params(s, q, kv, idx, sm_scale, out, lse), (dsa::Dtype)dt, ws,
                                        ws_bytes, (hipStream_t)stream, nullptr);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "sparse MLA launch");
}

dsa_status dsa_sparse_mla_backward(const dsa_shape* s, dsa_dtype dt, const void* q, const void* kv,
                                   const int32_t* idx, float sm_scale, const void* out, const float* lse,
                                   const void* dout, float* dq, float* dkv, void* ws, size_t ws_bytes,
                                   void* stream) {
  dsa_status st = check_mla_shape(s, dt);
  if (st == DSA_OK) st = check_sm_scale(sm_scale);
  if (st != DSA_OK) return st;
  const bool mfma = dsa::mla_bwd_uses_mfma(s->Hm, s->Dc, s->Dr, s->s_cap, (dsa::Dtype)dt);
  if (!mfma && !dsa::mla_bwd_supported(s->Hm, s->Dc, s->Dr, (dsa::Dtype)dt))
    return fail(DSA_ERR_UNSUPPORTED,
                "sparse MLA backward: Hm=%d Dc=%d Dr=%d need Hm <= 64, Dc <= 512, Dc+Dr <= 640 (or bf16 with "
                "Dc=512, Dr=64 and Hm a multiple of 64)",
                s->Hm, s->Dc, s->Dr);
  if (s->s_cap > 0 && (!kv || !dkv)) return fail(DSA_ERR_INVALID_ARG, "kv and dkv must be non-NULL");
  if (rows_of(s) > 0 && (!q || !idx || !out || !lse || !dout || !dq))
    return fail(DSA_ERR_INVALID_ARG, "q, topk_indices, out, lse, dout and dq must be non-NULL");
  const size_t need = mla_bwd_ws(s, dt);
  if (ws_bytes < need || (need && !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "sparse MLA backward workspace %zu < %zu", ws_bytes, need);
  const dsa::MlaBwdParams p{s->B, s->T, s->Hm, s->Dc, s->Dr, s->topk, s->s_cap, q, kv, idx, sm_scale,
                            out, lse, dout, dq, dkv};
  hipError_t e = dsa::launch_sparse_mla_bwd(p, (dsa::Dtype)dt, ws, ws_bytes, (hipStream_t)stream, nullptr);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "sparse MLA backward launch");
}

dsa_status dsa_index_backward(const dsa_shape* s, dsa_dtype dt, const void* q, const float* qs, const void* k,
                              const float* ksc, const float* w, const int32_t* idx, const float* dI, float* dq,
                              float* dk, float* dw, void* ws, size_t ws_bytes, void* stream) {
  dsa_status st = check_indexer_shape(s, dt);
  if (st == DSA_OK) st = check_topk_shape(s);
  if (st != DSA_OK) return st;
  if (!dsa::index_bwd_supported(s->H, s->D, s->Hk))
    return fail(DSA_ERR_UNSUPPORTED, "index backward: H=%d D=%d need H <= 64", s->H, s->D);
  if (rows_of(s) > 0) {
    if (!q || !w || !idx || !dI || !dq || !dw)
      return fail(DSA_ERR_INVALID_ARG, "q, w, topk_indices, dI, dq and dw must be non-NULL");
    if (dt == DSA_FP8_E4M3 && !qs) return fail(DSA_ERR_INVALID_ARG, "fp8 inputs need q_scale and k_scale");
  }
  if (s->s_cap > 0) {
    if (!k || !dk) return fail(DSA_ERR_INVALID_ARG, "k and dk must be non-NULL");
    if (dt == DSA_FP8_E4M3 && !ksc) return fail(DSA_ERR_INVALID_ARG, "fp8 inputs need q_scale and k_scale");
  }
  const size_t need = index_bwd_ws(s, dt);
  if (ws_bytes < need || (need && !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "index backward workspace %zu < %zu", ws_bytes, need);
  const dsa::IndexBwdParams p{s->B, s->T, s->H, s->D, s->Hk, s->topk, s->s_cap, q, qs, k, ksc, w, idx, dI,
                              dq, dk, dw};
  hipError_t e = dsa::launch_index_bwd(p, (dsa::Dtype)dt, ws, ws_bytes, (hipStream_t)stream, nullptr);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "index backward launch");
}

dsa_status dsa_group_forward(const dsa_shape* s, dsa_dtype mla_dtype, int32_t n_layers,
                             const dsa_layer_type* types, const dsa_layer_io* layers, float sm_scale,
                             dsa_topk_cache* cache, uint64_t tag, void* ws, size_t ws_bytes, void* const* events,
                             dsa_group_stats* stats, void* stream) {
  // ---- every check first: a failing call enqueues nothing
  dsa_status st = check_common(s);
  if (st == DSA_OK) st = check_sm_scale(sm_scale);
  if (st != DSA_OK) return st;
  if (n_layers < 0) return fail(DSA_ERR_INVALID_ARG, "n_layers=%d", n_layers);
  if (n_layers > 0 && (!types || !layers)) return fail(DSA_ERR_INVALID_ARG, "indexer_types and layers must be non-NULL");
  if (!cache) return fail(DSA_ERR_INVALID_ARG, "cache handle is NULL");
  if (n_layers > 0) {
    st = check_mla_shape(s, mla_dtype);
    if (st != DSA_OK) return st;
    if (rows_of(s) > 0 && !cache->indices) return fail(DSA_ERR_INVALID_ARG, "cache->indices is NULL");
  }
  for (int l = 0; l < n_layers; ++l) {
    if (types[l] != DSA_FULL && types[l] != DSA_SHARED)
      return fail(DSA_ERR_INVALID_ARG, "layer %d: indexer type %d is neither FULL nor SHARED", l, (int)types[l]);
    const dsa_layer_io& L = layers[l];
    if (types[l] == DSA_FULL) {
      if (!L.index) return fail(DSA_ERR_INVALID_ARG, "layer %d is FULL but has no index inputs", l);
      st = check_indexer_shape(s, L.index->idx_dtype);
      if (st == DSA_OK)
        st = check_indexer_ptrs(s, L.index->idx_dtype, L.index->q, L.index->q_scale, L.index->k, L.index->k_scale,
                                L.index->w);
      if (st != DSA_OK) return fail(st, "layer %d: %s", l, g_last_error.c_str());
    }
    st = check_mla_ptrs(s, L.q, L.kv, L.out);
    if (st != DSA_OK) return fail(st, "layer %d: %s", l, g_last_error.c_str());
  }
  if (n_layers > 0 && types[0] == DSA_SHARED) {
    if (!cache->valid) return fail(DSA_ERR_NO_DONOR, "layer 0 is SHARED and the cache holds no indices from a full layer");
    if (cache->tag != tag || cache->B != s->B || cache->T != s->T || cache->topk != s->topk)
      return fail(DSA_ERR_STALE_CACHE,
                  "cached indices (tag %llu, B=%d T=%d topk=%d) do not belong to this call (tag %llu, B=%d T=%d topk=%d)",
                  (unsigned long long)cache->tag, cache->B, cache->T, cache->topk, (unsigned long long)tag, s->B, s->T,
                  s->topk);
  }
  const size_t need = dsa_workspace_bytes(s, DSA_OP_GROUP);
  const size_t sb = scores_bytes(s);
  if (ws_bytes < need || (need && !ws))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "group workspace %zu < %zu", ws_bytes, need);
  dsa_dtype idx_dtype = DSA_BF16;
  for (int l = 0; l < n_layers; ++l)
    if (types[l] == DSA_FULL) {
      idx_dtype = layers[l].index->idx_dtype;
      break;
    }
  if (stats) {
    if ((s->key_start && !s->key_start_host) || (s->key_end && !s->key_end_host))
      return fail(DSA_ERR_INVALID_ARG,
                  "stats need host copies of the device key ranges (shape->key_start_host / key_end_host)");
    group_counters(s, idx_dtype, mla_dtype, n_layers, types, s->key_start ? s->key_start_host : nullptr,
                   s->key_end ? s->key_end_host : nullptr, stats);
  }

  // ---- enqueue
  hipStream_t strm = (hipStream_t)stream;
  float* scores = static_cast<float*>(ws);
  void* kws = ws ? static_cast<char*>(ws) + sb : nullptr;
  const size_t kws_bytes = ws_bytes - std::min(ws_bytes, sb);
  int launches = 0;
  int last_full = -1;           // last full layer whose top-k was enqueued
  auto rec = [&](int l, int slot) -> hipError_t {
    if (!events) return hipSuccess;
    hipEvent_t ev = static_cast<hipEvent_t>(events[6 * l + slot]);
    return ev ? hipEventRecord(ev, strm) : hipSuccess;
  };
  hipError_t e = hipSuccess;
  for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
    const dsa_layer_io& L = layers[l];
    if (types[l] == DSA_FULL) {
      const dsa_index_io& I = *L.index;
      if ((e = rec(l, 0)) != hipSuccess) break;
      const dsa::IndexerParams ip = indexer_params(s, I.q, I.q_scale, I.k, I.k_scale, I.w, scores, s->s_cap);
      if (group_fuses(s, I.idx_dtype)) {
        last_full = l;  // from here on the indices buffer holds this call's data
        e = dsa::launch_indexer_topk(ip, (dsa::Dtype)I.idx_dtype, s->topk, 0, cache->indices, ws, ws_bytes, strm,
                                     &launches);
        if (e != hipSuccess) break;
        if ((e = rec(l, 1)) != hipSuccess) break;
        if ((e = rec(l, 2)) != hipSuccess) break;
        if ((e = rec(l, 3)) != hipSuccess) break;
      } else {
        e = dsa::launch_indexer(ip, (dsa::Dtype)I.idx_dtype, strm, &launches);
        if (e != hipSuccess) break;
        if ((e = rec(l, 1)) != hipSuccess) break;
        if ((e = rec(l, 2)) != hipSuccess) break;
        last_full = l;  // from here on the indices buffer holds this call's data
        e = dsa::launch_topk(topk_params(s, scores, s->s_cap, cache->indices), kws, kws_bytes, strm, &launches);
        if (e != hipSuccess) break;
        if ((e = rec(l, 3)) != hipSuccess) break;
      }
    }
    if ((e = rec(l, 4)) != hipSuccess) break;
    e = dsa::launch_sparse_mla(mla_params(s, L.q, L.kv, cache->indices, sm_scale, L.out, L.lse),
                               (dsa::Dtype)mla_dtype, kws, kws_bytes, strm, &launches);
    if (e != hipSuccess) break;
    e = rec(l, 5);
  }
  if (stats) stats->n_launches = launches;
  if (last_full >= 0) {
    // the handle describes the indices buffer only once every launch was enqueued
    cache->valid = e == hipSuccess ? 1 : 0;
    if (e == hipSuccess) {
      cache->B = s->B;
      cache->T = s->T;
      cache->topk = s->topk;
      cache->donor_layer = last_full;
      cache->tag = tag;
    }
  }
  return e == hipSuccess ? DSA_OK : hip_fail(e, "group forward");
}

dsa_status dsa_group_forward_noalloc(const dsa_shape* s, dsa_dtype mla_dtype, int32_t n_layers,
                                     const dsa_layer_type* types, const dsa_layer_io* layers, float sm_scale,
                                     dsa_topk_cache* cache, uint64_t tag, void* const* events,
                                     dsa_group_stats* stats, void* stream) {
  dsa_status st = check_common(s);
  if (st != DSA_OK) return st;
  const size_t need = dsa_workspace_bytes(s, DSA_OP_GROUP);
  if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL,
                "this group call needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                "(use dsa_group_forward with a workspace)",
                need, (size_t)DSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && (st = current_scratch(&ws)) != DSA_OK) return st;
  return dsa_group_forward(s, mla_dtype, n_layers, types, layers, sm_scale, cache, tag, ws,
                           need > 0 ? (size_t)DSA_NOALLOC_SCRATCH_BYTES : 0, events, stats, stream);
}

dsa_status dsa_group_stats_compute(const dsa_shape* s, dsa_dtype idx_dtype, dsa_dtype mla_dtype, int32_t n_layers,
                                   const dsa_layer_type* types, const int32_t* ks_h, const int32_t* ke_h,
                                   dsa_group_stats* out) {
  dsa_status st = check_common(s);
  if (st != DSA_OK) return st;
  if (!out || (n_layers > 0 && !types)) return fail(DSA_ERR_INVALID_ARG, "stats and indexer_types must be non-NULL");
  if (!valid_dtype(idx_dtype) || !valid_dtype(mla_dtype)) return fail(DSA_ERR_INVALID_ARG, "unknown dtype");
  group_counters(s, idx_dtype, mla_dtype, n_layers, types, ks_h, ke_h, out);
  return DSA_OK;
}

dsa_status dsa_index_prep(int32_t n, int32_t heads, int32_t D, float rope_theta, dsa_dtype out_dtype,
                          const float* x, const int32_t* pos, const int64_t* rows, int64_t n_rows, void* out,
                          float* out_scale, void* stream) {
  if (n < 0 || heads < 1 || n_rows < 0)
    return fail(DSA_ERR_INVALID_ARG, "n=%d heads=%d n_rows=%lld: need n >= 0, heads >= 1, n_rows >= 0", n, heads,
                (long long)n_rows);
  if (D < 4 || D > 1024 || D % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "D=%d: need D %% 4 == 0, 4 <= D <= 1024", D);
  if (!(rope_theta > 0.f) || !std::isfinite(rope_theta))
    return fail(DSA_ERR_INVALID_ARG, "rope_theta must be a positive finite number (got %g)", (double)rope_theta);
  if (out_dtype != DSA_BF16 && out_dtype != DSA_FP8_E4M3)
    return fail(DSA_ERR_INVALID_ARG, "out_dtype must be DSA_BF16 or DSA_FP8_E4M3 (got %d)", (int)out_dtype);
  if (!rows && n_rows < n) return fail(DSA_ERR_INVALID_ARG, "without rows, n_rows=%lld must be >= n=%d",
                                       (long long)n_rows, n);
  if (n > 0 && (!x || !pos || !out)) return fail(DSA_ERR_INVALID_ARG, "x, pos and out must be non-NULL");
  if (n > 0 && out_dtype == DSA_FP8_E4M3 && !out_scale)
    return fail(DSA_ERR_INVALID_ARG, "fp8 storage needs out_scale");
  const dsa::PrepParams p{n, heads, D, rope_theta, (int)out_dtype, x, pos, rows, n_rows, out, out_scale};
  const hipError_t e = dsa::launch_index_prep(p, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "index prep launch");
}

dsa_status dsa_latent_append(int32_t n, int32_t R, dsa_dtype dtype, const void* latent_new, const int64_t* rows,
                             int64_t n_rows, void* latent_cache, void* stream) {
  if (n < 0 || R < 1 || n_rows < 0)
    return fail(DSA_ERR_INVALID_ARG, "n=%d R=%d n_rows=%lld: need n >= 0, R >= 1, n_rows >= 0", n, R,
                (long long)n_rows);
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "latent dtype must be DSA_F32 or DSA_BF16 (got %d)", (int)dtype);
  const int row_bytes = R * (dtype == DSA_F32 ? 4 : 2);
  if (row_bytes % 16 != 0) return fail(DSA_ERR_UNSUPPORTED, "a latent row of %d bytes is not a multiple of 16", row_bytes);
  if (n > 0 && (!latent_new || !rows || !latent_cache))
    return fail(DSA_ERR_INVALID_ARG, "latent_new, rows and latent_cache must be non-NULL");
  const dsa::LatentAppendParams p{n, row_bytes, latent_new, rows, n_rows, latent_cache};
  const hipError_t e = dsa::launch_latent_append(p, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "latent append launch");
}

}  // extern "C"
