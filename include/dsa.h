/*
 * dsa.h -- C ABI of the MI355X (gfx950) DSA lightning indexer -> top-k -> sparse
 * MLA path with GLM-5.2 cross-layer IndexShare.
 *
 * What the calls compute (the pages describe the method; they print no formula,
 * so the readings are stated where they are used):
 *   GLM-5.2 IndexShare page, section 1 "What DSA does before sharing": for each
 *   query a light indexer scores the prefix tokens, the top-k positions are kept,
 *   and the main attention runs only over them.  Section 2 "What IndexShare
 *   changes" and the table "What is actually shared?": full layers compute and
 *   cache the top-k indices, shared layers reuse the nearest preceding full
 *   layer's indices and still compute their own attention.
 *
 * Conventions for every call:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; tensors are
 *     dense, row-major, in the layouts given below.  Pointers marked "host" are
 *     host memory.  The library keeps no pointer past the call and frees nothing.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *     the call returns without waiting.  Device faults surface at the caller's
 *     next synchronisation.
 *   - All argument checks run on the host before anything is enqueued: a call
 *     that returns an error has enqueued nothing.  No call aborts, exits or
 *     throws; dsa_last_error() gives a thread-local message for the last error.
 *   - Query (b, t) owns a candidate range [key_start[b*T+t], key_end[b*T+t]) of
 *     absolute key positions.  Device code clamps each range to [0, s_cap] so
 *     a bad range cannot address memory outside the tensors; the result for
 *     such a row is the result for the clamped range.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 4

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,         /* null or inconsistent pointer / size / shape */
  DSA_ERR_UNSUPPORTED = 2,         /* valid request this build has no kernel for */
  DSA_ERR_NO_DONOR = 3,            /* a shared layer has no full layer and no cached indices */
  DSA_ERR_STALE_CACHE = 4,         /* cached indices belong to another call (tag/shape) */
  DSA_ERR_WORKSPACE_TOO_SMALL = 5, /* ws_bytes < dsa_workspace_bytes(...) */
  DSA_ERR_HIP = 6                  /* a HIP runtime call failed (message in dsa_last_error) */
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2 /* OCP e4m3fn */ } dsa_dtype;
typedef enum { DSA_FULL = 0, DSA_SHARED = 1 } dsa_layer_type;
typedef enum {
  DSA_OP_INDEXER = 0,
  DSA_OP_TOPK = 1,
  DSA_OP_SPARSE_MLA = 2,
  DSA_OP_GROUP = 3,
  DSA_OP_INDEXER_TOPK = 4,
  DSA_OP_SPARSE_MLA_BWD = 5,
  DSA_OP_INDEX_BWD = 6
} dsa_op;

/* Problem shape (host struct).  Fields a call does not use are ignored. */
typedef struct {
  int32_t B, T;          /* batch items, queries per item (B*T query rows) */
  int64_t s_cap;         /* key capacity per item: index keys and latent rows hold s_cap rows */
  int32_t H, D, Hk;      /* index query heads, index head dim, index key heads (H or 1) */
  int32_t topk;          /* index_topk: width of every topk_indices row */
  int32_t Hm, Dc, Dr;    /* MLA heads, latent rank (value dims), rope dims; a latent row has Dc+Dr values */
  const int32_t* key_start; /* device int32 [B*T], or NULL for 0 */
  const int32_t* key_end;   /* device int32 [B*T] (exclusive), or NULL for s_cap */
  /* Optional HOST copies of key_start / key_end (same layout, NULL = not given).  The
   * kernels never read them; dsa_group_forward needs them only to fill the analytic
   * counters of dsa_group_stats when the device ranges are given. */
  const int32_t* key_start_host;
  const int32_t* key_end_host;
} dsa_shape;

/*
 * Lightning-indexer scores of every candidate key (section 1 of the IndexShare
 * page; reading of the score: the pages name the per-head index q/k and a
 * per-head scalar weight but print no formula):
 *     scores[b,t,s] = sum_h w[b,t,h] * max(0, q~[b,t,h,:] . k~[b,s,g(h),:])
 * for s in [key_start, key_end); g(h) = h when Hk == H, else 0.  q~ and k~ are
 * the stored values, times q_scale / k_scale for fp8.
 *   q       [B,T,H,D]   idx_dtype          q_scale [B,T,H]  fp32 (fp8 only, else NULL)
 *   k       [B,s_cap,Hk,D] idx_dtype       k_scale [B,s_cap,Hk] fp32 (fp8 only)
 *   w       [B,T,H]     fp32
 *   scores  [B,T,ld_scores] fp32, ld_scores >= s_cap; only candidate cells are written.
 * Arithmetic: exact products, fp32 accumulation (MFMA for bf16/fp8 with D == 128).
 * Supported: D % 16 == 0 and D <= 256; H <= 128; Hk in {1, H}.
 */
dsa_status dsa_indexer_scores(const dsa_shape* shape, dsa_dtype idx_dtype,
                              const void* q, const float* q_scale,
                              const void* k, const float* k_scale,
                              const float* w, float* scores, int64_t ld_scores,
                              void* stream);

/*
 * Top-k selection per query row (section 1 of the IndexShare page; the -1 padding
 * follows the Megatron-Bridge pull request's commit that fixes top-k for packed
 * sequences shorter than index_topk).  For each row the topk candidates with the
 * largest score are kept; among equal scores the lower position wins (-0.0 and
 * +0.0 are equal).  The kept absolute positions are written in ascending order.
 * A row with n = key_end - key_start <= topk keeps all n candidates and fills
 * the remaining topk - n slots with -1.  NaN scores give an unspecified (but
 * in-range) selection.
 *   scores        [B,T,ld_scores] fp32 (only the candidate cells are read)
 *   topk_indices  [B,T,topk] int32
 *   workspace     device scratch of ws_bytes >= dsa_workspace_bytes(shape, DSA_OP_TOPK)
 */
dsa_status dsa_topk_select(const dsa_shape* shape, const float* scores, int64_t ld_scores,
                           int32_t* topk_indices, void* workspace, size_t ws_bytes,
                           void* stream);

/*
 * Lightning indexer and top-k in one call (section 1 of the IndexShare page: the
 * indexer scores the prefix and only the top-k positions go on; the DeepSeek-V3.2
 * material names this scan and selection as the long-context cost).  The result is
 * bit-identical to dsa_indexer_scores followed by dsa_topk_select on the same inputs;
 * the arguments are those two calls' (without scores), and topk_indices is written in
 * the same way.
 * Where the shape runs on a kernel with sampling and candidate modes (fp8 with
 * Hk == H, D == 128 and T >= 64; or decode rows, T <= 4, D == 128, H in {16,32,64},
 * bf16 or fp8) and topk <= 4096, the fp32 score matrix is not written:
 *   1. every sample_stride-th key of each row is scored;
 *   2. each row's threshold is the r-th largest of its samples, r = ceil(k/R + y) with
 *      y^2 = 36 (k/R + y) (R = sample_stride, k = topk): about R r keys reach it, six
 *      standard deviations of that count above k;
 *   3. every key is scored again and those at or above the threshold are kept, with
 *      their positions, in a list of up to 12288 per row;
 *   4. a row whose list holds c keys with topk <= c <= 12288 holds every key at or above
 *      its topk-th largest score, and selects from the list (same order and ties);
 *   5. any other row is scored in full into the workspace and selected as by
 *      dsa_topk_select.
 * Other shapes run the two calls back to back through the workspace.
 *   sample_stride  0 for the default (64), else 16 .. 1048576 (DSA_ERR_INVALID_ARG
 *                  otherwise); it changes the time taken, never the result
 *   workspace      ws_bytes >= dsa_workspace_bytes(shape, DSA_OP_INDEXER_TOPK).  Its
 *                  first B*T*s_cap*4 bytes are the [B*T, s_cap] fp32 score buffer of
 *                  step 5: the candidate cells of the rows that fell back are written
 *                  there and nothing else is (so a caller can tell which rows did).
 */
dsa_status dsa_indexer_topk(const dsa_shape* shape, dsa_dtype idx_dtype,
                            const void* q, const float* q_scale,
                            const void* k, const float* k_scale,
                            const float* w, int32_t* topk_indices, int32_t sample_stride,
                            void* workspace, size_t ws_bytes, void* stream);

/*
 * Sparse MLA attention over the selected latent rows (section 1 of the IndexShare
 * page; the latent row of kv_lora_rank 512 + rope 64 = 576 values is in the
 * Megatron-Bridge pull request's commit on the rope-dim parse).  Absorbed form:
 * keys are the whole Dc+Dr row, values its first Dc entries.  For each (b,t,h):
 *     z_j = sm_scale * q[b,t,h,:] . kv[b,idx_j,:],  p = softmax(z),
 *     out[b,t,h,:] = sum_j p_j kv[b,idx_j,:Dc],     lse[b,t,h] = log sum_j exp(z_j)
 * over the entries idx_j of topk_indices[b,t,:] that lie in [0, s_cap); other
 * entries (-1 padding) are skipped.  A row with no valid entry gives out = 0 and
 * lse = -inf.  Each listed entry counts once per occurrence.  sm_scale must be a
 * positive finite number (DSA_ERR_INVALID_ARG otherwise).
 *   q    [B,T,Hm,Dc+Dr] mla_dtype     kv  [B,s_cap,Dc+Dr] mla_dtype
 *   out  [B,T,Hm,Dc]    mla_dtype     lse [B,T,Hm] fp32 or NULL
 * Arithmetic: fp32 softmax and accumulation; bf16 MFMA for bf16 with Dc == 512,
 * Dr == 64 and Hm % 64 == 0, fp32 FMA otherwise.  Supported: mla_dtype F32 or
 * BF16, Dc % 8 == 0, Dr % 8 == 0, Dc+Dr <= 1024, Hm <= 1024.
 */
dsa_status dsa_sparse_mla_attention(const dsa_shape* shape, dsa_dtype mla_dtype,
                                    const void* q, const void* kv,
                                    const int32_t* topk_indices, float sm_scale,
                                    void* out, float* lse,
                                    void* workspace, size_t ws_bytes, void* stream);

/* Cached top-k indices carried between layers and calls (host struct).  The
 * indices buffer is caller-owned device memory [B,T,topk].  The host fields are
 * written at enqueue time; the device contents follow stream order, so a handle
 * belongs to one stream.  This plays the part of the carried indexer state of a
 * scanned layer loop (MaxText pull request, key change 2) and of the per-micro-
 * batch top-k holder (Megatron-Bridge pull request, cross-layer DSA commit). */
typedef struct {
  int32_t* indices;
  int32_t B, T, topk;   /* shape the indices were produced for */
  int32_t valid;        /* 0 = empty */
  int32_t donor_layer;  /* layer index (in the producing call) that wrote them */
  uint64_t tag;         /* caller's tag of the producing call */
} dsa_topk_cache;

/* Index inputs of a full layer (host struct, device pointers; layouts as in
 * dsa_indexer_scores). */
typedef struct {
  dsa_dtype idx_dtype;
  const void* q;
  const float* q_scale;
  const void* k;
  const float* k_scale;
  const float* w;
} dsa_index_io;

/* Per-layer inputs and outputs (host struct, device pointers; layouts as in
 * dsa_sparse_mla_attention).  `index` is required on full layers and ignored on
 * shared ones. */
typedef struct {
  const dsa_index_io* index;
  const void* q;
  const void* kv;
  void* out;
  float* lse;
} dsa_layer_io;

/* Analytic work of a group call (counts, not timings).  Candidate count n of a query =
 * key_end - key_start after clamping to [0, s_cap]; selected rows |J| = min(n, topk). */
typedef struct {
  int32_t n_full, n_shared;
  int32_t n_launches;      /* kernels enqueued by the call (dsa_group_forward only) */
  int32_t n_fused;         /* full layers run as dsa_indexer_topk runs (no score matrix); the
                            * byte counters below still count the score matrix's write and read */
  double indexer_flops;    /* 2*H*D per (query, candidate) pair, per full layer */
  double indexer_bytes;    /* index q, w (+scales), index k of each item's prefix, fp32 scores written */
  double topk_bytes;       /* fp32 scores read + int32 indices written */
  double attn_flops;       /* 2*Hm*(2*Dc+Dr) per (query, selected row), per layer */
  double attn_bytes;       /* gathered latent rows + q read + out written, per layer */
} dsa_group_stats;

/*
 * One IndexShare layer group (section 2 of the IndexShare page and its layer-
 * pattern figure; the list comes from indexer_types as the page's config
 * evidence and implementation checklist ask, not from a fixed layer modulo).
 * For l in 0..n_layers-1:
 *   FULL:   indexer scores -> workspace, top-k -> cache->indices; with s_cap >= 65536
 *           and T >= 64, on shapes that dsa_indexer_topk runs without the score matrix,
 *           as that call does (same indices).
 *   SHARED: the cache's indices are used unchanged (no device work).
 *   both:   sparse MLA with layer l's own q and kv and the current indices.
 * The handle's host fields change only when the call returns: after a successful
 * enqueue of a list with full layers, valid = 1, donor_layer = the last full layer,
 * tag = the call's tag and B, T, topk = the shape's.  If an enqueue fails after a full
 * layer's top-k was enqueued (the indices buffer may then hold partial results),
 * valid = 0; if it fails before that, the handle is left as it was.
 * Errors (checked for the whole list before anything is enqueued):
 *   DSA_ERR_INVALID_ARG  a full layer without `index`, null required pointers;
 *   DSA_ERR_NO_DONOR     the first layer is shared and cache->valid == 0 (a
 *                        pipeline stage must not start on a shared layer without
 *                        its source: Megatron-Bridge pull request, build-time
 *                        stage-start check);
 *   DSA_ERR_STALE_CACHE  the first layer is shared and the cache's tag, B, T or
 *                        topk differ from this call (a stale holder must be
 *                        rejected, not read: same pull request, bshd+recompute
 *                        guard).
 *   events: NULL, or host array of 6*n_layers hipEvent_t; when given, for layer l
 *           events[6l+0/1] bracket the indexer, [6l+2/3] the top-k and [6l+4/5]
 *           the attention kernels (entries of shared layers' indexer/top-k unused;
 *           on a layer that runs as dsa_indexer_topk, [6l+0/1] bracket the whole
 *           indexer -> top-k and [6l+2/3] are recorded together after it).
 *   stats:  NULL, or filled with every field: the analytic counters (the same numbers as
 *           dsa_group_stats_compute, computed before anything is enqueued, so they are
 *           set even when an enqueue fails) and n_launches.  When the shape gives device
 *           key ranges, the counters need their host copies (shape->key_start_host /
 *           key_end_host): a call with stats, a device range and no host copy of it fails
 *           with DSA_ERR_INVALID_ARG and enqueues nothing.
 *   workspace: ws_bytes >= dsa_workspace_bytes(shape, DSA_OP_GROUP).
 */
dsa_status dsa_group_forward(const dsa_shape* shape, dsa_dtype mla_dtype, int32_t n_layers,
                             const dsa_layer_type* indexer_types, /* host [n_layers] */
                             const dsa_layer_io* layers,          /* host [n_layers] */
                             float sm_scale, dsa_topk_cache* cache, uint64_t tag,
                             void* workspace, size_t ws_bytes,
                             void* const* events, dsa_group_stats* stats, void* stream);

/*
 * dsa_group_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and errors as dsa_group_forward; the
 * scratch it needs (scores, top-k histograms, split-attention partials) lives in a
 * device array of DSA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends.  The call allocates nothing.
 *   - A call whose dsa_workspace_bytes(shape, DSA_OP_GROUP) exceeds
 *     DSA_NOALLOC_SCRATCH_BYTES fails with DSA_ERR_WORKSPACE_TOO_SMALL and enqueues
 *     nothing (decode batches of the sizes served here need tens of MiB).
 *   - The scratch is the current device's (hipGetDevice): make the device that owns
 *     the stream and buffers current.  The first call on a device looks its address
 *     up (hipGetSymbolAddress); make that call outside graph capture.
 *   - Every call on one GPU shares that GPU's scratch and the scratch keeps the last
 *     call's contents (no result depends on them).  Calls that overlap on one GPU
 *     (other streams, other threads, or replays of graphs holding such calls) race:
 *     order them on one stream.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dsa_status dsa_group_forward_noalloc(const dsa_shape* shape, dsa_dtype mla_dtype, int32_t n_layers,
                                     const dsa_layer_type* indexer_types, const dsa_layer_io* layers,
                                     float sm_scale, dsa_topk_cache* cache, uint64_t tag,
                                     void* const* events, dsa_group_stats* stats, void* stream);

/* Analytic counters of a group call from host copies of the key ranges (host
 * arrays [B*T]; key_start_host may be NULL for 0, key_end_host NULL for s_cap).
 * Pure host function. */
dsa_status dsa_group_stats_compute(const dsa_shape* shape, dsa_dtype idx_dtype,
                                   dsa_dtype mla_dtype, int32_t n_layers,
                                   const dsa_layer_type* indexer_types,
                                   const int32_t* key_start_host, const int32_t* key_end_host,
                                   dsa_group_stats* out);

/*
 * Backward of dsa_sparse_mla_attention (training with shared indices: a shared layer
 * differentiates through the donor's selection, which is a constant).  The forward is
 * the IndexShare page's section 1 attention over the selected rows; its gradient for
 * an output gradient dout, with P_j = exp(z_j - lse), z_j = sm_scale q.c_j, D = dout.o:
 *   dz_j = P_j (dout.c_j[:Dc] - D),  dq = sm_scale sum_j dz_j c_j,
 *   dkv[row j] += sm_scale dz_j q + [P_j dout, 0]   (summed over heads and queries).
 *   q, kv, topk_indices, sm_scale: as passed to the forward (mla dtype F32 or BF16)
 *   out [B,T,Hm,Dc] (mla dtype), lse [B,T,Hm] fp32: the forward's results
 *   dout [B,T,Hm,Dc] (mla dtype)
 *   dq  [B,T,Hm,Dc+Dr] fp32, overwritten (for fewer than 1024 query tokens each
 *       selection is split over several workgroups that add their shares with fp32
 *       atomics: then dq too is reproducible to fp32 rounding only)
 *   dkv [B,S,Dc+Dr] fp32, overwritten: zeroed by the call, then every selected row
 *       collects its contributions with fp32 atomics (their order is not fixed, so dkv
 *       is reproducible to fp32 rounding, not bit for bit)
 *   workspace  ws_bytes >= dsa_workspace_bytes(shape, DSA_OP_SPARSE_MLA_BWD), device memory
 *       the call may overwrite: nonzero only for bf16 with Dc = 512, Dr = 64 and Hm a
 *       multiple of 64, which runs on the matrix cores.  It holds D per (query, head) and
 *       sm_scale dz per (query, selected slot rounded up to 64, head) in bf16, then either
 *       P and sm_scale dz once more per (query, slot, head) (the latent-row gradient formed
 *       per selected slot), or, when 8 * topk >= s_cap (dense selections: the gradient
 *       formed per 64-row tile of latent rows), an int32 multiplicity per (query, latent
 *       row, s_cap rounded up to 64) and a byte per (query, 64-row tile).  Either way dkv
 *       collects fp32 atomics.
 * Requires Hm <= 64, Dc <= 512, Dc + Dr <= 640, or the matrix-core shape above
 * (DSA_ERR_UNSUPPORTED otherwise); DSA_ERR_INVALID_ARG on NULL pointers or a bad sm_scale;
 * DSA_ERR_WORKSPACE_TOO_SMALL.
 */
dsa_status dsa_sparse_mla_backward(const dsa_shape* shape, dsa_dtype mla_dtype, const void* q, const void* kv,
                                   const int32_t* topk_indices, float sm_scale, const void* out,
                                   const float* lse, const void* dout, float* dq, float* dkv, void* workspace,
                                   size_t ws_bytes, void* stream);

/*
 * Backward of the index score at the selected positions (training the indexer: a loss
 * on the scores of the kept positions, e.g. an auxiliary indexer loss, supplies dI).
 * The score is dsa_indexer_scores' I[t,s] = sum_h w[t,h] max(0, q[t,h].k[s,g(h)]); with
 * s = q[t,h].k[j,g(h)] and the ReLU derivative 0 at 0:
 *   dw[t,h] = sum_j dI_j max(0, s),   dq[t,h] = sum_j dI_j w[t,h] [s > 0] k[j,g(h)],
 *   dk[j,g(h)] += dI_j w[t,h] [s > 0] q[t,h].
 * Gradients are with respect to the dequantised values (fp8 codes times their scales).
 *   q, q_scale, k, k_scale, w: as for dsa_indexer_scores (shape->H, D, Hk, s_cap)
 *   topk_indices [B,T,topk] int32 (slots outside [0, s_cap) are ignored)
 *   dI  [B,T,topk] fp32, the gradient at each slot's position
 *   dq  [B,T,H,D] fp32, dk [B,S,Hk,D] fp32, dw [B,T,H] fp32, all overwritten.
 *   workspace  ws_bytes >= dsa_workspace_bytes(shape, DSA_OP_INDEX_BWD), device memory the
 *       call may overwrite; may be NULL when that is 0.
 * Two paths, chosen from the shape alone:
 *   - dense selections (bf16 or fp8, D == 128, 8 * topk >= s_cap, B*T*s_cap*4 <= 4 GiB):
 *     dI is scattered into a dense [B*T][s_cap] fp32 matrix in the workspace (slots naming
 *     one key add up) and the sums over keys and queries run as matrix-core tile products
 *     (G = dI w [s > 0] entering them as two bf16 terms, so fp32-level rounding); every row
 *     of dq, dk and dw is written once, deterministically;
 *   - otherwise (no workspace): dk is zeroed by the call and collects contributions with
 *     fp32 atomics; for fewer than 1024 query tokens dq and dw do too (reproducible to
 *     fp32 rounding only).
 * Requires H <= 64 (DSA_ERR_UNSUPPORTED otherwise) and the indexer's shape rules;
 * DSA_ERR_INVALID_ARG on NULL pointers; DSA_ERR_WORKSPACE_TOO_SMALL.
 */
dsa_status dsa_index_backward(const dsa_shape* shape, dsa_dtype idx_dtype, const void* q, const float* q_scale,
                              const void* k, const float* k_scale, const float* w, const int32_t* topk_indices,
                              const float* dI, float* dq, float* dk, float* dw, void* workspace,
                              size_t ws_bytes, void* stream);

/*
 * Decode-step preparation of new index vectors (the Megatron-Bridge pull request's
 * commit on the indexer RoPE half swap: the LAST D/2 dims of every index head are
 * rotated; rope_theta = 8e6 in its config fix).  For each vector x[i, h, :] (fp32,
 * before RoPE), rotate-half pairs (j, j + D/4) of the last D/2 dims turn by
 * pos[i] * rope_theta^(-2j/(D/2)) (angle in double precision), the result is rounded
 * to fp32 and stored at row rows[i] (row i when rows is NULL) as
 *   DSA_BF16       round to nearest even, or
 *   DSA_FP8_E4M3   scale = amax/448 (1 if amax is 0), codes e4m3fn(y/scale) rounded to
 *                  nearest even and saturated at 448; the scale goes to out_scale.
 * Serves both the queries of a step (rows NULL) and the append of new keys to the
 * index-key cache (rows = cache rows, e.g. b * s_cap + slot).
 *   x         [n, heads, D] fp32          pos [n] int32 (position in the sequence)
 *   rows      [n] int64 or NULL; rows outside [0, n_rows) are skipped; two entries that
 *             name one row race (the row ends up holding either vector)
 *   out       [n_rows, heads, D] bf16 or e4m3fn codes
 *   out_scale [n_rows, heads] fp32 (fp8 only)
 * Requires D % 4 == 0, 4 <= D <= 1024, rope_theta > 0 finite; NaN inputs give
 * unspecified codes.  DSA_ERR_INVALID_ARG on bad sizes, types or NULL pointers.
 */
dsa_status dsa_index_prep(int32_t n, int32_t heads, int32_t D, float rope_theta, dsa_dtype out_dtype,
                          const float* x, const int32_t* pos, const int64_t* rows, int64_t n_rows,
                          void* out, float* out_scale, void* stream);

/*
 * Append new latent rows (kv_lora_rank + rope = Dc + Dr values, the latent row of the
 * sparse MLA call) of a decode step to the latent cache: latent_new[i, :] is copied to
 * latent_cache[rows[i], :]; rows outside [0, n_rows) are skipped, and two entries
 * that name one row race.
 *   latent_new [n, R], latent_cache [n_rows, R], dtype DSA_F32 or DSA_BF16; a row must
 *   be a multiple of 16 bytes (DSA_ERR_UNSUPPORTED otherwise).
 */
dsa_status dsa_latent_append(int32_t n, int32_t R, dsa_dtype dtype, const void* latent_new,
                             const int64_t* rows, int64_t n_rows, void* latent_cache, void* stream);

/* Device scratch a call needs (bytes, 0 if none).  Pure host function; returns 0
 * for an invalid shape. */
size_t dsa_workspace_bytes(const dsa_shape* shape, dsa_op op);

const char* dsa_status_string(dsa_status status);
const char* dsa_last_error(void);
int dsa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
