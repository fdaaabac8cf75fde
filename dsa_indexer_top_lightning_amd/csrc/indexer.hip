// Lightning-indexer scores on gfx950.
//
//   scores[b,t,s] = sum_h w[b,t,h] * max(0, q~[b,t,h,:] . k~[b,s,g(h),:])
//
// for every candidate key s of query (b,t) (GLM-5.2 IndexShare page, section 1
// "What DSA does before sharing": the indexer scores the prefix tokens of each
// query).  The pages print no formula; the per-head ReLU and scalar head weight
// follow the Megatron-Bridge pull request's naming of the indexer weights
// (per-head index q/k projections and a per-head scalar `weights_proj`).
//
// Kernels (D == 128 unless noted; the launcher picks one per shape):
//  * indexer_fp8_groups: fp8 (OCP e4m3fn) with one key head per query head, T >= 64 (the
//    long-prefix prefill chunk): 128-query x 256-key tiles, copy waves and compute waves, with
//    the sample, candidate and row-mask modes the fused indexer -> top-k uses;
//  * indexer_tile: bf16 or fp8 prefill, T >= 32: 128 x 128 tiles, the copies and the epilogue
//    of the previous head spread over each head's k-steps;
//  * indexer_stream: decode rows (T <= 4): the keys streamed once from HBM on the vector ALUs,
//    with the same modes;
//  * indexer_mfma: the other bf16 / fp8 shapes: 64 x 64 tiles, one head at a time on the matrix
//    cores (v_mfma_f32_32x32x16_bf16, or v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
//    scales) from LDS-staged tiles, then the ReLU * weight reduction in fp32 registers;
//  * indexer_generic: any dtype / D (fp32 inputs), one thread per key, fp32 FMA;
//  * g8_vectors: the head-major per-head vectors indexer_fp8_groups reads inside the fused call.
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// OCP e4m3fn code -> float (exact).
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  const uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float v;
  if (e == 0xF && m == 7) v = __builtin_nanf("");
  else if (e == 0) v = (float)m * 0x1p-9f;
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80) ? -v : v;
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (DT == F32) return static_cast<const float*>(base)[i];
  else if constexpr (DT == BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return e4m3_to_f32(static_cast<const uint8_t*>(base)[i]);
}

// ----------------------------------------------------------------- generic kernel
// grid: x = query row (b*T + t), y = block of 256 key positions.  Dynamic LDS:
// H*D decoded query values (times q_scale) and H weights.
template <int DT>
__global__ __launch_bounds__(256) void indexer_generic(IndexerParams p) {
  extern __shared__ float lds[];
  const int64_t row = blockIdx.x;
  int64_t ks, ke;
  clamp_range(p.key_start, p.key_end, row, p.s_cap, ks, ke);
  const int64_t s = (int64_t)blockIdx.y * 256 + threadIdx.x;
  const int64_t sblk = (int64_t)blockIdx.y * 256;
  if (sblk >= ke || sblk + 256 <= ks) return;  // whole block outside the range
  const int H = p.H, D = p.D, Hk = p.Hk;
  float* qs = lds;
  float* ws = lds + H * D;
  for (int i = threadIdx.x; i < H * D; i += 256) {
    float v = load_elem<DT>(p.q, row * H * D + i);
    if constexpr (DT == FP8) v *= p.q_scale[row * H + i / D];
    qs[i] = v;
  }
  for (int i = threadIdx.x; i < H; i += 256) ws[i] = p.w[row * H + i];
  __syncthreads();
  if (s < ks || s >= ke) return;
  const int64_t b = row / p.T;
  const int64_t krow = (b * p.s_cap + s) * Hk;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) {
    const int g = (Hk == H) ? h : 0;
    const int64_t kb = (krow + g) * D;
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot = fmaf(qs[h * D + d], load_elem<DT>(p.k, kb + d), dot);
    if constexpr (DT == FP8) dot *= p.k_scale[krow + g];
    acc = fmaf(ws[h], fmaxf(dot, 0.f), acc);
  }
  p.scores[row * p.ld + s] = acc;
}

// ----------------------------------------------------------------- MFMA kernel
constexpr int TM = 64;   // queries per tile
constexpr int TN = 64;   // keys per tile
constexpr int HD = 128;  // index head dim handled by the MFMA kernel

template <int DT>
struct MfmaCfg {
  static constexpr int ESZ = (DT == BF16) ? 2 : 1;
  static constexpr int RB = HD * ESZ;        // bytes per row
  static constexpr int RS = RB + 16;         // padded LDS row stride (bank-conflict free b128 reads)
  static constexpr int CHUNKS = RB / 16;     // 16-byte chunks per row
};

// grid: x = key tile, y = query tile, z = batch item.  256 threads = 4 waves,
// wave w computes rows [32*(w&1), +32) x keys [32*(w>>1), +32) of the tile.
// Dynamic LDS: Q tile, K tile, weights [H][TM] (times q_scale for fp8), key scales [Hk][TN].
template <int DT>
__global__ __launch_bounds__(256) void indexer_mfma(IndexerParams p) {
  using C = MfmaCfg<DT>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* qt = smem;
  unsigned char* kt = smem + TM * C::RS;
  float* wl = reinterpret_cast<float*>(smem + (TM + TN) * C::RS);
  float* ksl = wl + p.H * TM;
  __shared__ int32_t rks[TM], rke[TM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * TM;
  const int64_t s0 = (int64_t)blockIdx.x * TN;
  const int H = p.H, Hk = p.Hk, T = p.T;

  // ranges of the tile's rows; skip tiles with no candidate cell
  int live = 0;
  if (tid < TM) {
    const int t = t0 + tid;
    int64_t ks = 0, ke = 0;
    if (t < T) clamp_range(p.key_start, p.key_end, (int64_t)b * T + t, p.s_cap, ks, ke);
    rks[tid] = (int32_t)ks;
    rke[tid] = (int32_t)ke;
    live = (t < T) && (ks < s0 + TN) && (ke > s0) && (ks < ke);
  }
  if (!__syncthreads_or(live)) return;

  // weights (x q_scale) for all heads of the tile's rows; key scales
  for (int i = tid; i < H * TM; i += 256) {
    const int h = i / TM, r = i % TM, t = t0 + r;
    float v = 0.f;
    if (t < T) {
      const int64_t qi = ((int64_t)b * T + t) * H + h;
      v = p.w[qi];
      if constexpr (DT == FP8) v *= p.q_scale[qi];
    }
    wl[i] = v;
  }
  if constexpr (DT == FP8) {
    for (int i = tid; i < Hk * TN; i += 256) {
      const int g = i / TN, c = i % TN;
      const int64_t s = s0 + c;
      ksl[i] = (s < p.s_cap) ? p.k_scale[((int64_t)b * p.s_cap + s) * Hk + g] : 0.f;
    }
  }

  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lg = lane >> 5;
  f32x16 tot;
  for (int r = 0; r < 16; ++r) tot[r] = 0.f;

  const unsigned char* qg = static_cast<const unsigned char*>(p.q);
  const unsigned char* kg = static_cast<const unsigned char*>(p.k);

  for (int h = 0; h < H; ++h) {
    const int g = (Hk == H) ? h : 0;
    // stage Q_h tile and (if it changes) K_g tile
    for (int c = tid; c < TM * C::CHUNKS; c += 256) {
      const int r = c / C::CHUNKS, ch = c % C::CHUNKS, t = t0 + r;
      i32x4 v = {0, 0, 0, 0};
      if (t < T) v = *reinterpret_cast<const i32x4*>(qg + ((((int64_t)b * T + t) * H + h) * HD) * C::ESZ + ch * 16);
      *reinterpret_cast<i32x4*>(qt + r * C::RS + ch * 16) = v;
    }
    if (Hk == H || h == 0) {
      for (int c = tid; c < TN * C::CHUNKS; c += 256) {
        const int r = c / C::CHUNKS, ch = c % C::CHUNKS;
        const int64_t s = s0 + r;
        i32x4 v = {0, 0, 0, 0};
        if (s < p.s_cap) v = *reinterpret_cast<const i32x4*>(kg + ((((int64_t)b * p.s_cap + s) * Hk + g) * HD) * C::ESZ + ch * 16);
        *reinterpret_cast<i32x4*>(kt + r * C::RS + ch * 16) = v;
      }
    }
    __syncthreads();

    f32x16 acc;
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const unsigned char* qrow = qt + (32 * wm + lr) * C::RS;
    const unsigned char* krow = kt + (32 * wn + lr) * C::RS;
    if constexpr (DT == BF16) {
#pragma unroll
      for (int st = 0; st < HD / 16; ++st) {
        const int off = (16 * st + 8 * lg) * 2;
        bf16x8 a = *reinterpret_cast<const bf16x8*>(qrow + off);
        bf16x8 bb = *reinterpret_cast<const bf16x8*>(krow + off);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int st = 0; st < HD / 64; ++st) {
        const int off = 64 * st + 32 * lg;
        i32x8 a, bb;
        i32x4 a0 = *reinterpret_cast<const i32x4*>(qrow + off), a1 = *reinterpret_cast<const i32x4*>(qrow + off + 16);
        i32x4 b0 = *reinterpret_cast<const i32x4*>(krow + off), b1 = *reinterpret_cast<const i32x4*>(krow + off + 16);
        a[0] = a0[0]; a[1] = a0[1]; a[2] = a0[2]; a[3] = a0[3]; a[4] = a1[0]; a[5] = a1[1]; a[6] = a1[2]; a[7] = a1[3];
        bb[0] = b0[0]; bb[1] = b0[1]; bb[2] = b0[2]; bb[3] = b0[3]; bb[4] = b1[0]; bb[5] = b1[1]; bb[6] = b1[2]; bb[7] = b1[3];
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bb, acc, 0, 0, 0, 127, 0, 127);
      }
    }
    // fused ReLU * weight: result row m = 8*(r/4) + 4*lg + r%4, column n = lr
    const float* wrow = wl + h * TM + 32 * wm + 4 * lg;
    float kscale = 1.f;
    if constexpr (DT == FP8) kscale = ksl[g * TN + 32 * wn + lr];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float wv = wrow[8 * (r >> 2) + (r & 3)];
      tot[r] = fmaf(wv, fmaxf(acc[r] * kscale, 0.f), tot[r]);
    }
    __syncthreads();
  }

  const int64_t s = s0 + 32 * wn + lr;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 32 * wm + 8 * (r >> 2) + 4 * lg + (r & 3);
    const int t = t0 + m;
    if (t < T && s >= rks[m] && s < rke[m]) p.scores[((int64_t)b * T + t) * p.ld + s] = tot[r];
  }
}

// ----------------------------------------------------------------- prefill tile kernel
// A workgroup of 8 waves (two per SIMD, so one wave's LDS reads and epilogue run
// under the other's MFMAs) owns a 128-query x 128-key tile of one batch item; wave
// (wm, wn) owns the 64 x 32 block [64wm, +64) x [32wn, +32) (2 MFMA tiles of 32 x 32).  For
// each head the Q_h and K_g tiles, the head weights (and fp8 scales) are gathered
// straight into LDS with global_load_lds into one of two alternating stages, so the
// loads of head h+1 run under the contraction of head h.  Each wave load moves 8
// rows x 128 bytes (whole cache lines); a tile is stored as 128-byte row segments
// whose 16-byte chunks are XOR-permuted by the row, which keeps the fragment reads
// of 16 consecutive rows bank-conflict free.  The ReLU * weight epilogue of head
// h-1 runs while the MFMAs of head h are in flight; the per-row weights and scales
// live in a ring of three LDS stages so that epilogue can still read them.
constexpr int PQ = 128;  // queries per tile
constexpr int PK = 128;  // keys per tile
constexpr int TILE_WAVES = 8;
constexpr int TILE_THREADS = 64 * TILE_WAVES;

template <int DT>
struct TileCfg {
  static constexpr int ESZ = (DT == BF16) ? 2 : 1;
  static constexpr int SEGS = HD * ESZ / 128;      // 128-byte segments per row (2 bf16 / 1 fp8)
  static constexpr int SEG_BYTES = 128 * 128;      // one segment of the 128 rows
  static constexpr int TILE = SEGS * SEG_BYTES;    // 32 KiB bf16, 16 KiB fp8
  static constexpr int STAGE = 2 * TILE;            // Q and K tiles of one head
  // tile stages in flight: copies run NSTAGE - 1 heads ahead of the contraction
  static constexpr int NSTAGE = (DT == BF16) ? 2 : 4;
  static constexpr int NVSTAGE = NSTAGE + 1;        // vector stages (the epilogue lags one head)
  static constexpr int VEC = 128 * 4;               // one fp32 per row
  static constexpr int W_OFF = 0;                   // w          (in a vector stage)
  static constexpr int QS_OFF = VEC;                // q scale    (fp8)
  static constexpr int KS_OFF = 2 * VEC;            // k scale    (fp8)
  static constexpr int VSTAGE = 3 * VEC;
  static constexpr int VBASE = NSTAGE * STAGE;      // the vector stages follow the tile stages
  static constexpr int LDS = NSTAGE * STAGE + NVSTAGE * VSTAGE;
  static constexpr int LOADS = 2 * SEGS * 16;       // wave loads per stage: 2 tiles x segments x 16 row octets
  static constexpr int DMA_PER_WAVE = LOADS / TILE_WAVES;
};

// 16-byte chunk u (0..7) of row r's segment is stored at chunk u ^ tperm(r)
__device__ __forceinline__ int tperm(int r) {
  const int j = (r >> 1) & 7;
  return ((j & 1) << 2) | (j & 2) | ((j >> 2) & 1);
}

// Global-to-LDS copies of the tile kernel, issued as inline asm: written with the
// compiler's builtin they are LDS stores that the compiler cannot tell apart from the
// stage being read, so every later LDS read would wait for all of them (vmcnt(0)) and the
// next head's copies could not run under this head's MFMAs.  They are ordered by the
// memory clobber and waited for explicitly at the head barrier.  M0 (set one wait state
// before the load reads it) holds the LDS address; lane i's data lands at M0 + size * i.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void tile_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void tile_dma4_off(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void tile_dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// Per-workgroup state and steps of indexer_tile (all inlined into the kernel).
template <int DT>
struct TileWork {
  using C = TileCfg<DT>;
  static constexpr int KS = (DT == BF16) ? HD / 16 : HD / 64;  // MFMA k-steps per head
  static constexpr int DPW = C::DMA_PER_WAVE;
  const IndexerParams& p;
  unsigned char* smem;
  int lane, wave, wv, b, t0, H, Hk, T;
  int64_t s0, s_cap;
  int wm, wn, lr, lg;
  uint32_t smem_lds;      // LDS address of smem
  uint32_t dma_off;       // this wave's first tile copy inside a stage (its copies follow 1 KiB apart)
  bool dma_k;             // this wave copies key rows (else query rows)
  const unsigned char* dbase;      // first row of the tile this wave copies from (head 0)
  uint32_t doff[DPW];              // per-lane byte offsets of this wave's copies from dbase
  uint32_t abase, bbase;  // fragment addresses (k-step 0) of this lane's query and key rows in a stage
  const float* vsrc;      // per-row vector (w, q scale or k scale) of head 0 for waves 0..2
  int64_t vstride;        // its step per head
  int vr0, vr1;           // its two rows
  f32x16 acc0[2], acc1[2];  // accumulators of even / odd heads, one per 32-row tile
  f32x16 tot[2];

  // wave copy j of a stage: tile j / (SEGS*16) (0 = Q, 1 = K), segment, row octet; lane i
  // fills row 8*octet + i/8, stored chunk i%8 <- logical chunk (i%8) ^ tperm(row); rows
  // beyond T / s_cap load a valid row (their results are never written)
  __device__ __forceinline__ void setup(const unsigned char* qg, const unsigned char* kg, int64_t qrow, int64_t krow) {
    smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    const int j0 = wv * DPW;
    const int tile = j0 / (C::SEGS * 16);
    dma_k = tile == 1;
    dbase = dma_k ? kg + ((int64_t)b * s_cap + s0) * krow : qg + ((int64_t)b * T + t0) * qrow;
    dma_off = tile * C::TILE + ((j0 / 16) % C::SEGS) * C::SEG_BYTES + (j0 % 16) * 1024;
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int j = j0 + i, seg = (j / 16) % C::SEGS, oct = j % 16;
      const int row = 8 * oct + (lane >> 3);
      const int chunk = (lane & 7) ^ tperm(row);
      // (tile rows are < 128 and a row holds at most 64 heads of 256 bytes: fits 32 bits)
      const int rr = dma_k ? (int)(min<int64_t>(s0 + row, s_cap - 1) - s0) : min(t0 + row, T - 1) - t0;
      doff[i] = (uint32_t)(rr * (dma_k ? krow : qrow) + seg * 128 + chunk * 16);
    }
    // Fragment addresses.  Rows r and r + 32 share tperm(r), and a query row 64wm + 32i + lr
    // and a key row 32wn + lr both have tperm(lr).  With the chunks of a k-step at bits
    // above the lane's own chunk bits, the swizzled byte offset of k-step ks inside a
    // 128-byte segment is the lane's base XOR (32 (bf16) or 64 (fp8)) * ks, plus 16 for the
    // second fp8 chunk.
    const uint32_t sw = DT == BF16 ? 16u * (uint32_t)(lg ^ tperm(lr)) : 16u * (uint32_t)((2 * lg) ^ tperm(lr));
    abase = (uint32_t)(64 * wm + lr) * 128u + sw;
    bbase = (uint32_t)C::TILE + (uint32_t)(32 * wn + lr) * 128u + sw;
    // per-row vectors: wave 0 w, wave 1 q scale, wave 2 k scale (fp8)
    vsrc = nullptr;
    vstride = 0;
    vr0 = vr1 = 0;
    if (wv == 0) {
      vsrc = p.w + (int64_t)b * T * H;
      vstride = 1;
      vr0 = min(t0 + lane, T - 1);
      vr1 = min(t0 + 64 + lane, T - 1);
    } else if (DT == FP8 && wv == 1) {
      vsrc = p.q_scale + (int64_t)b * T * H;
      vstride = 1;
      vr0 = min(t0 + lane, T - 1);
      vr1 = min(t0 + 64 + lane, T - 1);
    } else if (DT == FP8 && wv == 2) {
      vsrc = p.k_scale + (int64_t)b * s_cap * Hk;
      vstride = (Hk == H) ? 1 : 0;
      vr0 = (int)min<int64_t>(s0 + lane, s_cap - 1);
      vr1 = (int)min<int64_t>(s0 + 64 + lane, s_cap - 1);
    }
  }

  // copy i of head h into tile stage st (skipped for key rows of a shared key head)
  __device__ __forceinline__ void copy_part(int i, int h, int st) const {
    const int hh = dma_k ? ((Hk == H) ? h : 0) : h;
    tile_dma16(dbase + (int64_t)hh * HD * C::ESZ, doff[i], smem_lds + st * C::STAGE + dma_off + i * 1024);
  }

  // head h's per-row vectors into vector stage h % NVSTAGE
  __device__ __forceinline__ void copy_vectors(int h) const {
    if (vsrc == nullptr) return;
    const int64_t rs = (wv == 2) ? Hk : H;
    const float* src = vsrc + (int64_t)h * vstride;
    const int off = (wv == 0) ? C::W_OFF : (wv == 1 ? C::QS_OFF : C::KS_OFF);
    const uint32_t dst = smem_lds + C::VBASE + (h % C::NVSTAGE) * C::VSTAGE + off;
    tile_dma4(src + (int64_t)vr0 * rs, dst);
    tile_dma4(src + (int64_t)vr1 * rs, dst + 256);
  }

  // 16-byte fragment of row r, logical chunk c: segment c / 8, stored chunk (c % 8) ^ tperm(r)
  __device__ __forceinline__ const unsigned char* frag(const unsigned char* tile, int r, int c) const {
    return tile + (c >> 3) * C::SEG_BYTES + r * 128 + 16 * ((c & 7) ^ tperm(r));
  }

  // elements [E0, E0 + NE) of the ReLU * weight epilogue of head hh (accumulators `acc`,
  // weights / scales from its vector stage); element e is row tile e / 16, register e % 16
  template <int E0, int NE>
  __device__ __forceinline__ void epilogue_part(const f32x16 (&acc)[2], int hh) {
    const unsigned char* vb = smem + C::VBASE + (hh % C::NVSTAGE) * C::VSTAGE;
    const float* wl = reinterpret_cast<const float*>(vb + C::W_OFF);
    const float* kl = reinterpret_cast<const float*>(vb + C::KS_OFF);
    float kc = 1.f;
    if constexpr (DT == FP8) kc = kl[32 * wn + lr];
#pragma unroll
    for (int e = E0; e < E0 + NE; ++e) {
      const int i = e >> 4, r = e & 15;
      const int row = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * lg + (r & 3);
      const float wv_ = wl[row];  // fp8: already times the query scale
      float v = acc[i][r];
      if constexpr (DT == FP8) v *= kc;
      tot[i][r] = fmaf(wv_, fmaxf(v, 0.f), tot[i][r]);
    }
  }

  // k-step ks of head h's contraction (tile stage st) into `acc`; ab / bb_ are abase /
  // bbase as seen by this head (kept opaque so the compiler forms each address when used)
  __device__ __forceinline__ void kstep(int ks, f32x16 (&acc)[2], int st, uint32_t ab, uint32_t bb_) const {
    const unsigned char* qt = smem + st * C::STAGE;
    const unsigned char* kt = (Hk == H) ? qt : smem;  // a shared key head stays in stage 0
    if constexpr (DT == BF16) {
      const uint32_t x = 32u * (uint32_t)(ks & 3), seg = (uint32_t)(ks >> 2) * C::SEG_BYTES;
      const uint32_t ao = (ab ^ x) + seg, bo = (bb_ ^ x) + seg;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(qt + ao);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(qt + ao + 32 * 128);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(kt + bo);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bv, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bv, acc[1], 0, 0, 0);
    } else {
      const uint32_t x = 64u * (uint32_t)ks;
      const uint32_t ao = ab ^ x, bo = bb_ ^ x;
      i32x8 a[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(qt + (ao + i * 32 * 128));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(qt + ((ao ^ 16u) + i * 32 * 128));
        a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      const i32x4 lo = *reinterpret_cast<const i32x4*>(kt + bo);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(kt + (bo ^ 16u));
      const i32x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], bv, acc[i], 0, 0, 0, 127, 0, 127);
    }
  }

  // copies this wave issues for one head after the first (tile rows, per-row vectors)
  __device__ __forceinline__ int copies_per_head() const {
    return ((!dma_k || Hk == H) ? DPW : 0) + (vsrc != nullptr ? 2 : 0);
  }

  // wait until this wave's copies of head h have landed while the n newer ones may fly
  __device__ __forceinline__ static void wait_copies(int n) {
    switch (n) {
      case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
      case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
      case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
      case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
      case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
  }

  // the k-steps of head h with (COPY) a share of the copies of head hp into stage sp and
  // (EPI) a share of head h-1's epilogue each; straight-line code, so the compiler can
  // interleave the parts
  template <bool COPY, bool EPI>
  __device__ __forceinline__ void body(int h, int hp, int st, int sp, f32x16 (&cur)[2], const f32x16 (&prev)[2],
                                       uint32_t ab, uint32_t bb_) {
    constexpr int CPK = DPW / KS;   // copies per k-step
    constexpr int EPK = 32 / KS;    // epilogue elements per k-step
    static_assert(CPK * KS == DPW && EPK * KS == 32, "copies and epilogue must split evenly over the k-steps");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kstep(ks, cur, st, ab, bb_);
      if constexpr (COPY) {
        if constexpr (DT == BF16 && KS == 8 && CPK == 1) {
          // front-loaded: four copies in each of the first two k-steps, so the last ones have
          // most of this head's k-steps to land before the next head waits for them (spread
          // one per k-step, the last landed about 1,100 cycles into the next head)
          if (ks < 2) {
#pragma unroll
            for (int c = 0; c < 4; ++c) copy_part(4 * ks + c, hp, sp);
          }
        } else {
#pragma unroll
          for (int c = 0; c < CPK; ++c) copy_part(ks * CPK + c, hp, sp);
        }
      }
      if constexpr (EPI) {
        if constexpr (KS == 8) {
          switch (ks) {
            case 0: epilogue_part<0 * EPK, EPK>(prev, h - 1); break;
            case 1: epilogue_part<1 * EPK, EPK>(prev, h - 1); break;
            case 2: epilogue_part<2 * EPK, EPK>(prev, h - 1); break;
            case 3: epilogue_part<3 * EPK, EPK>(prev, h - 1); break;
            case 4: epilogue_part<4 * EPK, EPK>(prev, h - 1); break;
            case 5: epilogue_part<5 * EPK, EPK>(prev, h - 1); break;
            case 6: epilogue_part<6 * EPK, EPK>(prev, h - 1); break;
            default: epilogue_part<7 * EPK, EPK>(prev, h - 1); break;
          }
        } else {
          if (ks == 0) epilogue_part<0, EPK>(prev, h - 1);
          else epilogue_part<EPK, EPK>(prev, h - 1);
        }
      }
    }
  }

  // Head h (tile stage h % NSTAGE): after the barrier, its KS k-steps each carry a share
  // of the copies of head h + NSTAGE - 1 into the stage head h-1 used and a share of head
  // h-1's epilogue, so the copies drain and the epilogue runs while the matrix cores work.
  __device__ __forceinline__ void head(int h, f32x16 (&cur)[2], const f32x16 (&prev)[2]) {
    const int st = h % C::NSTAGE;
    const int hp = h + C::NSTAGE - 1, sp = hp % C::NSTAGE;
    wait_copies(min(C::NSTAGE - 2, H - 1 - h) * copies_per_head());
    // stage st holds head h; stage sp is free (LDS-only barrier: later heads' copies fly on)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const bool next = hp < H;
    const bool copy = next && (!dma_k || Hk == H);  // uniform per wave
    uint32_t ab = abase, bb_ = bbase;
    asm volatile("" : "+v"(ab), "+v"(bb_));
    if constexpr (DT == FP8) {
      // head h's weights times its query scales, in place; its epilogue reads them after
      // the next barrier
      if (wv == 7) {  // a wave that copies no per-row vectors (balances the per-head barrier)
        float* vb = reinterpret_cast<float*>(smem + C::VBASE + (h % C::NVSTAGE) * C::VSTAGE);
        vb[C::W_OFF / 4 + lane] *= vb[C::QS_OFF / 4 + lane];
        vb[C::W_OFF / 4 + 64 + lane] *= vb[C::QS_OFF / 4 + 64 + lane];
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) cur[i][r] = 0.f;
    if (copy) {
      if (h > 0) body<true, true>(h, hp, st, sp, cur, prev, ab, bb_);
      else body<true, false>(h, hp, st, sp, cur, prev, ab, bb_);
    } else {
      if (h > 0) body<false, true>(h, hp, st, sp, cur, prev, ab, bb_);
      else body<false, false>(h, hp, st, sp, cur, prev, ab, bb_);
    }
    if (next) copy_vectors(hp);
  }

  __device__ __forceinline__ void run() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) tot[i][r] = 0.f;
    for (int x = 0; x < C::NSTAGE - 1 && x < H; ++x) {
      if (x == 0 || !dma_k || Hk == H) {
#pragma unroll
        for (int i = 0; i < DPW; ++i) copy_part(i, x, x);
      }
      copy_vectors(x);
    }
    int h = 0;
    for (; h + 1 < H; h += 2) {
      head(h, acc0, acc1);
      head(h + 1, acc1, acc0);
    }
    if (h < H) head(h, acc0, acc1);
    __syncthreads();  // (fp8) the last head's weights were scaled in LDS by wave 1
    if (h < H) epilogue_part<0, 32>(acc0, h);
    else epilogue_part<0, 32>(acc1, H - 1);
  }
};

template <int DT>
__global__ __attribute__((amdgpu_flat_work_group_size(TILE_THREADS, TILE_THREADS), amdgpu_waves_per_eu(2, 2)))
void indexer_tile(IndexerParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int32_t rks[PQ], rke[PQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z;
  int qy = blockIdx.y, kx = blockIdx.x;  // query tile, key tile
  if (gridDim.x == gridDim.y && gridDim.x <= 16384) {
    // A square tile grid (a prefill over its own prefix) is walked lower triangle first
    // (key tile <= query tile: the causal tiles, all the work), then the upper triangle,
    // so that the live tiles are the first blocks dispatched and spread evenly over the
    // compute units instead of piling up on those that the triangle's rows map to.
    const int n = (int)gridDim.x, id = (int)(blockIdx.y * gridDim.x + blockIdx.x), ntri = n * (n + 1) / 2;
    if (id < ntri) {
      int y = (int)((sqrtf(8.f * (float)id + 1.f) - 1.f) * 0.5f);
      while (y * (y + 1) / 2 > id) --y;
      while ((y + 1) * (y + 2) / 2 <= id) ++y;
      qy = y;
      kx = id - y * (y + 1) / 2;
    } else {
      const int j = id - ntri;  // upper triangle, key tile x > query tile y, x-major
      int x = (int)((sqrtf(8.f * (float)j + 1.f) + 1.f) * 0.5f);
      while (x * (x - 1) / 2 > j) --x;
      while ((x + 1) * x / 2 <= j) ++x;
      kx = x;
      qy = j - x * (x - 1) / 2;
    }
  }
  const int t0 = qy * PQ;
  const int64_t s0 = (int64_t)kx * PK;
  const int T = p.T;
  const int64_t s_cap = p.s_cap;

  int live = 0;
  if (tid < PQ) {
    const int t = t0 + tid;
    int64_t ks = 0, ke = 0;
    if (t < T) clamp_range(p.key_start, p.key_end, (int64_t)b * T + t, s_cap, ks, ke);
    rks[tid] = (int32_t)ks;
    rke[tid] = (int32_t)ke;
    live = (t < T) && (ks < s0 + PK) && (ke > s0) && (ks < ke);
  }
  if (!__syncthreads_or(live)) return;

  TileWork<DT> w{p, smem, lane, wave, __builtin_amdgcn_readfirstlane(wave), b, t0, p.H, p.Hk, T, s0, s_cap,
                 wave & 1, wave >> 1, lane & 31, lane >> 5};
  w.setup(static_cast<const unsigned char*>(p.q), static_cast<const unsigned char*>(p.k),
          (int64_t)p.H * HD * TileCfg<DT>::ESZ, (int64_t)p.Hk * HD * TileCfg<DT>::ESZ);
  w.run();

  // write the candidate cells: result row m = 8(r/4) + 4lg + r%4 of tile i, column lr
  const int64_t s = s0 + 32 * w.wn + w.lr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 64 * w.wm + 32 * i + 8 * (r >> 2) + 4 * w.lg + (r & 3);
      const int t = t0 + m;
      if (t < T && s >= rks[m] && s < rke[m]) p.scores[((int64_t)b * T + t) * p.ld + s] = w.tot[i][r];
    }
}

// ----------------------------------------------------------------- fp8 prefill kernel, specialised waves
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// fp8 index q/k with one key head per query head (D = 128).  A workgroup owns a 128-query x
// 256-key tile and has 12 waves, three per SIMD:
//  * 8 compute waves; wave w owns the 64 x 64 block [64 (w >> 2), +64) x [64 (w & 3), +64)
//    (2 x 2 MFMA tiles of 32 x 32).  They form two groups (waves 0-3 and 4-7, one of each on
//    every SIMD): in head h group 0 runs the MFMAs of head h and then its epilogue, group 1
//    the epilogue of head h-1 and then the MFMAs of head h, so on each SIMD one wave feeds the
//    matrix core while the other keeps the vector ALU busy.  They issue no global loads.
//  * 4 copy waves (8-11, one per SIMD) issue every global-to-LDS copy: head h's Q and K rows
//    (128 bytes each) form one 48 KiB LDS stage, three stages are in flight, and the copies
//    run two heads ahead.  A copy waits in the memory pipeline until its data lands, which
//    would stall a wave that also has MFMAs or vector work to issue; here only the copy waves
//    wait.  They also copy each head's per-row and per-key vectors a head early (head-major
//    runs where the caller's workspace holds them, else 4-byte loads and the w * q scale
//    product formed in LDS).
// One barrier per head: after it head h's stage and the per-row vectors of head h+1 are in
// LDS, and the stage of head h-1 is free for head h+2's copies.  In candidate mode the tile's
// sums then go to a row-major copy in the stages, and all 12 waves select its cells (g8_select).
//
// A tile's key rows are shared by the workgroups of an XCD that own its query tiles (four on
// the 128K-prefix chunk), and a copy that misses the L2 takes several heads to land; so one of
// them, the one with the XCD's first query tile, also requests the key rows of head h + PF
// into the L2 (a 4-byte global-to-LDS load per 64 bytes into a scratch word per lane).
//
// Epilogue, two vector operations per cell: the key scale of each column is pre-scaled by
// 2^-E, where 2^E bounds the tile's largest key scale times 2^25, so every positive product
// acc * ks 2^-E lies in (0, 1) (|acc| < 128 * 448^2 < 2^25 for e4m3 codes) and ReLU is the
// clamp of one v_mul_f32; the weighted sum is one fma with w * q scale.  The tile's sums carry
// the factor 2^-E, removed when the scores are written; all the powers of two are exact, so
// each cell is the fp32 number sum over heads of w qs max(acc ks, 0).
constexpr int G8_BM = 128;                           // queries per tile
constexpr int G8_BN = 256;                           // keys per tile
constexpr int G8_CW = 8;                             // compute waves
constexpr int G8_DW = 4;                             // copy waves
constexpr int G8_THREADS = 64 * (G8_CW + G8_DW);
constexpr int G8_NST = 3;                            // tile stages in flight
constexpr int G8_NV = 5;                             // per-row vector slots (heads h-1 .. h+3)
constexpr int G8_PF = 3;                             // L2 requests run this many heads ahead
constexpr int G8_QB = G8_BM * 128;                   // Q rows of one head
constexpr int G8_STAGE = G8_QB + G8_BN * 128;        // + K rows: 48 KiB
constexpr int G8_V_WQS = 0;                          // slot: per copy wave c, w then q scale of rows [32c, +32)
constexpr int G8_V_KC = G8_V_WQS + 2 * G8_BM * 4;    //       k scale [BN]
constexpr int G8_V_WQ = G8_V_KC + G8_BN * 4;         //       w * q scale [BM]
constexpr int G8_VSLOT = G8_V_WQ + G8_BM * 4;
constexpr int G8_VBASE = G8_NST * G8_STAGE;
constexpr int G8_SINK = G8_VBASE + G8_NV * G8_VSLOT;  // 256 B that the L2 requests land in
constexpr int G8_LDS = G8_SINK + 256;
constexpr int G8_CPW = (G8_BM + G8_BN) / 8 / G8_DW;  // 1 KiB tile copies per copy wave per stage (12)
constexpr int G8_VPW = 2;                            // per-row vector loads per copy wave per head
constexpr int G8_L2N = 2;                            // L2 requests per copy wave per head (lead)
constexpr int G8_KMAX_LOADS = 12;                    // key-scale loads in flight per thread (tile maximum)
static_assert(G8_CPW * 8 * G8_DW == G8_BM + G8_BN, "tile copies must split evenly over the copy waves");
static_assert(G8_DW * G8_L2N * 64 * 64 == G8_BN * 128, "L2 requests cover the key rows in 64 B steps");

// wait until at most n of this wave's global loads are in flight (n above 40 waits for all)
__device__ __forceinline__ void g8_wait_loads(int n) {
  switch (n) {
#define G8W(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    G8W(0) G8W(1) G8W(2) G8W(3) G8W(4) G8W(5) G8W(6) G8W(7) G8W(8) G8W(9) G8W(10) G8W(11) G8W(12) G8W(13)
    G8W(14) G8W(15) G8W(16) G8W(17) G8W(18) G8W(19) G8W(20) G8W(21) G8W(22) G8W(23) G8W(24) G8W(25) G8W(26)
    G8W(27) G8W(28) G8W(29) G8W(30) G8W(31) G8W(32) G8W(33) G8W(34) G8W(35) G8W(36) G8W(37) G8W(38) G8W(39)
    G8W(40)
#undef G8W
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}
__device__ __forceinline__ void g8_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The copy waves' part.
struct G8Copy {
  const IndexerParams& p;
  unsigned char* smem;
  uint32_t smem_lds;
  int lane, c, b, t0, H, T;
  int64_t s0, S, kst;                  // first key of the tile, key capacity, key stride (sampling)
  bool lead;                           // this workgroup requests the key rows into the L2
  const unsigned char* cbase[G8_CPW];  // source of copy i for head 0 (uniform)
  uint32_t coff[G8_CPW];               // per-lane byte offset from it
  uint32_t cdst[G8_CPW];               // LDS offset inside a stage (uniform)
  bool tv;                             // head-major vectors (p.ks_t, p.wq_t) for this tile
  const float* kvt;                    // head-major: k scale of key s0, head 0 (uniform)
  const float* wvt;                    //             w * q scale of row t0, head 0 (uniform)
  const float* wqsrc;                  // this lane's w (lanes 0-31) or q scale (32-63) of head 0
  const float* kcbase;                 // k scale of key s0, head 0 (uniform)
  uint32_t kcoff;                      // this lane's byte offset from it
  const unsigned char* l2base;         // key row s0, head 0 (uniform)
  uint32_t l2off[G8_L2N];              // per-lane 64 B steps of key rows [64c, +64)
  int issued;                          // global loads issued so far
  int mark_new, mark_old;              // `issued` after the newest / second-newest tile copies

  __device__ __forceinline__ void setup() {
    smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    const unsigned char* qg = static_cast<const unsigned char*>(p.q);
    const unsigned char* kg = static_cast<const unsigned char*>(p.k);
    const int64_t row_bytes = (int64_t)H * HD;  // bytes per token of q and of k (fp8, Hk == H)
#pragma unroll
    for (int i = 0; i < G8_CPW; ++i) {
      const int j = G8_CPW * c + i;  // copy j of the stage: 16 Q row octets, then 32 K row octets
      const bool isk = j >= G8_BM / 8;
      const int oct = isk ? j - G8_BM / 8 : j;
      const int row = 8 * oct + (lane >> 3);
      const int chunk = (lane & 7) ^ tperm(row);
      // rows past T / S load a valid row; their results are never written
      const int rr = isk ? (int)(min<int64_t>(s0 + kst * row, S - 1) - s0) : min(t0 + row, T - 1) - t0;
      cbase[i] = isk ? kg + ((int64_t)b * S + s0) * row_bytes : qg + ((int64_t)b * T + t0) * row_bytes;
      coff[i] = (uint32_t)(rr * row_bytes + chunk * 16);
      cdst[i] = (uint32_t)((isk ? G8_QB : 0) + oct * 1024);
    }
    // vectors: rows [32c, +32) of w (lanes 0-31) and q scale (lanes 32-63); columns [64c, +64) of k scale
    {
      const int r = min(t0 + 32 * c + (lane & 31), T - 1);  // w and q scale: separate tensors, full addresses
      wqsrc = (lane < 32 ? p.w : p.q_scale) + ((int64_t)b * T + r) * H;
      const int k = (int)(min<int64_t>(s0 + kst * (64 * c + lane), S - 1) - s0);
      kcbase = p.k_scale + ((int64_t)b * S + s0) * H;
      kcoff = (uint32_t)(k * H * 4);
    }
    tv = p.ks_t != nullptr && kst == 1;
    kvt = tv ? p.ks_t + (int64_t)b * H * p.vec_s + s0 : nullptr;
    wvt = tv ? p.wq_t + (int64_t)b * H * p.vec_t + t0 : nullptr;
    l2base = kg + ((int64_t)b * S + s0) * row_bytes;
#pragma unroll
    for (int n = 0; n < G8_L2N; ++n) {
      const int u = 64 * n + lane;  // 0 .. 127: row 64c + u / 2, half u % 2
      const int rr = (int)(min<int64_t>(s0 + kst * (64 * c + (u >> 1)), S - 1) - s0);
      l2off[n] = (uint32_t)(rr * row_bytes + 64 * (u & 1));
    }
    issued = mark_new = mark_old = 0;
  }

  __device__ __forceinline__ void copy_vec(int h) {
    const uint32_t slot = smem_lds + G8_VBASE + (uint32_t)(h % G8_NV) * G8_VSLOT;
    if (tv) {
      // head-major: the tile's 256 key scales are 1 KiB in a row (copy wave 0, one 16-byte
      // load per lane), its 128 row weights 512 B (copy wave 1, lanes 0-31); the vectors are
      // padded to whole tiles, so neither reads past its head's run
      if (c == 0) {
        tile_dma16(kvt + (int64_t)h * p.vec_s, (uint32_t)lane * 16u, slot + G8_V_KC);
        ++issued;
      } else if (c == 1) {
        if (lane < 32) tile_dma16(wvt + (int64_t)h * p.vec_t, (uint32_t)lane * 16u, slot + G8_V_WQ);
        ++issued;
      }
      return;
    }
    tile_dma4(wqsrc + h, slot + G8_V_WQS + 256 * c);
    tile_dma4_off(kcbase + h, kcoff, slot + G8_V_KC + 256 * c);
    issued += G8_VPW;
  }
  __device__ __forceinline__ void copy_tiles(int h) {
    const uint32_t st = smem_lds + (uint32_t)(h % G8_NST) * G8_STAGE;
#pragma unroll
    for (int i = 0; i < G8_CPW; ++i) tile_dma16(cbase[i] + (int64_t)h * HD, coff[i], st + cdst[i]);
    issued += G8_CPW;
    mark_old = mark_new;
    mark_new = issued;
  }
  __device__ __forceinline__ void l2_request(int h) {
#pragma unroll
    for (int n = 0; n < G8_L2N; ++n) tile_dma4_off(l2base + (int64_t)h * HD, l2off[n], smem_lds + G8_SINK);
    issued += G8_L2N;
  }
  // the copies issued so far are those of heads 0 .. min(h + 1, H - 1): head h's are the
  // second-newest or, for the last head, the newest (loads complete in issue order)
  __device__ __forceinline__ void wait_head(int h) const {
    g8_wait_loads(issued - (h + 1 < H ? mark_old : mark_new));
  }
  // w * q scale of head h for rows [32c, +32) (this wave loaded both)
  __device__ __forceinline__ void prep(int h) const {
    if (tv) return;  // the product came with the vectors
    float* v = reinterpret_cast<float*>(smem + G8_VBASE + (h % G8_NV) * G8_VSLOT);
    if (lane < 32) v[G8_V_WQ / 4 + 32 * c + lane] = v[G8_V_WQS / 4 + 64 * c + lane] * v[G8_V_WQS / 4 + 64 * c + 32 + lane];
  }

  __device__ __forceinline__ void run() {
    // prologue: vectors of heads 0..2 and tile copies of heads 0..1, each head's vectors ahead
    // of the copies of the head before it, then L2 requests of heads 2 .. PF-1
    copy_vec(0);
    for (int h = 0; h < min(2, H); ++h) {
      if (h + 1 < H) copy_vec(h + 1);
      copy_tiles(h);
    }
    if (!tv) {
      g8_wait_loads(issued - G8_VPW);  // head 0's vectors
      prep(0);
    }
    if (lead)
      for (int h = 2; h < min(G8_PF, H); ++h) l2_request(h);
    for (int h = 0; h < H; ++h) {
      wait_head(h);                  // head h's tile and head h+1's vectors (issued before it)
      if (h + 1 < H) prep(h + 1);
      g8_barrier();
      if (h + 2 < H) {
        if (h + 3 < H) copy_vec(h + 3);
        copy_tiles(h + 2);
        if (lead && h + G8_PF < H) l2_request(h + G8_PF);
      }
    }
  }
};

// The compute waves' part.
struct G8Math {
  unsigned char* smem;
  int lane, wv, grp, wm, wn, lr, lg, H;
  uint32_t abase, bbase;               // fragment offsets (k-step 0) inside a stage
  float down;                          // 2^-E of the tile
  f32x16 acc[2][2], tot[2][2];

  __device__ __forceinline__ void setup() {
    const uint32_t sw = 16u * (uint32_t)((2 * lg) ^ tperm(lr));
    abase = (uint32_t)(64 * wm + lr) * 128u + sw;
    bbase = (uint32_t)G8_QB + (uint32_t)(64 * wn + lr) * 128u + sw;
  }
  // 32-byte fragment (k-step ks) of the row at `o` (k-step 0 offset) of a stage
  __device__ __forceinline__ static i32x8 frag(const unsigned char* st, uint32_t o, int ks) {
    const uint32_t x = o ^ (64u * (uint32_t)ks);
    const i32x4 lo = *reinterpret_cast<const i32x4*>(st + x);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(st + (x ^ 16u));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // head h's contraction (stage h % NST) into acc
  __device__ __forceinline__ void mfma(int h) {
    const unsigned char* st = smem + (h % G8_NST) * G8_STAGE;
    uint32_t ab = abase, bb_ = bbase;
    asm volatile("" : "+v"(ab), "+v"(bb_));
    const f32x16 zero = {};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const i32x8 b0 = frag(st, bb_, ks), b1 = frag(st, bb_ + 4096u, ks);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const i32x8 a = frag(st, ab + 4096u * i, ks);
        acc[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b0, ks ? acc[i][0] : zero, 0, 0, 0, 127, 0, 127);
        acc[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b1, ks ? acc[i][1] : zero, 0, 0, 0, 127, 0, 127);
      }
    }
  }
  // epilogue of head h: tot += (w qs) * clamp(acc * ks 2^-E); result row 8(r/4) + 4lg + r%4
  __device__ __forceinline__ void epilogue(int h) {
    const float* v = reinterpret_cast<const float*>(smem + G8_VBASE + (h % G8_NV) * G8_VSLOT);
    float kc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) kc[j] = v[G8_V_KC / 4 + 64 * wn + 32 * j + lr] * down;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float4 w4 = *reinterpret_cast<const float4*>(v + G8_V_WQ / 4 + 64 * wm + 32 * i + 8 * rq + 4 * lg);
        const float wr[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rq + e;
            tot[i][j][r] = fmaf(wr[e], __builtin_amdgcn_fmed3f(acc[i][j][r] * kc[j], 0.f, 1.f), tot[i][j][r]);
          }
      }
  }
  __device__ __forceinline__ void run() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) tot[i][j][r] = 0.f;
    if (grp == 0) {
      for (int h = 0; h < H; ++h) {
        g8_barrier();
        mfma(h);
        epilogue(h);
      }
    } else {
      for (int h = 0; h < H; ++h) {
        g8_barrier();
        if (h > 0) epilogue(h - 1);
        mfma(h);
      }
      epilogue(H - 1);
    }
  }
};

// MODE: G8_SCORES (every key, scores stored), G8_SAMPLES (keys kstride * i, stored at column i),
// G8_CANDIDATES (every key, cells reaching the row's threshold appended to its list)
enum G8Mode : int { G8_SCORES = 0, G8_SAMPLES = 1, G8_CANDIDATES = 2 };

struct G8Shared {
  int32_t rks[G8_BM], rke[G8_BM];  // each row's key range (absolute; empty for masked rows)
  uint32_t lkey[G8_BM];            // candidate mode: each row's threshold (see below)
  float wmax[G8_CW + G8_DW];
};

// Candidate selection of a tile, by all 12 waves over the row-major LDS copy of its scores
// ([128][G8_SROW] fp32, scores times 2^E): wave v takes rows v, v + 12, ...; a row's 256
// columns are 4 per lane.  Pass 1 counts each row's cells at or above its threshold (inside
// its range); lane k of the wave then reserves the slots of its k-th row with one atomic for
// all of the wave's rows; pass 2 writes the cells to them (slots past cap are dropped: the
// count still records them, and such a row falls back).
constexpr int G8_SROW = G8_BN + 8;  // the +8 words put rows 4 apart 32 banks apart
static_assert(G8_BM * G8_SROW * 4 <= G8_VBASE, "the row-major tile fits the stages");
__device__ __forceinline__ void g8_select(const IndexerParams& p, unsigned char* smem, const G8Shared& sh, int b,
                                          int t0, int64_t s0, float up, bool all_in, int wv, int lane) {
  constexpr int NW = G8_CW + G8_DW;
  const float* tl = reinterpret_cast<const float*>(smem);
  const int T = p.T;
  auto takes = [&](int m, bool (&tk)[4]) {
    const float4 x = *reinterpret_cast<const float4*>(tl + m * G8_SROW + 4 * lane);
    const float xv[4] = {x.x, x.y, x.z, x.w};
    const uint32_t lk = sh.lkey[m];
    const int64_t rks = sh.rks[m], rke = sh.rke[m];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t v = __float_as_uint(xv[u]);
      const uint32_t key = v ^ (uint32_t)(((int32_t)v >> 31) | (int32_t)0x80000000);
      const int64_t s = s0 + 4 * lane + u;
      tk[u] = key >= lk && (all_in || (s >= rks && s < rke));
    }
    return x;
  };
  uint32_t mycnt = 0u;
  int k = 0;
  for (int m = wv; m < G8_BM; m += NW, ++k) {
    bool tk[4];
    (void)takes(m, tk);
    uint32_t c = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) c += (uint32_t)__popcll(__ballot(tk[u]));
    mycnt = lane == k ? c : mycnt;
  }
  uint32_t base = 0u;
  if (mycnt) base = (uint32_t)atomicAdd(p.cand_cnt + (int64_t)b * T + t0 + wv + NW * lane, (int32_t)mycnt);
  // a plain-register copy of the atomics' results (read from their destination, each read
  // below would also wait for every candidate store before it)
  uint32_t slots;
  asm volatile("v_mov_b32 %0, %1" : "=v"(slots) : "v"(base));
  unsigned char* lpos = reinterpret_cast<unsigned char*>(p.cand_pos + ((int64_t)b * T + t0) * p.cap);
  unsigned char* lval = reinterpret_cast<unsigned char*>(p.cand_val + ((int64_t)b * T + t0) * p.cap);
  const uint32_t cap = (uint32_t)p.cap;
  k = 0;
  for (int m = wv; m < G8_BM; m += NW, ++k) {
    bool tk[4];
    const float4 x = takes(m, tk);
    const float xv[4] = {x.x, x.y, x.z, x.w};
    uint64_t bal[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) bal[u] = __ballot(tk[u]);
    if ((bal[0] | bal[1] | bal[2] | bal[3]) == 0) continue;
    uint32_t slot = __builtin_amdgcn_readlane(slots, k);
    const uint32_t roff = (uint32_t)m * cap;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (tk[u]) {
        const uint32_t sl = slot + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[u] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[u], 0u));
        if (sl < cap) {
          const uint32_t at = (roff + sl) * 4u;
          *reinterpret_cast<int32_t*>(lpos + at) = (int32_t)(s0 + 4 * lane + u);
          *reinterpret_cast<float*>(lval + at) = xv[u];
        }
      }
      slot += (uint32_t)__popcll(bal[u]);
    }
  }
}

// One tile: query tile qy (rows t0 = 128 qy ..), key tile kx, batch item b.  Every wave
// returns from it (the copy waves once their loads have landed).
template <int MODE>
__device__ __forceinline__ void g8_tile(const IndexerParams& p, unsigned char* smem, G8Shared& sh, int b, int qy,
                                        int kx, bool lead) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = qy * G8_BM;
  const int64_t kst = MODE == G8_SAMPLES ? p.kstride : 1;  // key stride
  const int64_t s0 = (int64_t)kx * G8_BN * kst;  // first key of the tile; column i is key s0 + kst i
  const int T = p.T;
  const int64_t S = p.s_cap;

  int live = 0, inside = 1;
  if (tid < G8_BM) {
    const int t = t0 + tid;
    int64_t ks = 0, ke = 0;
    if (t < T && (!p.row_mask || p.row_mask[(int64_t)b * T + t]))
      clamp_range(p.key_start, p.key_end, (int64_t)b * T + t, S, ks, ke);
    sh.rks[tid] = (int32_t)ks;  // masked rows and rows past T get the empty range
    sh.rke[tid] = (int32_t)ke;
    live = (ks < s0 + G8_BN * kst) && (ke > s0) && (ks < ke);
    if (MODE == G8_CANDIDATES) {
      inside = ks <= s0 && ke >= s0 + G8_BN;
      // The epilogue compares keys that do not fold -0.0 onto +0.0 (u ^ 0x80000000 or ~u); a
      // threshold of +0.0's key is lowered by one, to -0.0's: the same cells pass as with folding.
      const uint32_t lk = ks < ke ? p.lkey[(int64_t)b * T + t] : 0u;
      sh.lkey[tid] = lk == 0x80000000u ? 0x7fffffffu : lk;
    }
  }
  if (!__syncthreads_or(live)) return;
  const bool all_in = MODE == G8_CANDIDATES && __syncthreads_and(inside);

  // 2^E bounds the tile's largest key scale (all heads) times 2^25
  int tile_e;
  {
    const float* ksrc = p.k_scale + ((int64_t)b * S + s0) * p.H;
    const int ncol = (int)min<int64_t>(G8_BN, (S - s0 + kst - 1) / kst);  // columns inside the prefix
    // (every load of a round is issued before any is waited for: one loop step per load made
    // each wait for the one before, a dozen global round trips per tile)
    float m = 0.f;
    const int n = ncol * p.H;
    for (int i0 = tid; i0 < n; i0 += G8_KMAX_LOADS * G8_THREADS) {
      float v[G8_KMAX_LOADS];
#pragma unroll
      for (int u = 0; u < G8_KMAX_LOADS; ++u) {
        const int i = i0 + u * G8_THREADS;
        v[u] = i < n ? (MODE != G8_SAMPLES ? ksrc[i] : ksrc[(i / p.H) * kst * p.H + i % p.H]) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < G8_KMAX_LOADS; ++u) m = fmaxf(m, v[u]);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (lane == 0) sh.wmax[wave] = m;
    __syncthreads();
    m = sh.wmax[0];
#pragma unroll
    for (int i = 1; i < G8_CW + G8_DW; ++i) m = fmaxf(m, sh.wmax[i]);
    int x = 0;
    (void)frexpf(m, &x);  // m < 2^x
    tile_e = 25 + x;
  }
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform, so the role branches are too
  const float up = ldexpf(1.f, tile_e);
  if (wv >= G8_CW) {
    G8Copy cw{p, smem, 0u, lane, wv - G8_CW, b, t0, p.H, T, s0, S, kst, lead};
    cw.setup();
    cw.run();  // every load it issued has landed (the last head waits for all)
    if constexpr (MODE == G8_CANDIDATES) {
      g8_barrier();  // every product of the tile is done: the stages are free
      g8_barrier();  // the compute waves' sums are in LDS
      g8_select(p, smem, sh, b, t0, s0, up, all_in, wv, lane);
    }
    return;
  }
  G8Math w{smem, lane, wv, wv >> 2, wv >> 2, wv & 3, lane & 31, lane >> 5, p.H};
  w.down = ldexpf(1.f, -tile_e);
  w.setup();
  w.run();
  if constexpr (MODE == G8_CANDIDATES) {
    // the scores (times 2^E, exactly the stored values) into the tile's row-major LDS copy
    g8_barrier();
    float* tl = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 64 * w.wm + 32 * i + 8 * (r >> 2) + 4 * w.lg + (r & 3);
#pragma unroll
        for (int j = 0; j < 2; ++j) tl[m * G8_SROW + 64 * w.wn + 32 * j + w.lr] = w.tot[i][j][r] * up;
      }
    g8_barrier();
    g8_select(p, smem, sh, b, t0, s0, up, all_in, wv, lane);
    return;
  }

  // the wave's cells: row 64wm + 32i + 8(r/4) + 4lg + r%4, column 64wn + 32j + lr (key s0 + kst *
  // column); the sums carry 2^-E
  {
    float* dst = p.scores + ((int64_t)b * T + t0) * p.ld + (int64_t)kx * G8_BN;  // row t0, column 0 of the tile
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = 64 * w.wn + 32 * j + w.lr;  // column of the tile: key s0 + kst * c
      const int64_t s = s0 + kst * c;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 64 * w.wm + 32 * i + 8 * (r >> 2) + 4 * w.lg + (r & 3);
          if (s >= sh.rks[m] && s < sh.rke[m]) dst[(int64_t)m * p.ld + c] = w.tot[i][j][r] * up;
        }
    }
  }
}

constexpr int G8_QWORDS = 64;  // query-tile bits of the walking variant (up to 2048 query tiles)

// grid (tiles, B).  QLOOP = false: block x is one tile (query-tile order as below).  QLOOP =
// true: block x is key tile x and walks every query tile, skipping those without live rows
// (for a row mask that leaves few rows: a tile-per-block grid would spend its time starting
// and ending blocks).
template <int MODE, bool QLOOP>
__global__ __attribute__((amdgpu_flat_work_group_size(G8_THREADS, G8_THREADS), amdgpu_waves_per_eu(3, 3)))
void indexer_fp8_groups(IndexerParams p, int nq, int nk, int xcd_order) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ G8Shared sh;
  const int b = blockIdx.y;
  const int bid = blockIdx.x;
  if constexpr (QLOOP) {
    // the query tiles that hold a row of the mask (one bit each; nq <= 32 G8_QWORDS)
    __shared__ uint32_t qbits[G8_QWORDS];
    const int tid = threadIdx.x;
    for (int i = tid; i < G8_QWORDS; i += G8_THREADS) qbits[i] = 0u;
    __syncthreads();
    const int32_t* mrow = p.row_mask + (int64_t)b * p.T;
    for (int r0 = 0; r0 < p.T; r0 += 8 * G8_THREADS) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = r0 + u * G8_THREADS + tid;
        v[u] = t < p.T ? mrow[t] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = (r0 + u * G8_THREADS + tid) / G8_BM;
        if (v[u]) atomicOr(&qbits[q >> 5], 1u << (q & 31));
      }
    }
    __syncthreads();
    for (int qy = 0; qy < nq; ++qy) {
      if (!((qbits[qy >> 5] >> (qy & 31)) & 1u)) continue;
      g8_tile<MODE>(p, smem, sh, b, qy, bid, false);
      __syncthreads();  // the next tile reuses every LDS buffer
    }
  } else {
    int qy, kx;
    if (xcd_order) {
      // Workgroups are dispatched to the 8 XCDs in turn (block i to XCD i % 8).  Each XCD owns
      // nq / 8 query tiles and sweeps the key tiles in order, so its query tiles stay in its L2
      // and the workgroups of an XCD that share a key tile read it at about the same time.
      const int per = nq / 8, xcd = bid % 8, slot = bid / 8;
      qy = xcd * per + slot % per;
      kx = slot / per;
    } else {
      qy = bid % nq;
      kx = bid / nq;
    }
    g8_tile<MODE>(p, smem, sh, b, qy, kx, xcd_order && qy % (nq / 8) == 0);
  }
}
#pragma clang diagnostic pop

// Head-major copies of the fp8 tile kernel's per-head vectors: ks_t[b][h][s] = k_scale[b][s][h]
// and wq_t[b][h][t] = w[b][t][h] * q_scale[b][t][h] (the product the kernel forms otherwise),
// zero in the padding past s_cap and T.  Block x < nks transposes keys [64x, +64) of batch item
// y, the others rows [64 (x - nks), +64), through an LDS tile (H <= 128).
constexpr int GV_N = 64;
__global__ __launch_bounds__(256) void g8_vectors(IndexerParams p, float* ks_t, float* wq_t, int nks) {
  __shared__ float tile[GV_N][129];
  const int b = blockIdx.y, H = p.H, tid = threadIdx.x;
  const bool keys = (int)blockIdx.x < nks;
  const int64_t n = keys ? p.s_cap : p.T;       // valid columns
  const int64_t ld = keys ? p.vec_s : p.vec_t;  // padded columns
  const int64_t c0 = (int64_t)(keys ? blockIdx.x : blockIdx.x - nks) * GV_N;
  // eight elements per thread in flight: every load of a round before any is used (clamped
  // in-bounds addresses; the values past n are replaced by 0 afterwards)
  const int64_t last = (int64_t)b * n * H + n * H - 1;  // the item's last element
  for (int i0 = tid; i0 < GV_N * H; i0 += 8 * 256) {
    float x[8], y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + 256 * u;
      const int64_t o = min(((int64_t)b * n + c0 + i / H) * H + i % H, last);
      x[u] = keys ? p.k_scale[o] : p.w[o];
      y[u] = keys ? 1.f : p.q_scale[o];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + 256 * u;
      if (i < GV_N * H) tile[i / H][i % H] = c0 + i / H < n ? (keys ? x[u] : x[u] * y[u]) : 0.f;
    }
  }
  __syncthreads();
  float* dst = keys ? ks_t : wq_t;
  for (int i = tid; i < GV_N * H; i += 256) {
    const int h = i / GV_N, r = i % GV_N;
    if (c0 + r < ld) dst[((int64_t)b * H + h) * ld + c0 + r] = tile[r][h];
  }
}

// ----------------------------------------------------------------- decode streaming kernel
// Few queries per batch item (decode): the work is one pass over the item's index
// keys, so this kernel streams them from HBM with whole-row 16-byte loads and does
// the products on the vector ALUs (the matrix cores would idle on one query row).
// A key row holds all Hk heads (Hk*D contiguous values); lane l owns head l / LPH,
// elements (l % LPH) * D/LPH .. +D/LPH of it (LPH = 64 / H lanes per head), the
// query slice stays in registers, per-head dots are completed by lane shuffles,
// then ReLU * weight and a shuffle reduction over the heads give the score.
// grid: x = block of 64 keys (or samples), y = query row.  256 threads: wave w takes keys
// w, w+4, ...  With sampling, column c of the row is key kstride * c; in candidate mode
// lane 0 appends each key whose order key reaches the row's threshold.
template <int DT, int LPH, int MODE>
__global__ __launch_bounds__(256) void indexer_stream(IndexerParams p) {
  constexpr int H = 64 / LPH;
  constexpr int EPL = HD / LPH;                 // elements per lane
  constexpr int ESZ = (DT == BF16) ? 2 : 1;
  constexpr int BYTES = EPL * ESZ;              // bytes per lane per key
  constexpr int LOADS = BYTES / 16;
  static_assert(BYTES % 16 == 0, "lane slice must be whole 16-byte loads");
  constexpr int KPB = 64;                       // keys per workgroup

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.y;
  if (p.row_mask && !p.row_mask[row]) return;
  int64_t ks, ke;
  clamp_range(p.key_start, p.key_end, row, p.s_cap, ks, ke);
  const int64_t kst = MODE == G8_SAMPLES ? p.kstride : 1;
  const int64_t sblk = (int64_t)blockIdx.x * KPB;  // first column of the block
  if (sblk * kst >= ke || (sblk + KPB - 1) * kst < ks) return;
  const uint32_t lk = MODE == G8_CANDIDATES ? p.lkey[row] : 0u;
  const int64_t b = row / p.T;
  const int Hk = p.Hk;
  const int h = lane / LPH, part = lane % LPH;

  // query slice (decoded, times the fp8 query scale) and head weight
  float q[EPL];
  {
    const int64_t qo = (row * H + h) * HD + part * EPL;
    if constexpr (DT == BF16) {
      const uint16_t* qb = static_cast<const uint16_t*>(p.q) + qo;
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[e] = __uint_as_float((uint32_t)qb[e] << 16);
    } else {
      const uint8_t* qb = static_cast<const uint8_t*>(p.q) + qo;
      const float qs = p.q_scale[row * H + h];
#pragma unroll
      for (int e = 0; e < EPL; e += 2) {
        const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((uint32_t)qb[e] | ((uint32_t)qb[e + 1] << 8), false);
        q[e] = v[0] * qs;
        q[e + 1] = v[1] * qs;
      }
    }
  }
  const float wh = p.w[row * H + h];
  const int g = (Hk == H) ? h : 0;
  const unsigned char* kg = static_cast<const unsigned char*>(p.k);
  const int64_t krow = (int64_t)Hk * HD * ESZ;
  __shared__ float sv[KPB];  // the block's scores, stored by one wave at the end

  for (int j = wave; j < KPB; j += 4) {
    const int64_t col = sblk + j;
    const int64_t s = col * kst;
    if (s < ks || s >= ke) continue;  // the whole wave takes the same branch
    const unsigned char* src = kg + (b * p.s_cap + s) * krow + (int64_t)g * HD * ESZ + part * BYTES;
    i32x4 raw[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) raw[u] = *reinterpret_cast<const i32x4*>(src + 16 * u);
    float dot = 0.f;
    if constexpr (DT == BF16) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t kk = (uint32_t)raw[u][e];
          dot = fmaf(q[8 * u + 2 * e], __uint_as_float(kk << 16), dot);
          dot = fmaf(q[8 * u + 2 * e + 1], __uint_as_float(kk & 0xffff0000u), dot);
        }
    } else {
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t kk = (uint32_t)raw[u][e];
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(kk, false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(kk, true);
          dot = fmaf(q[16 * u + 4 * e], lo[0], dot);
          dot = fmaf(q[16 * u + 4 * e + 1], lo[1], dot);
          dot = fmaf(q[16 * u + 4 * e + 2], hi[0], dot);
          dot = fmaf(q[16 * u + 4 * e + 3], hi[1], dot);
        }
      dot *= p.k_scale[(b * p.s_cap + s) * Hk + g];
    }
#pragma unroll
    for (int off = 1; off < LPH; off <<= 1) dot += __shfl_xor(dot, off, 64);
    float v = (part == 0) ? wh * fmaxf(dot, 0.f) : 0.f;
#pragma unroll
    for (int off = LPH; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) {
      if constexpr (MODE != G8_CANDIDATES) {
        sv[j] = v;
      } else if (order_key(v) >= lk) {
        const int32_t slot = atomicAdd(p.cand_cnt + row, 1);
        if (slot < p.cap) {
          p.cand_pos[row * p.cap + slot] = (int32_t)s;
          p.cand_val[row * p.cap + slot] = v;
        }
      }
    }
  }
  if constexpr (MODE != G8_CANDIDATES) {
    // one 256-byte store per block instead of one 4-byte store per key
    __syncthreads();
    const int64_t col = sblk + lane;
    if (wave == 0 && col * kst >= ks && col * kst < ke) p.scores[row * p.ld + col] = sv[lane];
  }
}

// one allowance record per launch site (each site launches one kernel)
#define DSA_ALLOW_LDS(kernel, bytes)                                                   \
  [&]() -> hipError_t {                                                                \
    static std::atomic<size_t> high{0};                                                \
    return allow_dynamic_lds(reinterpret_cast<const void*>(&(kernel)), (bytes), high); \
  }()

}  // namespace

namespace {
// the fp8 tile kernel with one key head per query head (prefill)
bool g8_path(const IndexerParams& p, Dtype dt) {
  if (!(dt == FP8 && p.D == HD && p.Hk == p.H && p.T >= 64 && p.B <= 65535)) return false;
  const int64_t nq = (p.T + G8_BM - 1) / G8_BM;
  const int64_t nk = ((p.s_cap + p.kstride - 1) / p.kstride + G8_BN - 1) / G8_BN;
  return nq * nk <= INT32_MAX;
}
template <int DT, int MODE>
void launch_stream_dm(const IndexerParams& p, dim3 grid, hipStream_t st) {
  if (p.H == 16) hipLaunchKernelGGL((indexer_stream<DT, 4, MODE>), grid, dim3(256), 0, st, p);
  else if (p.H == 32) hipLaunchKernelGGL((indexer_stream<DT, 2, MODE>), grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((indexer_stream<DT, 1, MODE>), grid, dim3(256), 0, st, p);
}
template <int DT>
void launch_stream_d(const IndexerParams& p, int mode, dim3 grid, hipStream_t st) {
  if (mode == G8_CANDIDATES) launch_stream_dm<DT, G8_CANDIDATES>(p, grid, st);
  else if (mode == G8_SAMPLES) launch_stream_dm<DT, G8_SAMPLES>(p, grid, st);
  else launch_stream_dm<DT, G8_SCORES>(p, grid, st);
}
void launch_stream(const IndexerParams& p, Dtype dt, int mode, dim3 grid, hipStream_t st) {
  if (dt == BF16) launch_stream_d<BF16>(p, mode, grid, st);
  else launch_stream_d<FP8>(p, mode, grid, st);
}
// the decode stream kernel
bool stream_path(const IndexerParams& p, Dtype dt) {
  return (dt == BF16 || dt == FP8) && p.D == HD && p.T <= 4 && (int64_t)p.B * p.T <= 65535 &&
         (p.H == 16 || p.H == 32 || p.H == 64) && (p.s_cap + p.kstride - 1) / p.kstride / 64 < INT32_MAX;
}
}  // namespace

bool indexer_modes_supported(const IndexerParams& p, Dtype dt) { return g8_path(p, dt) || stream_path(p, dt); }

namespace {
int64_t vec_cols_s(int64_t s_cap) { return (s_cap + G8_BN - 1) / G8_BN * G8_BN; }
int64_t vec_cols_t(int64_t T) { return (T + G8_BM - 1) / G8_BM * G8_BM; }
size_t al256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

size_t indexer_vectors_bytes(int B, int T, int H, int D, int Hk, int64_t s_cap, Dtype dt) {
  IndexerParams p{};
  p.B = B; p.T = T; p.H = H; p.D = D; p.Hk = Hk; p.s_cap = s_cap; p.kstride = 1;
  if (!g8_path(p, dt) || H > 128 || s_cap == 0) return 0;
  return al256((size_t)B * H * vec_cols_s(s_cap) * 4) + al256((size_t)B * H * vec_cols_t(T) * 4);
}

hipError_t launch_indexer_vectors(IndexerParams& p, Dtype dt, void* dst, hipStream_t st, int* n_launches) {
  if (!dst || indexer_vectors_bytes(p.B, p.T, p.H, p.D, p.Hk, p.s_cap, dt) == 0) return hipSuccess;
  p.vec_s = vec_cols_s(p.s_cap);
  p.vec_t = vec_cols_t(p.T);
  float* ks = static_cast<float*>(dst);
  float* wq = reinterpret_cast<float*>(static_cast<char*>(dst) + al256((size_t)p.B * p.H * p.vec_s * 4));
  const int nks = (int)(p.vec_s / GV_N), nts = (int)(p.vec_t / GV_N);
  hipLaunchKernelGGL(g8_vectors, dim3((unsigned)(nks + nts), (unsigned)p.B), dim3(256), 0, st, p, ks, wq, nks);
  if (n_launches) ++*n_launches;
  p.ks_t = ks;
  p.wq_t = wq;
  return hipGetLastError();
}

hipError_t launch_indexer(const IndexerParams& p, Dtype dt, hipStream_t st, int* n_launches) {
  if ((int64_t)p.B * p.T == 0 || p.s_cap == 0) return hipSuccess;
  const bool mfma = (dt == BF16 || dt == FP8) && p.D == HD;
  const bool modes = p.row_mask || p.kstride != 1 || p.lkey;
  if (p.kstride < 1 || (p.lkey && p.kstride != 1) || (modes && !indexer_modes_supported(p, dt)))
    return hipErrorInvalidValue;
  const int64_t ncols = (p.s_cap + p.kstride - 1) / p.kstride;  // keys (or samples) per row
  if (g8_path(p, dt)) {
    const int nq = (p.T + G8_BM - 1) / G8_BM;
    const int64_t nk = (ncols + G8_BN - 1) / G8_BN;
    hipError_t e;
    // query tiles per XCD when they split evenly and the grid is not a causal square
    const int xcd = (nq % 8 == 0) && (p.T != p.s_cap);
    const dim3 grid((unsigned)(nq * nk), (unsigned)p.B);
    if (p.lkey) {
      if ((e = DSA_ALLOW_LDS((indexer_fp8_groups<G8_CANDIDATES, false>), G8_LDS)) != hipSuccess) return e;
      hipLaunchKernelGGL((indexer_fp8_groups<G8_CANDIDATES, false>), grid, dim3(G8_THREADS), G8_LDS, st, p, nq,
                         (int)nk, xcd);
    } else if (p.kstride != 1) {
      if ((e = DSA_ALLOW_LDS((indexer_fp8_groups<G8_SAMPLES, false>), G8_LDS)) != hipSuccess) return e;
      hipLaunchKernelGGL((indexer_fp8_groups<G8_SAMPLES, false>), grid, dim3(G8_THREADS), G8_LDS, st, p, nq,
                         (int)nk, xcd);
    } else if (p.few_rows && p.row_mask && nq <= 32 * G8_QWORDS) {
      if ((e = DSA_ALLOW_LDS((indexer_fp8_groups<G8_SCORES, true>), G8_LDS)) != hipSuccess) return e;
      hipLaunchKernelGGL((indexer_fp8_groups<G8_SCORES, true>), dim3((unsigned)nk, (unsigned)p.B), dim3(G8_THREADS),
                         G8_LDS, st, p, nq, (int)nk, 0);
    } else {
      if ((e = DSA_ALLOW_LDS((indexer_fp8_groups<G8_SCORES, false>), G8_LDS)) != hipSuccess) return e;
      hipLaunchKernelGGL((indexer_fp8_groups<G8_SCORES, false>), grid, dim3(G8_THREADS), G8_LDS, st, p, nq,
                         (int)nk, xcd);
    }
    if (n_launches) ++*n_launches;
    return hipGetLastError();
  }
  if (mfma && p.T >= 32) {
    const size_t lds = (size_t)(dt == BF16 ? TileCfg<BF16>::LDS : TileCfg<FP8>::LDS);
    dim3 grid((unsigned)((p.s_cap + PK - 1) / PK), (unsigned)((p.T + PQ - 1) / PQ), (unsigned)p.B);
    hipError_t e;
    if (dt == BF16) {
      if ((e = DSA_ALLOW_LDS(indexer_tile<BF16>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(indexer_tile<BF16>, grid, dim3(TILE_THREADS), lds, st, p);
    } else {
      if ((e = DSA_ALLOW_LDS(indexer_tile<FP8>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(indexer_tile<FP8>, grid, dim3(TILE_THREADS), lds, st, p);
    }
  } else if (stream_path(p, dt)) {
    // decode: stream the keys once per query row
    dim3 grid((unsigned)((ncols + 63) / 64), (unsigned)((int64_t)p.B * p.T));
    const int mode = p.lkey ? G8_CANDIDATES : (p.kstride != 1 ? G8_SAMPLES : G8_SCORES);
    launch_stream(p, dt, mode, grid, st);
  } else if (mfma) {
    const int rs = (dt == BF16) ? MfmaCfg<BF16>::RS : MfmaCfg<FP8>::RS;
    const size_t lds = (size_t)(TM + TN) * rs + (size_t)p.H * TM * 4 + (dt == FP8 ? (size_t)p.Hk * TN * 4 : 0);
    dim3 grid((unsigned)((p.s_cap + TN - 1) / TN), (unsigned)((p.T + TM - 1) / TM), (unsigned)p.B);
    hipError_t e;
    if (dt == BF16) {
      if ((e = DSA_ALLOW_LDS(indexer_mfma<BF16>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(indexer_mfma<BF16>, grid, dim3(256), lds, st, p);
    } else {
      if ((e = DSA_ALLOW_LDS(indexer_mfma<FP8>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(indexer_mfma<FP8>, grid, dim3(256), lds, st, p);
    }
  } else {
    const size_t lds = ((size_t)p.H * p.D + p.H) * 4;
    dim3 grid((unsigned)((int64_t)p.B * p.T), (unsigned)((p.s_cap + 255) / 256));
    hipError_t e;
    switch (dt) {
      case F32:
        if ((e = DSA_ALLOW_LDS(indexer_generic<F32>, lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(indexer_generic<F32>, grid, dim3(256), lds, st, p);
        break;
      case BF16:
        if ((e = DSA_ALLOW_LDS(indexer_generic<BF16>, lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(indexer_generic<BF16>, grid, dim3(256), lds, st, p);
        break;
      default:
        if ((e = DSA_ALLOW_LDS(indexer_generic<FP8>, lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(indexer_generic<FP8>, grid, dim3(256), lds, st, p);
        break;
    }
  }
  if (n_launches) ++*n_launches;
  return hipGetLastError();
}

}  // namespace dsa
