// Backward of the sparse MLA attention on the matrix cores (bf16, 576/512 latent rows,
// heads in groups of 64).  The math is the vector kernel's (sparse_mla_bwd.hip):
//
//   P_j  = exp(z_j - lse),  z_j = sm_scale q . c_j        dP_j = dout . c_j[:512]
//   dz_j = P_j (dP_j - D),  D = dout . o                   dz'_j = sm_scale dz_j
//   dq   = sum_j dz'_j c_j                                  dc_j += sum_h dz'_j q + [P_j dout, 0]
//
// as separate launches, so that no kernel holds more than one head-major operand set:
//   mla_bwd_delta  D = dout . o per (query, head), fp32, into the workspace;
//   mla_bwd_pz     per (query, split, head group): the forward's 64-row tiles gathered into
//                  LDS; S^T = C Q^T and dP^T = C dO^T on v_mfma_f32_32x32x16_bf16 (query and
//                  output-gradient fragments held in registers), then dz' as bf16 into the
//                  workspace in mla_bwd_dq's fragment order (per query, head group and
//                  64-slot tile, one 16-byte B fragment per lane and k-step) and, on the
//                  per-slot path, P and dz' as [query][slot][head] for mla_bwd_dc;
//   the latent-row gradient, one of:
//   mla_bwd_dc     per (query, split, head group): the query's 64 head rows and output
//                  gradients in LDS; per tile dC = dz'^T Q + P^T [dO, 0] (K = heads), added to
//                  the selected latent rows with fp32 atomics;
//   mla_bwd_dkv    dense selections (8 topk >= s_cap): per (64 latent rows, query chunk), S
//                  and dP recomputed per query that selected any of the rows, dC summed over
//                  the chunk in registers and added once (after bm_dense_clear and
//                  bm_dense_scatter build the multiplicity map); the chunks of an XCD take
//                  all their tiles one chunk at a time;
//   mla_bwd_dq     per (query, split, head group): the tiles gathered again, dq^T += C^T dz'^T.
// Slots past the last valid entry of a row are never touched; invalid slots inside that
// range get P = dz' = 0, so the later kernels read whole tiles without masks.
//
// Fragment order along the contraction: the transposing LDS reads (ds_read_b64_tr_b16) of
// a 16-row block starting at rb give lane group lg the rows rb + 8 (i / 4) + 4 lg + i % 4
// (i = 0..7), the order in which a 32 x 32 accumulator holds its rows; every fragment
// paired with such a read (global loads of dz' and P) follows the same order.
#include <algorithm>

#include "dsa_internal.h"
#include "mla_tile.h"

namespace dsa {
namespace {
using namespace mla;

constexpr float BM_LOG2E = 1.4426950408889634f;

// workspace arrays (bf16 bits); Tp = topk rounded up to whole 64-row tiles
struct BwWs {
  float* delta;   // [rows][Hm]
  uint16_t* p;    // [rows][Tp][Hm]
  uint16_t* dz;   // [rows][Tp][Hm]   sm_scale * dz
  // the same in mla_bwd_dq's fragment order: per (token, head group of 64, 64-slot tile) a block
  // of 4096 values, entry ((hb * 4 + ks) * 64 + lane) holding, for head 32 hb + lane % 32, the
  // slots 16 ks + 4 (lane / 32) + {0..3} and 8 more (the k-step's permuted B fragment)
  uint16_t* dzt;
  int Tp;
};

__device__ __forceinline__ bool bm_valid(int32_t v, int64_t s_cap) { return v >= 0 && (int64_t)v < s_cap; }

// the last slot of the row whose entry is valid (-1: none), from every wave's scan
__device__ int bm_last_valid(const int32_t* gidx, int topk, int64_t s_cap, int* xs) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int emax = -1;
  for (int e0 = 64 * wave; e0 < topk; e0 += 8 * 256) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + 256 * u + lane;
      v[u] = e < topk ? gidx[e] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (bm_valid(v[u], s_cap)) emax = e0 + 256 * u + lane;
  }
  for (int off = 32; off > 0; off >>= 1) emax = max(emax, __shfl_xor(emax, off, 64));
  if (lane == 0) xs[wave] = emax;
  __syncthreads();
  emax = max(max(xs[0], xs[1]), max(xs[2], xs[3]));
  __syncthreads();
  return emax;
}

// Transposing read of a 16-row block of a tile-layout buffer: dims [32 nb, +32) (segment
// nb / 2), rows [rb, rb + 16) (rb a multiple of 16, so perm(row) = perm(row - rb)).
struct TrOff {
  int o[2][2];  // [read][dim-block parity]
  __device__ __forceinline__ TrOff(int lane) {
    const int lr = lane & 31, lg = lane >> 5;
    const int blk = lr >> 4, li = lr & 15, x = (li & 3) >> 1;
    const int vrow = 4 * lg + (li >> 2);
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
      for (int dp = 0; dp < 2; ++dp)
        o[rd][dp] = (vrow + 8 * rd) * SEG + 16 * ((4 * dp + 2 * blk + x) ^ perm(vrow + 8 * rd)) + ((li & 1) << 3);
  }
  __device__ __forceinline__ bf16x8 read(const unsigned char* buf, int nb, int rb) const {
    const int off = (nb >> 1) * GROUP_BYTES + rb * SEG;
    union {
      i16x4 h[2];
      bf16x8 b;
    } a;
    const bool odd = nb & 1;  // a select, not an index: nb may vary per wave
    a.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(buf + (odd ? o[0][1] : o[0][0]) + off));
    a.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(buf + (odd ? o[1][1] : o[1][0]) + off));
    return a.b;
  }
};

// 8 bf16 at p[0..3] and p[8..11] (the two halves of a permuted fragment), 8-byte loads.
// Kept as 32-bit words until the product: held as a bf16 vector, the fragment gets
// element-wise no-op moves right after the loads, which make the wave wait for them (and
// for everything issued before them) at once.
__device__ __forceinline__ i32x4 ld_split8(const uint16_t* p) {
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
  return i32x4{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
}
__device__ __forceinline__ bf16x8 as_bf16(const i32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- D = dout . o
// grid = rows; wave w takes heads w, w + 4, ...; 8 values per lane
__global__ __launch_bounds__(256) void mla_bwd_delta(MlaBwdParams p, float* __restrict__ delta) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tok = blockIdx.x;
  for (int h = wave; h < p.Hm; h += 4) {
    const int64_t o = ((tok * p.Hm + h) * MDC + 8 * lane);
    const i32x4 g = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.dout) + o);
    const i32x4 y = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.out) + o);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a = (uint32_t)g[e], c = (uint32_t)y[e];
      d = fmaf(__uint_as_float(a << 16), __uint_as_float(c << 16), d);
      d = fmaf(__uint_as_float(a & 0xffff0000u), __uint_as_float(c & 0xffff0000u), d);
    }
    for (int off = 32; off > 0; off >>= 1) d += __shfl_xor(d, off, 64);
    if (lane == 0) delta[tok * p.Hm + h] = d;
  }
}

// ---------------------------------------------------------------- P and dz'
constexpr int PZ_RING = 4 * 4 * MT * 4;                  // per-wave ring of 4 tiles' entries
constexpr int PZ_LDS = 2 * TILE_BYTES + PZ_RING + 64;

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_bwd_pz(MlaBwdParams p, int nsplit, int tiles_per_split, BwWs w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* xs = reinterpret_cast<int*>(smem + 2 * TILE_BYTES + PZ_RING);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int hh = wave & 1, vv = wave >> 1;
  const int lr = lane & 31, lg = lane >> 5;
  const int64_t rows = (int64_t)p.B * p.T;
  const int64_t tok = rows - 1 - (int64_t)blockIdx.x / nsplit;
  const int split = (int)((int64_t)blockIdx.x % nsplit);
  const int hg = blockIdx.y;
  const int64_t b = tok / p.T;
  const int64_t s_cap = p.s_cap;
  const int topk = p.topk, Tp = w.Tp;
  const int32_t* gidx = p.idx + tok * (int64_t)topk;
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  auto tile_dst = [&](int bf) -> uint32_t { return smem_lds + bf * TILE_BYTES + wv * (16 * SEG); };

  // tiles of this split, up to the row's last valid entry (the same range for every split
  // and for the later kernels)
  const int emax = bm_last_valid(gidx, topk, s_cap, xs);
  const int t_row = emax < 0 ? 0 : emax / MT + 1;
  const int t0 = split * tiles_per_split;
  const int ntiles = max(0, min(t_row, t0 + tiles_per_split) - t0);
  if (ntiles == 0) return;

  const int32_t* ering = reinterpret_cast<const int32_t*>(smem + 2 * TILE_BYTES) + wv * 4 * MT;
  const uint32_t ering_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const int32_t*)ering;
  auto fetch_entries = [&](int t) { dma4(gidx + min((t0 + t) * MT + lane, topk - 1), ering_lds + (t & 3) * MT * 4); };
  auto read_entry = [&](int t) -> int32_t { return ering[(t & 3) * MT + lane]; };
  auto in_range = [&](int t) -> bool { return (t0 + t) * MT + lane < topk; };
  const unsigned char* kvg = static_cast<const unsigned char*>(p.kv) + b * s_cap * MRB;
  auto tile_src = [&](int32_t ent) -> GatherSrc {
    return gather_src(kvg, MRB, bm_valid(ent, s_cap) ? ent : 0, wave, lane);
  };

  // prologue: entries of tiles 0 and 1, the query's 64 head rows into buffer 1 and their
  // output gradients (1024-byte rows) into buffer 0, all in flight together
  fetch_entries(0);
  fetch_entries(1);
  {
    const unsigned char* qrows = static_cast<const unsigned char*>(p.q) + (tok * p.Hm + hg * MHG) * MRB;
    gather_tile(tile_dst(1), gather_src(qrows, MRB, lane, wave, lane));
    const unsigned char* grows = static_cast<const unsigned char*>(p.dout) + (tok * p.Hm + hg * MHG) * (MDC * 2);
    gather_tile<8>(tile_dst(0), gather_src(grows, MDC * 2, lane, wave, lane));
  }
  const int myhead = hg * MHG + 32 * hh + lr;
  const float Dh = w.delta[tok * p.Hm + myhead];
  const float lse2 = p.lse[tok * p.Hm + myhead] * BM_LOG2E;
  wait_vmem();
  lds_barrier();

  // query and output-gradient fragments of head 32hh + lr, dims 16 st + 8 lg .. +7
  bf16x8 qf[MROW / 16], gf[MDC / 16];
  {
    const int qr = 32 * hh + lr;
    const unsigned char* qt = smem + TILE_BYTES + qr * SEG;
    const unsigned char* gt = smem + qr * SEG;
#pragma unroll
    for (int st = 0; st < MROW / 16; ++st)
      qf[st] = *reinterpret_cast<const bf16x8*>(qt + (st >> 2) * GROUP_BYTES + 16 * ((2 * (st & 3) + lg) ^ perm(qr)));
#pragma unroll
    for (int st = 0; st < MDC / 16; ++st)
      gf[st] = *reinterpret_cast<const bf16x8*>(gt + (st >> 2) * GROUP_BYTES + 16 * ((2 * (st & 3) + lg) ^ perm(qr)));
  }
#pragma unroll
  for (int st = 0; st < MDC / 16; ++st) asm volatile("" : "+a"(qf[st]), "+a"(gf[st]));
#pragma unroll
  for (int st = MDC / 16; st < MROW / 16; ++st) asm volatile("" : "+v"(qf[st]));
  lds_barrier();  // every wave has read buffer 0 before the first gather overwrites it

  uint64_t vmask_nxt;
  {
    const int32_t e0 = read_entry(0);
    vmask_nxt = __ballot(bm_valid(e0, s_cap) && in_range(0));
    gather_tile(tile_dst(0), tile_src(e0));
  }
  fetch_entries(2);

  const float c1 = p.sm_scale * BM_LOG2E;
  const int mk = 32 * vv + lr;
  int koff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) koff[u] = mk * SEG + 16 * ((2 * u + lg) ^ perm(mk));
  uint16_t* wp = w.p + (tok * Tp) * p.Hm + myhead;
  uint16_t* wz = w.dz + (tok * Tp) * p.Hm + myhead;
  uint16_t* wzt = w.dzt + (tok * (p.Hm / MHG) + hg) * (int64_t)Tp * MHG + lane * 8;
  // P and dz' of a tile as bf16 pairs (rows r, r + 1 of the accumulator), stored after the
  // next tile barrier: stores count in vmcnt, and stored right away they would hold up that
  // barrier's wait for the gather
  uint32_t pp[8], pz[8];
  auto store_tile = [&](int t) {
    const int e0 = (t0 + t) * MT + 32 * vv;
    if (w.p) {  // the [slot][head] arrays feed mla_bwd_dc only (the dense path recomputes P, dz')
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t e = e0 + 8 * (r >> 2) + 4 * lg + (r & 3);
        wp[e * p.Hm] = (uint16_t)((r & 1) ? pp[r >> 1] >> 16 : pp[r >> 1]);
        wz[e * p.Hm] = (uint16_t)((r & 1) ? pz[r >> 1] >> 16 : pz[r >> 1]);
      }
    }
    // slots 32 vv + 16 qq + 4 lg + {0..3, 8..11}: k-step 2 vv + qq of dq's B fragments
    uint16_t* zt = wzt + (int64_t)(t0 + t) * (MT * MHG);
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
      *reinterpret_cast<uint4*>(zt + (hh * 4 + 2 * vv + qq) * 64 * 8) =
          make_uint4(pz[4 * qq], pz[4 * qq + 1], pz[4 * qq + 2], pz[4 * qq + 3]);
  };

  for (int i = 0; i < ntiles; ++i) {
    const int bf = i & 1;
    tile_barrier();
    if (i > 0) store_tile(i - 1);
    const uint64_t vmask = vmask_nxt;
    const bool more = i + 1 < ntiles;
    GatherSrc gnext;
    if (more) {
      const int32_t e_next = read_entry(i + 1);
      vmask_nxt = __ballot(bm_valid(e_next, s_cap) && in_range(i + 1));
      gnext = tile_src(e_next);
    }
    const unsigned char* tb = smem + bf * TILE_BYTES;
    f32x16 s, g;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      g[r] = 0.f;
    }
    {
      constexpr int KG = 4;
      auto kfrag = [&](int st) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(tb + koff[st & 3] + (st >> 2) * GROUP_BYTES);
      };
      constexpr int NG = MROW / 16 / KG;
      bf16x8 kf[3][KG];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int u = 0; u < KG; ++u) kf[gg][u] = kfrag(KG * gg + u);
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        if (gg + 2 < NG) {
#pragma unroll
          for (int u = 0; u < KG; ++u) kf[(gg + 2) % 3][u] = kfrag(KG * (gg + 2) + u);
        }
#pragma unroll
        for (int u = 0; u < KG; ++u) {
          const int st = KG * gg + u;
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[gg % 3][u], qf[st], s, 0, 0, 0);
          if (st < MDC / 16) g = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[gg % 3][u], gf[st], g, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (gg < 6 && more) {
          gather_part(gg, tile_dst(bf ^ 1), gnext);
          if (gg == 5) fetch_entries(i + 3);
        }
      }
    }
    // P, dz' of rows 32vv + 8(r/4) + 4lg + r%4 of the tile, head myhead
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float pv[2], zv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int m = 32 * vv + 8 * ((r + u) >> 2) + 4 * lg + ((r + u) & 3);
        const bool ok = (vmask >> m) & 1ull;
        const float P = ok ? __builtin_amdgcn_exp2f(fmaf(s[r + u], c1, -lse2)) : 0.f;
        pv[u] = P;
        zv[u] = ok ? p.sm_scale * P * (g[r + u] - Dh) : 0.f;
      }
      pp[r >> 1] = (uint32_t)f32_to_bf16_bits(pv[0]) | ((uint32_t)f32_to_bf16_bits(pv[1]) << 16);
      pz[r >> 1] = (uint32_t)f32_to_bf16_bits(zv[0]) | ((uint32_t)f32_to_bf16_bits(zv[1]) << 16);
    }
  }
  store_tile(ntiles - 1);
}

// ---------------------------------------------------------------- dC
// Dim blocks of wave w: (row block mb, dim block nb) for mb in {0, 1}, nb in [4w, 4w + 4),
// and the rope block (mb = w & 1, nb = 16 + w / 2): 9 accumulators.
constexpr int DC_LDS = TILE_BYTES + 8 * GROUP_BYTES + MT * 4 + 64;

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_bwd_dc(MlaBwdParams p, int nsplit, int tiles_per_split, BwWs w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* qbuf = smem;                       // the query's 64 head rows, tile layout
  unsigned char* gbuf = smem + TILE_BYTES;          // their output gradients, 8 segments
  int32_t* sidx = reinterpret_cast<int32_t*>(smem + TILE_BYTES + 8 * GROUP_BYTES);
  int* xs = reinterpret_cast<int*>(sidx + MT);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane & 31, lg = lane >> 5;
  const int64_t rows = (int64_t)p.B * p.T;
  const int64_t tok = rows - 1 - (int64_t)blockIdx.x / nsplit;
  const int split = (int)((int64_t)blockIdx.x % nsplit);
  const int hg = blockIdx.y;
  const int64_t b = tok / p.T;
  const int64_t s_cap = p.s_cap;
  const int topk = p.topk, Tp = w.Tp;
  const int32_t* gidx = p.idx + tok * (int64_t)topk;
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int emax = bm_last_valid(gidx, topk, s_cap, xs);
  const int t_row = emax < 0 ? 0 : emax / MT + 1;
  const int t0 = split * tiles_per_split;
  const int ntiles = max(0, min(t_row, t0 + tiles_per_split) - t0);
  if (ntiles == 0) return;
  {
    const unsigned char* qrows = static_cast<const unsigned char*>(p.q) + (tok * p.Hm + hg * MHG) * MRB;
    gather_tile(smem_lds + wv * (16 * SEG), gather_src(qrows, MRB, lane, wave, lane));
    const unsigned char* grows = static_cast<const unsigned char*>(p.dout) + (tok * p.Hm + hg * MHG) * (MDC * 2);
    gather_tile<8>(smem_lds + TILE_BYTES + wv * (16 * SEG), gather_src(grows, MDC * 2, lane, wave, lane));
  }

  const TrOff tr(lane);
  const int rope_mb = wv & 1, rope_nb = 16 + (wv >> 1);
  f32x16 acc[9];
#pragma unroll
  for (int j = 0; j < 9; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  // A fragments of a tile (dz'^T and P^T, rows 32mb + lr, heads of k-step ks in the permuted
  // order): two 8-byte loads each from the [slot][head] arrays
  const int64_t hoff = hg * MHG + 4 * lg;
  auto load_a = [&](int t, i32x4 (&az)[2][4], i32x4 (&ap)[2][4]) {
    const int64_t e0 = (int64_t)(t0 + t) * MT;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int64_t o = ((tok * Tp + e0 + 32 * mb + lr) * p.Hm) + hoff + 16 * ks;
        az[mb][ks] = ld_split8(w.dz + o);
        ap[mb][ks] = ld_split8(w.p + o);
      }
  };
  i32x4 az0[2][4], ap0[2][4], az1[2][4], ap1[2][4];
  load_a(0, az0, ap0);
  wait_vmem();
  __syncthreads();  // the query and gradient copies are in LDS

  float* dkv = p.dkv + b * s_cap * MROW;
  // one tile: its row indices into LDS, the next tile's A fragments requested, 68 products,
  // then the row gradients added to the latent rows
  auto step = [&](int i, const i32x4 (&az)[2][4], const i32x4 (&ap)[2][4], i32x4 (&nz)[2][4],
                  i32x4 (&np)[2][4]) {
    if (tid < MT) {
      const int e = (t0 + i) * MT + tid;
      const int32_t v = e < topk ? gidx[e] : -1;
      sidx[tid] = bm_valid(v, s_cap) ? v : -1;
    }
    if (i + 1 < ntiles) load_a(i + 1, nz, np);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int rb = 16 * ks;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int nb = 4 * wv + j;
        const bf16x8 bq = tr.read(qbuf, nb, rb), bg = tr.read(gbuf, nb, rb);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          acc[4 * mb + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(az[mb][ks]), bq, acc[4 * mb + j], 0, 0, 0);
          acc[4 * mb + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(ap[mb][ks]), bg, acc[4 * mb + j], 0, 0, 0);
        }
      }
      const bf16x8 bq = tr.read(qbuf, rope_nb, rb);
      acc[8] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(rope_mb ? az[1][ks] : az[0][ks]), bq, acc[8], 0, 0, 0);
    }
    lds_barrier();  // sidx of this tile is in place (no wait for the atomics or the prefetch)
    // accumulator (mb, nb) holds dim 32nb + lr of rows 32mb + 8(r/4) + 4lg + r%4
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const int mb = j < 8 ? (j >> 2) : rope_mb;
      const int nb = j < 8 ? 4 * wv + (j & 3) : rope_nb;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t ri = sidx[32 * mb + 8 * (r >> 2) + 4 * lg + (r & 3)];
        if (ri >= 0) unsafeAtomicAdd(dkv + (int64_t)ri * MROW + 32 * nb + lr, acc[j][r]);
        acc[j][r] = 0.f;
      }
    }
    lds_barrier();  // sidx is read before the next tile rewrites it
  };
  for (int i = 0; i < ntiles; i += 2) {
    step(i, az0, ap0, az1, ap1);
    if (i + 1 < ntiles) step(i + 1, az1, ap1, az0, ap0);
  }
}

// ---------------------------------------------------------------- dC, dense selections
// When the selection covers a large share of the key range (8 topk >= s_cap), the latent-row
// gradient is formed per latent row instead of per selected slot, with no atomics per slot:
// a per-(query, row) multiplicity map (how many of the query's slots name the row) and a byte
// per (query, 64-row tile) that holds any selection are scattered first; then a workgroup per
// (64-row tile, chunk of DK_TC queries) keeps its rows as fragments in registers and walks
// the chunk's queries that selected any of them:
//   S = Q C^T, dP = dO V^T           (64 heads x 64 rows, the query's rows and gradients in LDS)
//   P = m exp(z - lse), dz' = sm_scale P (dP - D)      (m: the row's multiplicity)
//   dC += P^T [dO, 0] + dz'^T Q       (K = heads)
// and adds its sums to the rows once at the end (one fp32 atomic per row value and chunk).
struct BwDense {
  int32_t* mult;  // [rows][ldm] multiplicity of each latent row in the query's selection
  uint8_t* occ;   // [rows][nkt] any selected row in the 64-row tile
  int64_t ldm;
  int nkt;
};
// queries per workgroup: short chunks spread the causal triangle's uneven work over more
// workgroups (4K prefill: 256 -> 32 queries, 10.4 -> 8.1 ms for the whole backward of the
// attention), at the cost of more flushes of the row sums
constexpr int DK_TC = 32;
constexpr int DK_XB = 4 * 64 * 64;                           // P / dz' exchange: 64 bytes per lane
constexpr int DK_LDS = TILE_BYTES + 8 * GROUP_BYTES + DK_XB + 2 * MHG * 4 + 256;  // + L2-request sink

__global__ __launch_bounds__(256) void bm_dense_clear(int32_t* m, int64_t n, uint8_t* occ, int64_t nocc) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) m[i] = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nocc; i += stride) occ[i] = 0;
}

// one workgroup per query row
__global__ __launch_bounds__(256) void bm_dense_scatter(MlaBwdParams p, BwDense d) {
  const int64_t row = blockIdx.x;
  const int32_t* idx = p.idx + row * p.topk;
  for (int j = threadIdx.x; j < p.topk; j += 256) {
    const int32_t e = idx[j];
    if (!bm_valid(e, p.s_cap)) continue;
    atomicAdd(d.mult + row * d.ldm + e, 1);
    d.occ[row * d.nkt + e / MT] = 1;
  }
}

// grid (nkt * nchunk8, B), nchunk8 = nchunk rounded up to a multiple of 8.  Block x runs on XCD
// x mod 8 (the dispatcher's round robin), so chunk ch goes to XCD ch mod 8 and each XCD walks all
// tiles of one chunk before its next: the 32 compute units of an XCD read the same query and
// output-gradient rows (held in its L2) while adding into different tiles of dkv.
// Wave w: latent rows 32 (w & 1) .. of the tile as the S and dP columns, heads 32 (w >> 1) .. as
// their rows; in the dC product rows 32 (w & 1) .. and dim blocks [9 (w >> 1), +9).
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_bwd_dkv(MlaBwdParams p, BwWs w, BwDense d, int nchunk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* qbuf = smem;
  unsigned char* gbuf = smem + TILE_BYTES;
  int32_t* xb = reinterpret_cast<int32_t*>(smem + TILE_BYTES + 8 * GROUP_BYTES);
  float* lsev = reinterpret_cast<float*>(smem + TILE_BYTES + 8 * GROUP_BYTES + DK_XB);
  float* dv = lsev + MHG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane & 31, lg = lane >> 5, kb = wv & 1, hb = wv >> 1;
  const int xk = (int)(blockIdx.x >> 3);
  const int kx = xk % d.nkt, ch = (xk / d.nkt) * 8 + (int)(blockIdx.x & 7);
  if (ch >= nchunk) return;
  const uint32_t sink = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(smem + DK_LDS - 256);
  const int64_t b = blockIdx.y;
  const int T = p.T, Hm = p.Hm;
  const int64_t s_cap = p.s_cap;
  const int64_t j0 = (int64_t)kx * MT;
  const int tq0 = ch * DK_TC, tq1 = min(T, tq0 + DK_TC);
  // which of the chunk's queries selected a row of the tile: one load per lane, all at once
  static_assert(DK_TC <= 64, "one occupancy flag per lane");
  const uint64_t live = __ballot(tq0 + lane < tq1 && d.occ[(b * T + tq0 + lane) * d.nkt + kx] != 0);
  if (live == 0) return;  // the same on every wave
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  // this wave's 32 latent rows: B fragments (dims 16 st + 8 lg .. +7 of row j0 + 32 kb + lr)
  i32x4 cf[MROW / 16];
  {
    const int64_t jr = min<int64_t>(j0 + 32 * kb + lr, s_cap - 1);  // rows past s_cap: multiplicity 0
    const unsigned char* crow = static_cast<const unsigned char*>(p.kv) + (b * s_cap + jr) * MRB;
#pragma unroll
    for (int st = 0; st < MROW / 16; ++st) cf[st] = *reinterpret_cast<const i32x4*>(crow + 32 * st + 16 * lg);
  }
  f32x16 acc[9];
#pragma unroll
  for (int j = 0; j < 9; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const int nb0 = 9 * hb;
  const float c1 = p.sm_scale * BM_LOG2E;
  const TrOff tr(lane);
  const int64_t jcol = j0 + 32 * kb + lr;
  const int qr = 32 * hb + lr;  // head row of this lane's S and dP fragments

  for (int t = tq0; t < tq1; ++t) {
    const int64_t row = b * T + t;
    if (!((live >> (t - tq0)) & 1)) continue;  // uniform
    const float m = (float)d.mult[row * d.ldm + jcol];
    for (int hg = 0; hg < Hm / MHG; ++hg) {
      {
        const unsigned char* qrows = static_cast<const unsigned char*>(p.q) + (row * Hm + hg * MHG) * MRB;
        gather_tile(smem_lds + wv * (16 * SEG), gather_src(qrows, MRB, lane, wave, lane));
        const unsigned char* grows = static_cast<const unsigned char*>(p.dout) + (row * Hm + hg * MHG) * (MDC * 2);
        gather_tile<8>(smem_lds + TILE_BYTES + wv * (16 * SEG), gather_src(grows, MDC * 2, lane, wave, lane));
        if (tid < MHG) {
          lsev[tid] = p.lse[row * Hm + hg * MHG + tid] * BM_LOG2E;
          dv[tid] = w.delta[row * Hm + hg * MHG + tid];
        }
      }
      wait_vmem();
      lds_barrier();
      // L2 requests for the next query's rows (one 4-byte load per 128-byte line into a scratch
      // word, 8.5 lines per lane); waited for only at the next gather, one query later
      if (t + 1 < tq1) {
        const int64_t nrow = row + 1;
        const unsigned char* qn = static_cast<const unsigned char*>(p.q) + (nrow * Hm + hg * MHG) * MRB;
        const unsigned char* gn = static_cast<const unsigned char*>(p.dout) + (nrow * Hm + hg * MHG) * (MDC * 2);
#pragma unroll
        for (int u = 0; u < 5; ++u) {
          const int ln = tid + 256 * u;  // line ln of Q's 576 (64 rows x 9), then dO's 512 (64 x 8)
          if (ln < 576) dma4(qn + (ln / 9) * MRB + (ln % 9) * 128, sink);
          else if (ln < 1088) dma4(gn + ((ln - 576) / 8) * (MDC * 2) + ((ln - 576) % 8) * 128, sink);
        }
      }
      // S and dP: heads 32 hb + rows, this wave's latent rows as columns
      f32x16 sz, gz;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sz[r] = 0.f;
        gz[r] = 0.f;
      }
      {
        const unsigned char* qt = qbuf + qr * SEG;
        const unsigned char* gt = gbuf + qr * SEG;
#pragma unroll
        for (int st = 0; st < MROW / 16; ++st) {
          const int o = (st >> 2) * GROUP_BYTES + 16 * ((2 * (st & 3) + lg) ^ perm(qr));
          sz = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(qt + o), as_bf16(cf[st]), sz, 0, 0, 0);
          if (st < MDC / 16)
            gz = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(gt + o), as_bf16(cf[st]), gz, 0, 0, 0);
        }
      }
      // P and dz' of heads 32 hb + 16 c + {4 lg + e, 8 + 4 lg + e} (e = 0..3), this lane's row,
      // as bf16 pairs: the A fragments (K = heads) of the dC product
      {
        uint32_t pw[8], zw[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float pv[2], zv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int h = 32 * hb + 8 * ((r + u) >> 2) + 4 * lg + ((r + u) & 3);
            const float P = m * __builtin_amdgcn_exp2f(fmaf(sz[r + u], c1, -lsev[h]));
            pv[u] = P;
            zv[u] = p.sm_scale * P * (gz[r + u] - dv[h]);
          }
          pw[r >> 1] = pack_bf16x2(pv[0], pv[1]);
          zw[r >> 1] = pack_bf16x2(zv[0], zv[1]);
        }
        i32x4* mine = reinterpret_cast<i32x4*>(xb + (wv * 64 + lane) * 16);
        mine[0] = i32x4{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};
        mine[1] = i32x4{(int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
        mine[2] = i32x4{(int)zw[0], (int)zw[1], (int)zw[2], (int)zw[3]};
        mine[3] = i32x4{(int)zw[4], (int)zw[5], (int)zw[6], (int)zw[7]};
      }
      lds_barrier();
      // heads 16 ks .. +16 come from the wave with this kb and hb = ks / 2
      i32x4 pf[4], zf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const i32x4* src = reinterpret_cast<const i32x4*>(xb + ((2 * (ks >> 1) + kb) * 64 + lane) * 16);
        pf[ks] = src[ks & 1];
        zf[ks] = src[2 + (ks & 1)];
      }
      // dC: rows 32 kb + .., dims 32 nb + lr
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const int nb = nb0 + j;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int rb = 16 * ks;
          if (nb < MDC / 32) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(pf[ks]), tr.read(gbuf, nb, rb), acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(zf[ks]), tr.read(qbuf, nb, rb), acc[j], 0, 0, 0);
        }
      }
      lds_barrier();  // every wave is done with the buffers before the next gather
    }
  }
  // accumulator j holds dims 32 (nb0 + j) + lr of rows 32 kb + 8 (r / 4) + 4 lg + r % 4
  float* dkv = p.dkv + b * s_cap * MROW;
#pragma unroll
  for (int j = 0; j < 9; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t key = j0 + 32 * kb + 8 * (r >> 2) + 4 * lg + (r & 3);
      if (key < s_cap && acc[j][r] != 0.f) unsafeAtomicAdd(dkv + key * MROW + 32 * (nb0 + j) + lr, acc[j][r]);
    }
}

// ---------------------------------------------------------------- dq
// Accumulators of wave w: dq^T blocks (dims 32nb, heads 32hb) for nb in [4w, 4w + 4), hb in
// {0, 1}, and the rope block (nb = 16 + w / 2, hb = w & 1).
constexpr int DQ_LDS = 2 * TILE_BYTES + PZ_RING + 64;

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_bwd_dq(MlaBwdParams p, int nsplit, int tiles_per_split, BwWs w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* xs = reinterpret_cast<int*>(smem + 2 * TILE_BYTES + PZ_RING);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane & 31, lg = lane >> 5;
  const int64_t rows = (int64_t)p.B * p.T;
  const int64_t tok = rows - 1 - (int64_t)blockIdx.x / nsplit;
  const int split = (int)((int64_t)blockIdx.x % nsplit);
  const int hg = blockIdx.y;
  const int64_t b = tok / p.T;
  const int64_t s_cap = p.s_cap;
  const int topk = p.topk, Tp = w.Tp;
  const int32_t* gidx = p.idx + tok * (int64_t)topk;
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  auto tile_dst = [&](int bf) -> uint32_t { return smem_lds + bf * TILE_BYTES + wv * (16 * SEG); };

  const int emax = bm_last_valid(gidx, topk, s_cap, xs);
  const int t_row = emax < 0 ? 0 : emax / MT + 1;
  const int t0 = split * tiles_per_split;
  const int ntiles = max(0, min(t_row, t0 + tiles_per_split) - t0);
  const int rope_hb = wv & 1, rope_nb = 16 + (wv >> 1);
  f32x16 acc[9];
#pragma unroll
  for (int j = 0; j < 9; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  if (ntiles > 0) {
    const int32_t* ering = reinterpret_cast<const int32_t*>(smem + 2 * TILE_BYTES) + wv * 4 * MT;
    const uint32_t ering_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const int32_t*)ering;
    auto fetch_entries = [&](int t) { dma4(gidx + min((t0 + t) * MT + lane, topk - 1), ering_lds + (t & 3) * MT * 4); };
    auto read_entry = [&](int t) -> int32_t { return ering[(t & 3) * MT + lane]; };
    const unsigned char* kvg = static_cast<const unsigned char*>(p.kv) + b * s_cap * MRB;
    // invalid slots gather row 0 (in bounds); their dz' is 0
    auto tile_src = [&](int32_t ent) -> GatherSrc {
      return gather_src(kvg, MRB, bm_valid(ent, s_cap) ? ent : 0, wave, lane);
    };
    // B fragments of a tile (dz'^T: heads 32hb + lr, slots of k-step ks in the permuted order),
    // stored by mla_bwd_pz in this order: one 16-byte load per lane and fragment
    const uint16_t* zq = w.dzt + (tok * (p.Hm / MHG) + hg) * (int64_t)Tp * MHG + lane * 8;
    auto load_b = [&](int t, i32x4 (&bz)[2][4]) {
      const uint16_t* zt = zq + (int64_t)(t0 + t) * (MT * MHG);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bz[hb][ks] = *reinterpret_cast<const i32x4*>(zt + (hb * 4 + ks) * 64 * 8);
    };
    fetch_entries(0);
    fetch_entries(1);
    wait_vmem();
    lds_barrier();
    gather_tile(tile_dst(0), tile_src(read_entry(0)));
    fetch_entries(2);
    // B fragments run two tiles ahead (a ring of three): they come from HBM, and waited for
    // one tile ahead they held up every tile
    i32x4 bz0[2][4], bz1[2][4], bz2[2][4];
    load_b(0, bz0);
    if (ntiles > 1) load_b(1, bz1);
    const TrOff tr(lane);
    // one tile: wait for its gather and B fragments, request the next tile's gather and the B
    // fragments of the tile after it, 36 products.  Loads complete in issue order; per lane a
    // gather is 18 loads, an entry fetch 1, a fragment set 8.  Issued after tile i's
    // gather: the entry fetch and, unless tile i is the last, the fragments of tile i + 1
    // (for tile 0: its own fragments, then those of tile 1).
    auto step = [&](int i, const i32x4 (&bz)[2][4], i32x4 (&nz)[2][4]) {
      const int bf = i & 1;
      if (i == 0) {
        if (ntiles > 1) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      } else {
        if (i + 1 < ntiles) asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(1)\n\ts_barrier" ::: "memory");
      }
      if (i + 1 < ntiles) {
        gather_tile(tile_dst(bf ^ 1), tile_src(read_entry(i + 1)));
        fetch_entries(i + 3);
        if (i + 2 < ntiles) load_b(i + 2, nz);
      }
      const unsigned char* tb = smem + bf * TILE_BYTES;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int rb = 16 * ks;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 a = tr.read(tb, 4 * wv + j, rb);
          acc[2 * j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16(bz[0][ks]), acc[2 * j], 0, 0, 0);
          acc[2 * j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16(bz[1][ks]), acc[2 * j + 1], 0, 0, 0);
        }
        const bf16x8 a = tr.read(tb, rope_nb, rb);
        // a select, not an index (rope_hb varies per wave: an index becomes indexed register moves)
        acc[8] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16(rope_hb ? bz[1][ks] : bz[0][ks]), acc[8], 0, 0, 0);
      }
    };
    for (int i = 0; i < ntiles; i += 3) {
      step(i, bz0, bz2);
      if (i + 1 < ntiles) step(i + 1, bz1, bz0);
      if (i + 2 < ntiles) step(i + 2, bz2, bz1);
    }
  }
  // accumulator (nb, hb) holds, for head 32hb + lr, dims 32nb + 8(r/4) + 4lg + r%4
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    const int nb = j < 8 ? 4 * wv + (j >> 1) : rope_nb;
    const int hb = j < 8 ? (j & 1) : rope_hb;
    float* dq = p.dq + (tok * p.Hm + hg * MHG + 32 * hb + lr) * MROW + 32 * nb + 4 * lg;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (nsplit == 1) {
        *reinterpret_cast<float4*>(dq + 8 * q) = make_float4(acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]);
      } else if (ntiles > 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) unsafeAtomicAdd(dq + 8 * q + e, acc[j][4 * q + e]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void bm_zero(float* x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.f;
}

struct BmPlan {
  int nsplit, tiles_per_split;
};
// few query tokens: split each selection so that about 1024 workgroups run
BmPlan bm_plan(int64_t rows, int groups, int topk) {
  const int tiles = (topk + MT - 1) / MT;
  int nsplit = 1;
  const int64_t items = rows * groups;
  if (items > 0 && items < 1024) nsplit = (int)std::min<int64_t>(tiles, (1024 + items - 1) / items);
  const int per = (tiles + nsplit - 1) / nsplit;
  return BmPlan{per > 0 ? (tiles + per - 1) / per : 1, per};
}

size_t bm_al(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool mla_bwd_uses_mfma(int Hm, int Dc, int Dr, int64_t s_cap, Dtype dt) {
  return dt == BF16 && Dc == MDC && Dr == MROW - MDC && Hm % MHG == 0 && s_cap * (int64_t)MRB < (int64_t(1) << 32);
}

// Dense selections: the latent-row gradient per 64-row tile (mla_bwd_dkv) instead of per
// selected slot (mla_bwd_dc).
bool mla_bwd_dense(int B, int T, int topk, int64_t s_cap) {
  if (B < 1 || T < 1 || s_cap < 1 || topk < 1) return false;
  const int64_t ldm = (s_cap + MT - 1) / MT * MT;
  return 8 * (int64_t)topk >= s_cap && (int64_t)B * T * ldm * 4 <= (int64_t(1) << 32);
}

// [delta][dz' slot-contiguous] then [P][dz'] (per-slot path) or [multiplicity][occupancy]
size_t mla_bwd_workspace_bytes(int B, int T, int Hm, int Dc, int Dr, int topk, int64_t s_cap, Dtype dt) {
  if (!mla_bwd_uses_mfma(Hm, Dc, Dr, s_cap, dt)) return 0;
  const size_t rows = (size_t)B * T, Tp = (size_t)(topk + MT - 1) / MT * MT;
  const size_t head = bm_al(rows * Hm * 4) + bm_al(rows * Tp * Hm * 2);
  if (mla_bwd_dense(B, T, topk, s_cap)) {
    const size_t ldm = (size_t)((s_cap + MT - 1) / MT * MT), nkt = ldm / MT;
    return head + bm_al(rows * ldm * 4) + bm_al(rows * nkt);
  }
  return head + 2 * bm_al(rows * Tp * Hm * 2);
}

hipError_t launch_sparse_mla_bwd_mfma(const MlaBwdParams& p, void* ws, size_t ws_bytes, hipStream_t st,
                                      int* n_launches) {
  const int64_t rows = (int64_t)p.B * p.T;
  const int Tp = (p.topk + MT - 1) / MT * MT;
  if (ws_bytes < mla_bwd_workspace_bytes(p.B, p.T, p.Hm, p.Dc, p.Dr, p.topk, p.s_cap, BF16) || (rows > 0 && !ws))
    return hipErrorInvalidValue;
  const int64_t nkv = (int64_t)p.B * p.s_cap * MROW;
  if (nkv > 0) {
    hipLaunchKernelGGL(bm_zero, dim3((unsigned)std::min<int64_t>((nkv + 255) / 256, 4096)), dim3(256), 0, st, p.dkv, nkv);
    if (n_launches) ++*n_launches;
  }
  if (rows == 0) return hipGetLastError();
  const bool dense = mla_bwd_dense(p.B, p.T, p.topk, p.s_cap);
  char* base = static_cast<char*>(ws);
  BwWs w;
  w.delta = reinterpret_cast<float*>(base);
  base += bm_al((size_t)rows * p.Hm * 4);
  const size_t arr = bm_al((size_t)rows * Tp * p.Hm * 2);
  w.dzt = reinterpret_cast<uint16_t*>(base);
  base += arr;
  w.Tp = Tp;
  BwDense d{};
  if (dense) {
    w.p = w.dz = nullptr;
    d.ldm = (p.s_cap + MT - 1) / MT * MT;
    d.nkt = (int)(d.ldm / MT);
    d.mult = reinterpret_cast<int32_t*>(base);
    d.occ = reinterpret_cast<uint8_t*>(base + bm_al((size_t)rows * d.ldm * 4));
  } else {
    w.p = reinterpret_cast<uint16_t*>(base);
    w.dz = reinterpret_cast<uint16_t*>(base + arr);
  }
  const int groups = p.Hm / MHG;
  const BmPlan pl = bm_plan(rows, groups, p.topk);
  const int64_t nq = rows * p.Hm * MROW;
  if (pl.nsplit > 1 && nq > 0) {
    hipLaunchKernelGGL(bm_zero, dim3((unsigned)std::min<int64_t>((nq + 255) / 256, 4096)), dim3(256), 0, st, p.dq, nq);
    if (n_launches) ++*n_launches;
  }
  hipLaunchKernelGGL(mla_bwd_delta, dim3((unsigned)rows), dim3(256), 0, st, p, w.delta);
  if (dense) {
    const int64_t nm = rows * d.ldm, nocc = rows * d.nkt;
    hipLaunchKernelGGL(bm_dense_clear, dim3((unsigned)std::min<int64_t>((nm + 255) / 256, 8192)), dim3(256), 0, st,
                       d.mult, nm, d.occ, nocc);
    hipLaunchKernelGGL(bm_dense_scatter, dim3((unsigned)rows), dim3(256), 0, st, p, d);
    if (n_launches) *n_launches += 2;
  }
  const dim3 grid((unsigned)(rows * pl.nsplit), (unsigned)groups);
  hipError_t e;
  {
    static std::atomic<size_t> high{0};
    if ((e = allow_dynamic_lds(reinterpret_cast<const void*>(mla_bwd_pz), PZ_LDS, high)) != hipSuccess) return e;
    hipLaunchKernelGGL(mla_bwd_pz, grid, dim3(256), PZ_LDS, st, p, pl.nsplit, pl.tiles_per_split, w);
  }
  if (dense) {
    static std::atomic<size_t> high{0};
    if ((e = allow_dynamic_lds(reinterpret_cast<const void*>(mla_bwd_dkv), DK_LDS, high)) != hipSuccess) return e;
    const int nchunk = (p.T + DK_TC - 1) / DK_TC, nchunk8 = (nchunk + 7) / 8 * 8;
    hipLaunchKernelGGL(mla_bwd_dkv, dim3((unsigned)((int64_t)d.nkt * nchunk8), (unsigned)p.B), dim3(256), DK_LDS, st,
                       p, w, d, nchunk);
  } else {
    static std::atomic<size_t> high{0};
    if ((e = allow_dynamic_lds(reinterpret_cast<const void*>(mla_bwd_dc), DC_LDS, high)) != hipSuccess) return e;
    hipLaunchKernelGGL(mla_bwd_dc, grid, dim3(256), DC_LDS, st, p, pl.nsplit, pl.tiles_per_split, w);
  }
  {
    static std::atomic<size_t> high{0};
    if ((e = allow_dynamic_lds(reinterpret_cast<const void*>(mla_bwd_dq), DQ_LDS, high)) != hipSuccess) return e;
    hipLaunchKernelGGL(mla_bwd_dq, grid, dim3(256), DQ_LDS, st, p, pl.nsplit, pl.tiles_per_split, w);
  }
  if (n_launches) *n_launches += 4;
  return hipGetLastError();
}

}  // namespace dsa
