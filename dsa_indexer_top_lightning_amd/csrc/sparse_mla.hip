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
// mla_mfma (bf16, Dc = 512, Dr = 64, 64 heads per workgroup, 4 waves):
//   * tiles of 64 selected rows are gathered from HBM straight into LDS with
//     16-byte global_load_lds (a latent row is 1152 contiguous bytes) into two
//     alternating tiles; the gather of tile i+1 runs while tile i is consumed.
//     Each wave load moves 8 rows x 128 bytes (8 whole cache lines).  A tile is
//     stored as 9 groups of 128-byte row segments; inside a segment the 16-byte
//     chunks are XOR-permuted by the row so that the matrix-core fragment reads
//     (16 rows x 16 B, and the transposing reads of 4 rows x 4 chunks per
//     half-wave) are bank-conflict free;
//   * wave (hh, vv) computes S^T = K Q^T for kv rows [32vv, +32) x heads
//     [32hh, +32) on v_mfma_f32_32x32x16_bf16 (Q^T fragments stay in registers
//     for the whole kernel); the two vv waves of a head half swap their row
//     maxima, then their bf16 probabilities, through LDS, so both hold P^T for all
//     64 rows with one shared running max (online softmax in exp2, fp32 state);
//     the running sum adds the bf16 probabilities actually used;
//   * the same wave accumulates O^T[256vv .. +256 dims][32 heads] += V^T P^T; the
//     V^T fragments come from the same tile through ds_read_b64_tr_b16
//     (transposing LDS reads), so K and V share one LDS copy;
//   * with few queries (decode) each query's selection is split over several
//     workgroups that write unnormalised partials (O, running max, sum) and
//     mla_combine merges them in a fixed order (no float atomics: results are
//     run-to-run identical).
// mla_generic: any Dc/Dr/Hm, fp32 or bf16, one wave per head, fp32 FMA.
#include <algorithm>

#include "dsa_internal.h"
#include "mla_tile.h"

namespace dsa {
namespace {

using namespace mla;

constexpr int LOADS_PER_WAVE = NGROUP * 2;       // each wave gathers 16 rows: 2 row octets x 9 segments
constexpr int LDS_XMAX = 4 * 32 * 4 + 64;        // per-wave tile maxima of 32 heads + rescale flags
constexpr int LDS_XP = 4 * 8 * 64 * 4;           // per-wave P^T tile as bf16 pairs
constexpr int LDS_RING = 4 * 4 * 64 * 4;         // per-wave ring of 4 tiles' entries
constexpr int LDS_MLA = 2 * TILE_BYTES + LDS_XMAX + LDS_XP + LDS_RING;
constexpr int MAX_TILES_PER_ITEM = 64;
// The running max is raised only when a tile's max exceeds it by more than 2^8 (log2
// units); until then probabilities are taken against the stale max (values <= 256),
// which is exact after the final division and saves rescaling the accumulators.
constexpr float RESCALE_LOG2 = 8.f;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Multiply an accumulator block in place in the AGPRs that hold it.  Written as
// read / multiply / write per register so the compiler keeps the matrix-core
// accumulators in AGPRs across the tile loop (a plain `acc *= alpha` on this rare
// path makes it carry all of them in VGPRs, copying every tile).
__device__ __forceinline__ void scale_agpr(f32x16& a, float alpha) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = a[r], t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(t)
                 : "v"(alpha));
    a[r] = x;
  }
}

// grid.x = (query, split) work item, heaviest queries first; grid.y = head group.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_mfma(MlaParams p, int nsplit, int tiles_per_split, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* xmax = reinterpret_cast<float*>(smem + 2 * TILE_BYTES);
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem + 2 * TILE_BYTES + LDS_XMAX);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int hh = wave & 1, vv = wave >> 1;
  const int lr = lane & 31, lg = lane >> 5;
  const int64_t rows = (int64_t)p.B * p.T;
  const int64_t item = blockIdx.x;
  const int64_t tok = rows - 1 - item / nsplit;  // heaviest (latest) queries first
  const int split = (int)(item % nsplit);
  const int hg = blockIdx.y;
  const int64_t b = tok / p.T;
  const int64_t s_cap = p.s_cap;
  const int topk = p.topk;
  const int32_t* gidx = p.idx + tok * (int64_t)topk;

  // ---- prologue: the entry copies of the first two tiles, the query copy and the scan
  //      for the last valid entry are all issued before any of them is waited for, so
  //      the workgroup pays one global round trip before its first gather
  const int t0 = split * tiles_per_split;
  const int e_lo = t0 * MT, e_hi = min(topk, (t0 + tiles_per_split) * MT);
  // The entries of tile t are copied by each wave into its own LDS ring slot t % 4 with
  // one 4-byte global-to-LDS load (lane i writes word i), so that no register carries a
  // pending load across tiles.  Past the end the loads re-read the last entry (never used).
  const int32_t* ering = reinterpret_cast<const int32_t*>(smem + 2 * TILE_BYTES + LDS_XMAX + LDS_XP) + wv * 4 * MT;
  const uint32_t ering_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const int32_t*)ering;
  auto fetch_entries = [&](int t) { dma4(gidx + min((t0 + t) * MT + lane, topk - 1), ering_lds + (t & 3) * MT * 4); };
  auto read_entry = [&](int t) -> int32_t { return ering[(t & 3) * MT + lane]; };
  // lanes of tile t past the split's last entry hold a clamped copy of that entry, not one
  // of their own: they never count as selected
  auto in_split = [&](int t) -> bool { return (t0 + t) * MT + lane < e_hi; };

  const unsigned char* kvg = static_cast<const unsigned char*>(p.kv) + b * s_cap * MRB;
  auto valid = [&](int32_t v) -> bool { return v >= 0 && (int64_t)v < s_cap; };
  // per-lane sources of a tile's gather (an invalid entry gathers row 0, in bounds, and is
  // masked out of the softmax)
  auto tile_src = [&](int32_t ent) -> GatherSrc { return gather_src(kvg, MRB, valid(ent) ? ent : 0, wave, lane); };
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  auto tile_dst = [&](int bf) -> uint32_t { return smem_lds + bf * TILE_BYTES + wv * (16 * SEG); };

  fetch_entries(0);
  fetch_entries(1);
  // The query's 64 head rows (1152 contiguous bytes each) are copied into the second tile
  // buffer in the tile layout, whole cache lines per load, by the same copies as a tile's
  // gather (row r = head 64hg + r); the first gather into that buffer is issued in tile 0,
  // after every wave has read its fragments.
  {
    const unsigned char* qrows = static_cast<const unsigned char*>(p.q) + (tok * p.Hm + hg * MHG) * MRB;
    gather_tile(tile_dst(1), gather_src(qrows, MRB, lane, wave, lane));
  }

  // The last valid entry: each wave scans every fourth 64-entry block of the split's
  // entries (8 independent loads in flight per lane) and the four wave maxima meet in LDS
  // at the barrier that also publishes the query copy.
  int emax = -1;
  for (int e0 = e_lo + 64 * wv; e0 < e_hi; e0 += 8 * 256) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + 256 * u + lane;
      v[u] = e < e_hi ? gidx[e] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (v[u] >= 0 && (int64_t)v[u] < s_cap) emax = e0 + 256 * u + lane;
  }
  for (int off = 32; off > 0; off >>= 1) emax = max(emax, __shfl_xor(emax, off, 64));
  int* xemax = reinterpret_cast<int*>(xmax);  // free until the first tile
  if (lane == 0) xemax[wv] = emax;

  const int head0 = hg * MHG + 32 * hh;
  const int myhead = head0 + lr;
  wait_vmem();    // entry and query copies of this wave have landed
  lds_barrier();  // ... and those of every wave, and every wave's scan result
  emax = max(max(xemax[0], xemax[1]), max(xemax[2], xemax[3]));
  // tiles of this split up to the last one holding a valid entry: [t0, t0 + ntiles)
  const int ntiles = emax < 0 ? 0 : emax / MT - t0 + 1;
  if (ntiles == 0) {
    if (nsplit == 1) {
      uint16_t* og = static_cast<uint16_t*>(p.out) + (tok * p.Hm + hg * MHG) * MDC;
      for (int i = tid; i < MHG * MDC; i += 256) og[i] = 0;
      if (p.lse && vv == 0 && lg == 0) p.lse[tok * p.Hm + myhead] = -__builtin_inff();
    } else if (vv == 0 && lg == 0) {
      float* ml = ws_ml + ((tok * nsplit + split) * p.Hm + myhead) * 2;
      ml[0] = -__builtin_inff();
      ml[1] = 0.f;
    }
    return;
  }

  // Q^T fragments for the whole kernel: lane (head lr, group lg) holds
  // q[head][16*st + 8*lg .. +7] for st = 0..35 (row 32hh + lr of the copy, logical chunk
  // 2st + lg: segment st/4, chunk-in-segment 2(st%4) + lg)
  bf16x8 qf[MROW / 16];
  {
    const int qr = 32 * hh + lr;
    const unsigned char* qt = smem + TILE_BYTES + qr * SEG;
#pragma unroll
    for (int st = 0; st < MROW / 16; ++st)
      qf[st] = *reinterpret_cast<const bf16x8*>(qt + (st >> 2) * GROUP_BYTES + 16 * ((2 * (st & 3) + lg) ^ perm(qr)));
  }
  // the query fragments are opaque to the compiler from here on (under register pressure
  // it would otherwise re-read them on every tile); the 512 latent dims live in
  // accumulation registers, which the matrix cores read directly, leaving the vector
  // registers for deeper LDS prefetch
#pragma unroll
  for (int st = 0; st < MDC / 16; ++st) asm volatile("" : "+a"(qf[st]));
#pragma unroll
  for (int st = MDC / 16; st < MROW / 16; ++st) asm volatile("" : "+v"(qf[st]));

  // Entries are fetched two tiles ahead of their gather and every gather is followed by
  // exactly one entry fetch, so at the top of tile i `vmcnt(1)` leaves only the newest
  // entry fetch in flight: the gather of tile i has landed and so have the entries of
  // tile i + 1, without waiting for anything issued later.
  uint64_t vmask_nxt;
  {
    const int32_t e0 = read_entry(0);
    vmask_nxt = __ballot(valid(e0) && in_split(0));
    gather_tile(tile_dst(0), tile_src(e0));
  }
  fetch_entries(2);

  const float qk_scale = p.sm_scale * LOG2E;
  // Running maxima (log2 units) of the two heads this lane meets in the O^T accumulators:
  // head lr of half 0 (m0) and of half 1 (m1); every wave holds the same values and
  // takes the same rescale decisions.  l_part sums the bf16 probabilities of this
  // wave's own S^T block (head 32hh + lr, rows of lane group lg).
  float m0 = -__builtin_inff(), m1 = -__builtin_inff(), l_part = 0.f;
  f32x16 acc[4][2];  // O^T: dims 128*wave + 32*db .. +32  x  heads 32*hb .. +32
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][hb][r] = 0.f;

  // K fragment of step st: row m = 32vv + lr, chunk 2st + lg = segment st/4, chunk-in-segment
  // 2(st%4) + lg: four per-lane offsets, the segment is an immediate
  const int mk = 32 * vv + lr;
  int koff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) koff[u] = mk * SEG + 16 * ((2 * u + lg) ^ perm(mk));
  // V^T fragment (k-step ks, dim block db) = dims 128*wave + 32db .. +32 x the 16 rows of ks:
  // read #1 gives rows rb + vrow, read #2 rows rb + 8 + vrow, chunk 16wave + 4db + 2blk + x =
  // segment 2wave + db/2, chunk-in-segment 4(db%2) + 2blk + x, byte 8(li & 1); rb is a
  // multiple of 16 so perm(row) = perm(vrow): per-lane offsets for (read, db parity)
  const int blk = lr >> 4, li = lr & 15, x = (li & 3) >> 1;
  const int vrow = 4 * lg + (li >> 2);
  int voff[2][2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
#pragma unroll
    for (int dp = 0; dp < 2; ++dp)
      voff[rd][dp] = 2 * wave * GROUP_BYTES + (vrow + 8 * rd) * SEG +
                     16 * ((4 * dp + 2 * blk + x) ^ perm(vrow + 8 * rd)) + ((li & 1) << 3);
  // P exchange: block of wave w, half j (k-step 2vv(w) + j) at xp[(2w + j) * 64 + lane] as 4 dwords
  i32x4* xpv = reinterpret_cast<i32x4*>(xp);

  // V^T fragment reads of k-step ks from tile tb (see the PV step below)
  auto load_v = [&](const unsigned char* tb, int ks, bf16x8* dst) {
    const int rb = 32 * (ks >> 1) + 16 * (ks & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int off = (db >> 1) * GROUP_BYTES + rb * SEG;
      union {
        i16x4 h[2];
        bf16x8 b;
      } a;
      a.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(tb + voff[0][db & 1] + off));
      a.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(tb + voff[1][db & 1] + off));
      dst[db] = a.b;
    }
  };
  int* xflag = reinterpret_cast<int*>(xmax + 4 * 32);

  for (int i = 0; i < ntiles; ++i) {
    const int bf = i & 1;
    tile_barrier();  // tile i is in LDS for every wave; buffer bf^1 is free
    const uint64_t vmask = vmask_nxt;
    const bool more = i + 1 < ntiles;
    GatherSrc gnext;
    if (more) {
      const int32_t e_next = read_entry(i + 1);
      vmask_nxt = __ballot(valid(e_next) && in_split(i + 1));
      gnext = tile_src(e_next);
    }
    const unsigned char* tb = smem + bf * TILE_BYTES;

    // ---- S^T for own 32 kv rows x 32 heads
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    {
      constexpr int KG = 4;
      auto kfrag = [&](int st) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(tb + koff[st & 3] + (st >> 2) * GROUP_BYTES);
      };
      constexpr int NG = MROW / 16 / KG;  // 9 groups of 4 steps, read two groups ahead
      bf16x8 kf[3][KG];
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int u = 0; u < KG; ++u) kf[g][u] = kfrag(KG * g + u);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g + 2 < NG) {
#pragma unroll
          for (int u = 0; u < KG; ++u) kf[(g + 2) % 3][u] = kfrag(KG * (g + 2) + u);
        }
#pragma unroll
        for (int u = 0; u < KG; ++u)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[g % 3][u], qf[KG * g + u], s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // the next tile's gather, three copies after each of the first six groups (issued
        // in one burst the copies fill the global-to-LDS path and stall the issuing
        // waves), then the entry copy, which must stay the newest global load for the
        // vmcnt(1) of the next tile barrier
        if (g < 6 && more) {
          gather_part(g, tile_dst(bf ^ 1), gnext);
          if (g == 5) fetch_entries(i + 3);
        }
      }
    }
    // the first two k-steps of V^T are read while the softmax runs
    bf16x8 vf[3][4];
    load_v(tb, 0, vf[0]);
    load_v(tb, 1, vf[1]);

    float mx = -__builtin_inff();
    if (vmask != ~0ull) {  // partial tile: mask rows without a valid index
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * vv + 8 * (r >> 2) + 4 * lg + (r & 3);
        s[r] = ((vmask >> m) & 1ull) ? s[r] : -__builtin_inff();
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * qk_scale;

    // P of the own block against the running max.  A wave whose tile maximum exceeds the
    // running max of one of its heads by more than 2^8 raises a flag; the flags travel
    // with the P blocks, and only when one is raised (the first tile, or a jump of the
    // maximum) do all waves exchange tile maxima, rescale and recompute P.
    uint32_t own[8];
    auto make_p = [&]() {
      const float m_own = hh ? m1 : m0;
      const float m_neg = m_own == -__builtin_inff() ? 0.f : -m_own;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        own[r] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[2 * r], qk_scale, m_neg)),
                             __builtin_amdgcn_exp2f(fmaf(s[2 * r + 1], qk_scale, m_neg)));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        xpv[(2 * wave + j) * 64 + lane] = i32x4{(int)own[4 * j], (int)own[4 * j + 1], (int)own[4 * j + 2], (int)own[4 * j + 3]};
    };
    make_p();
    const uint64_t need = __ballot(mx > (hh ? m1 : m0) + RESCALE_LOG2);
    if (lane == 0) xflag[wave] = need != 0ull;
    lds_barrier();
    // P^T fragment of k-step ks and head half hb: k-step ks uses C-layout values
    // 8(ks%2) .. +7 of the S^T block of rows 32(ks/2) .. +32 (every wave's block, own included)
    auto p_frag = [&](int ks, int hb) -> bf16x8 {
      return __builtin_bit_cast(bf16x8, xpv[(2 * (hb + 2 * (ks >> 1)) + (ks & 1)) * 64 + lane]);
    };
    // the flags and the first two k-steps' P fragments are read together; in the rare case
    // of a raised flag every wave rewrites its block and the fragments are read again
    const i32x4 flags = *reinterpret_cast<const i32x4*>(xflag);
    bf16x8 pf[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) pf[ks][hb] = p_frag(ks, hb);
    // one use of all four: issued here with the flag read (not sunk past the branch), one wait
    asm volatile("" : "+v"(pf[0][0]), "+v"(pf[0][1]), "+v"(pf[1][0]), "+v"(pf[1][1]));
    if (flags[0] | flags[1] | flags[2] | flags[3]) {  // the same in every wave
      if (lg == 0) xmax[wave * 32 + lr] = mx;
      lds_barrier();
      // tile maxima of head lr of each half (waves 0, 2 hold half 0; waves 1, 3 half 1)
      const float mt0 = fmaxf(xmax[lr], xmax[64 + lr]);
      const float mt1 = fmaxf(xmax[32 + lr], xmax[96 + lr]);
      const float n0 = fmaxf(m0, mt0), n1 = fmaxf(m1, mt1);
      const float a0 = n0 == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m0 - n0);
      const float a1 = n1 == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m1 - n1);
      l_part *= hh ? a1 : a0;
      m0 = n0;
      m1 = n1;
      if (i > 0) {  // before the first tile's P the accumulators are still zero
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          scale_agpr(acc[db][0], a0);
          scale_agpr(acc[db][1], a1);
        }
      }
      make_p();
      lds_barrier();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) pf[ks][hb] = p_frag(ks, hb);
    }
    {
      float ls = 0.f;  // the probabilities actually used, as rounded to bf16
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int r = 0; r < 8; ++r) ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, own[r]), ones, ls, false);
      l_part += ls;
    }

    // ---- O^T[dims 128wave + 32db][heads 32hb] += V^T . P^T over the tile's 4 k-steps of
    // 16 rows.  The V^T reads of step ks+2 are issued while step ks's matrix-core steps run.
    {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 p0 = ks < 2 ? pf[ks][0] : p_frag(ks, 0), p1 = ks < 2 ? pf[ks][1] : p_frag(ks, 1);
        if (ks + 2 < 4) load_v(tb, ks + 2, vf[(ks + 2) % 3]);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          acc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks % 3][db], p0, acc[db][0], 0, 0, 0);
          acc[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks % 3][db], p1, acc[db][1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- row sums per head: own block (both lane groups), then both row halves
  l_part += __shfl_xor(l_part, 32, 64);
  if (lg == 0) xmax[wave * 32 + lr] = l_part;  // every wave is past its last read of xmax
  __syncthreads();
  const float L0 = xmax[lr] + xmax[64 + lr], L1 = xmax[32 + lr] + xmax[96 + lr];

  if (nsplit == 1) {
    // normalise, transpose through LDS, write out[tok][hg*64 .. +64][512] with 16-byte stores
    constexpr int OST = MDC + 8;  // padded bf16 row stride of the staging buffer
    uint16_t* ost = reinterpret_cast<uint16_t*>(smem);
    const float inv[2] = {L0 > 0.f ? 1.f / L0 : 0.f, L1 > 0.f ? 1.f / L1 : 0.f};
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dim = 128 * wave + 32 * db + 8 * j + 4 * lg;
          uint32_t* dst = reinterpret_cast<uint32_t*>(ost + (32 * hb + lr) * OST + dim);
          dst[0] = pack_bf16x2(acc[db][hb][4 * j] * inv[hb], acc[db][hb][4 * j + 1] * inv[hb]);
          dst[1] = pack_bf16x2(acc[db][hb][4 * j + 2] * inv[hb], acc[db][hb][4 * j + 3] * inv[hb]);
        }
    __syncthreads();
    unsigned char* og = static_cast<unsigned char*>(p.out) + ((tok * p.Hm + hg * MHG) * MDC) * 2;
    for (int c = tid; c < MHG * (MDC * 2 / 16); c += 256) {
      const int h = c / (MDC * 2 / 16), ch = c % (MDC * 2 / 16);
      *reinterpret_cast<i32x4*>(og + (h * MDC) * 2 + ch * 16) =
          *reinterpret_cast<const i32x4*>(reinterpret_cast<const unsigned char*>(ost + h * OST) + ch * 16);
    }
    if (p.lse && wave == 0 && lg == 0) {
      p.lse[tok * p.Hm + hg * MHG + lr] = L0 > 0.f ? (m0 + log2f(L0)) * LN2 : -__builtin_inff();
      p.lse[tok * p.Hm + hg * MHG + 32 + lr] = L1 > 0.f ? (m1 + log2f(L1)) * LN2 : -__builtin_inff();
    }
  } else {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float* o = ws_o + ((tok * nsplit + split) * p.Hm + hg * MHG + 32 * hb + lr) * MDC;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dim = 128 * wave + 32 * db + 8 * j + 4 * lg;
          *reinterpret_cast<float4*>(o + dim) =
              make_float4(acc[db][hb][4 * j], acc[db][hb][4 * j + 1], acc[db][hb][4 * j + 2], acc[db][hb][4 * j + 3]);
        }
    }
    if (wave == 0 && lg == 0) {
      float* ml = ws_ml + ((tok * nsplit + split) * p.Hm + hg * MHG + lr) * 2;
      ml[0] = m0;
      ml[1] = L0;
      ml += 32 * 2;
      ml[0] = m1;
      ml[1] = L1;
    }
  }
}

// Merge the split partials of one (query, head) in split order.  grid.x = (query, group
// of 4 heads, half of the 512 value dims); 256 threads = 4 heads x 64 lanes x 4 dims
// (16-byte loads of the partials).
// The loads of a batch of splits are independent of each other (an empty split's
// partial is never written and gets weight 0 through a select), so they are all in
// flight at once.
// CMB_BATCH splits are loaded per round trip: 8, or 32 when there are more than 8 splits
// (few query rows, e.g. a 4-sequence decode over 32 splits: one round trip instead of four)
template <int CMB_BATCH>
__global__ __launch_bounds__(256) void mla_combine(MlaParams p, int nsplit, const float* __restrict__ ws_o,
                                                   const float* __restrict__ ws_ml) {
  const int halves = 2, groups = p.Hm / 4;
  const int64_t tok = blockIdx.x / (groups * halves);
  const int rest = (int)(blockIdx.x % (groups * halves));
  const int head = (rest / halves) * 4 + (threadIdx.x >> 6);
  const int d0 = (rest % halves) * (MDC / halves) + (threadIdx.x & 63) * 4;
  const float* ml = ws_ml + (tok * nsplit * p.Hm + head) * 2;  // split s at ml + s * Hm * 2
  const int64_t mstride = (int64_t)p.Hm * 2;
  // the largest split max, from batches of independent loads (a repeated last split does
  // not change it)
  float M = -__builtin_inff();
  for (int s0 = 0; s0 < nsplit; s0 += CMB_BATCH) {
    float f[CMB_BATCH];
#pragma unroll
    for (int u = 0; u < CMB_BATCH; ++u) f[u] = ml[min(s0 + u, nsplit - 1) * mstride];
#pragma unroll
    for (int u = 0; u < CMB_BATCH; ++u) M = fmaxf(M, f[u]);
  }
  float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f, L = 0.f;
  if (M != -__builtin_inff()) {
    const float* src = ws_o + (tok * nsplit * p.Hm + head) * MDC + d0;  // split s at src + s * Hm * MDC
    const int64_t ostride = (int64_t)p.Hm * MDC;
    for (int s0 = 0; s0 < nsplit; s0 += CMB_BATCH) {
      float4 v[CMB_BATCH];
      float f[CMB_BATCH], l[CMB_BATCH];
#pragma unroll
      for (int u = 0; u < CMB_BATCH; ++u) {
        const int s = min(s0 + u, nsplit - 1);
        v[u] = *reinterpret_cast<const float4*>(src + s * ostride);
        l[u] = ml[s * mstride + 1];
        f[u] = ml[s * mstride];
      }
#pragma unroll
      for (int u = 0; u < CMB_BATCH; ++u) {
        const bool use = s0 + u < nsplit && l[u] != 0.f;
        const float w = use ? exp2f(f[u] - M) : 0.f;
        L = use ? fmaf(l[u], w, L) : L;
        o0 = use ? fmaf(v[u].x, w, o0) : o0;
        o1 = use ? fmaf(v[u].y, w, o1) : o1;
        o2 = use ? fmaf(v[u].z, w, o2) : o2;
        o3 = use ? fmaf(v[u].w, w, o3) : o3;
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* og = static_cast<uint16_t*>(p.out) + (tok * p.Hm + head) * MDC + d0;
  og[0] = f32_to_bf16_bits(o0 * inv);
  og[1] = f32_to_bf16_bits(o1 * inv);
  og[2] = f32_to_bf16_bits(o2 * inv);
  og[3] = f32_to_bf16_bits(o3 * inv);
  if (p.lse && d0 == 0) p.lse[tok * p.Hm + head] = L > 0.f ? (M + log2f(L)) * LN2 : -__builtin_inff();
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
  int nsplit, tiles_per_split;
};

// Few queries (decode): split each query's selection over several workgroups so that
// about one workgroup per compute unit runs (one per CU fits in LDS); every split
// covers a run of whole 64-row tiles.
SplitPlan plan_split(int64_t rows, int Hm, int topk) {
  const int64_t wgs = rows * (Hm / MHG);
  const int tiles = (topk + MT - 1) / MT;
  int nsplit = 1;
  if (wgs < 256) nsplit = (int)std::min<int64_t>(tiles, (256 + wgs - 1) / std::max<int64_t>(wgs, 1));
  int tps = (tiles + nsplit - 1) / nsplit;
  tps = std::min(tps, MAX_TILES_PER_ITEM);
  nsplit = (tiles + tps - 1) / tps;
  return {nsplit, tps};
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
    const size_t lds = LDS_MLA;
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
    hipLaunchKernelGGL(mla_mfma, grid, dim3(256), lds, st, p, sp.nsplit, sp.tiles_per_split, ws_o, ws_ml);
    if (n_launches) ++*n_launches;
    if (sp.nsplit > 1) {
      const dim3 cgrid((unsigned)(rows * (p.Hm / 4) * 2));
      if (sp.nsplit > 8) hipLaunchKernelGGL(mla_combine<32>, cgrid, dim3(256), 0, st, p, sp.nsplit, ws_o, ws_ml);
      else hipLaunchKernelGGL(mla_combine<8>, cgrid, dim3(256), 0, st, p, sp.nsplit, ws_o, ws_ml);
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
