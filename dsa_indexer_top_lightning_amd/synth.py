"""Seeded synthetic inputs for the DSA lightning-indexer -> top-k -> sparse-MLA path.

This module draws numbers and stores them; it holds none of the method's
arithmetic (no index score, no selection, no attention).  It is the only code
shared by the CPU oracle side (tests) and the GPU side (tests, bench, smoke).

Input recipe (the workloads of the pages, restated as shapes):
  * Every tensor with a token axis is drawn in blocks of ``BLOCK_ROWS`` rows from
    ``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id, layer, b, block])))``
    so that any block can be regenerated alone (the oracle samples rows of
    tensors that do not fit host memory as float64).
  * Normal draws are float32 ``standard_normal``; head weights are float32
    ``random`` (U[0,1)).
  * Index q/k may get rotate-half RoPE on the last D/2 dims of each head (the
    Megatron-Bridge page, commit on the indexer RoPE half swap: Megatron rotates
    the LAST ``qk_pos_emb_head_dim`` dims; ``rope_theta`` = 8e6 from the same
    page's config fix), computed in float64.
  * Storage: fp32 as is; bf16 by round-to-nearest-even of the float32 bits;
    fp8 as OCP e4m3fn codes with one float32 scale per (token, head) vector of
    D values, ``scale = float32(amax / 448)``, codes by round-to-nearest-even
    with saturation at +-448.
  * Packed variable-length batch (``seqlens``): B = 1 and the sequences lie end to
    end on the token axis; a query sees the keys of its own sequence up to itself
    ([first token of its sequence, its position]) and RoPE positions restart at 0 in
    every sequence.
  * Planted keys (1M-context decode workload): a Bernoulli(p) subset of key
    positions gets ``k += gamma * sqrt(D) * u_h`` with gamma ~ U(0.5, 1.5) and
    u_h the unit index query of head h (Hk == H) or of sum_h w_h q_h (Hk == 1),
    added in float64 before quantisation.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

BLOCK_ROWS = 4096
ROPE_THETA = 8.0e6

# tensor ids of the block seeds
TID_IDX_Q, TID_IDX_K, TID_IDX_W, TID_MLA_Q, TID_MLA_KV, TID_PLANT_POS, TID_PLANT_GAMMA, TID_SCORES = 1, 2, 3, 4, 5, 6, 7, 8

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic workload.

    Query (b, t) sits at absolute position ``pos0 + t`` and sees the causal
    candidate set [0, pos0 + t] of a prefix of ``S`` keys.
    """
    name: str
    B: int
    T: int
    S: int
    pos0: int
    layers: str            # one char per layer: 'F' full, 'S' shared
    H: int                 # index heads
    D: int                 # index head dim
    Hk: int                # index key heads (H or 1)
    topk: int
    Hm: int                # MLA heads
    Dc: int                # latent rank (value dims)
    Dr: int                # rope dims of the latent row
    idx_dtype: str         # 'f32' | 'bf16' | 'fp8'
    mla_dtype: str         # 'f32' | 'bf16'
    seed: int
    rope: bool = False
    plant_frac: float = 0.0
    seqlens: tuple = ()    # packed variable-length batch: sequence lengths laid end to end (B == 1)

    def __post_init__(self):
        if self.seqlens:
            n = int(sum(self.seqlens))
            if self.B != 1 or self.pos0 != 0 or self.T != n or self.S != n or min(self.seqlens) < 1:
                raise ValueError("a packed batch has B = 1, pos0 = 0 and T = S = sum(seqlens), every length >= 1")

    @property
    def n_layers(self) -> int:
        return len(self.layers)

    @property
    def row(self) -> int:
        return self.Dc + self.Dr

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.Dc + self.Dr)

    def key_end(self) -> np.ndarray:
        """Exclusive causal end of every query's candidate range, int32 [B, T]."""
        t = np.arange(self.T, dtype=np.int64)
        ke = np.minimum(self.pos0 + t + 1, self.S)
        return np.broadcast_to(ke, (self.B, self.T)).astype(np.int32).copy()

    def seq_offsets(self) -> np.ndarray:
        """Packed batch: first packed position of each token's sequence, int64 [T]."""
        cu = np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int64)
        return np.repeat(cu[:-1], self.seqlens)

    def key_start(self) -> np.ndarray:
        """Start of every query's candidate range, int32 [B, T]: 0, or in a packed batch the
        first token of the query's own sequence (causal attention stays inside it)."""
        if self.seqlens:
            return self.seq_offsets().astype(np.int32)[None].copy()
        return np.zeros((self.B, self.T), np.int32)

    def positions(self, r0: int, r1: int, queries: bool) -> np.ndarray:
        """Positions of tokens [r0, r1) used by RoPE: absolute (queries start at pos0), or in a
        packed batch the position inside the token's own sequence."""
        if self.seqlens:
            return np.arange(r0, r1) - self.seq_offsets()[r0:r1]
        return (self.pos0 if queries else 0) + np.arange(r0, r1)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


PACKED_SEQLENS = (3000, 2049, 2048, 1500, 1000, 700, 511, 300, 256, 255, 129, 100, 65, 64, 33, 17, 9, 1)

# The workloads (shapes from the pages' settings: 4096-token synthetic
# pre-training sequences, index_topk 2048, 1M context, MLA latent 512 + 64).
WORKLOADS = {
    "tiny_prefill256_fp32": Workload(
        "tiny_prefill256_fp32", B=1, T=256, S=256, pos0=0, layers="FSSS", H=4, D=32, Hk=4,
        topk=32, Hm=8, Dc=64, Dr=16, idx_dtype="f32", mla_dtype="f32", seed=0),
    "prefill4k_bf16": Workload(
        "prefill4k_bf16", B=1, T=4096, S=4096, pos0=0, layers="FSSS", H=32, D=128, Hk=32,
        topk=2048, Hm=64, Dc=512, Dr=64, idx_dtype="bf16", mla_dtype="bf16", seed=1, rope=True),
    "decode32k_b64_bf16": Workload(
        "decode32k_b64_bf16", B=64, T=1, S=32768, pos0=32767, layers="FFFSSSFS", H=32, D=128,
        Hk=32, topk=2048, Hm=64, Dc=512, Dr=64, idx_dtype="bf16", mla_dtype="bf16", seed=2),
    "chunk128k_fp8": Workload(
        "chunk128k_fp8", B=1, T=4096, S=131072, pos0=126976, layers="FSSS", H=32, D=128,
        Hk=32, topk=2048, Hm=64, Dc=512, Dr=64, idx_dtype="fp8", mla_dtype="bf16", seed=3),
    # packed variable-length batch (the pages' RL-rollout / thd layout): 18 sequences end to
    # end, from a single token to longer than index_topk, so that many rows pad with -1
    "packed_varlen_bf16": Workload(
        "packed_varlen_bf16", B=1, T=sum(PACKED_SEQLENS), S=sum(PACKED_SEQLENS), pos0=0, layers="FSS", H=32,
        D=128, Hk=32, topk=2048, Hm=64, Dc=512, Dr=64, idx_dtype="bf16", mla_dtype="bf16", seed=5, rope=True,
        seqlens=PACKED_SEQLENS),
    "decode1m_b4_fp8": Workload(
        "decode1m_b4_fp8", B=4, T=1, S=1048576, pos0=1048575, layers="FSSS", H=32, D=128,
        Hk=32, topk=2048, Hm=64, Dc=512, Dr=64, idx_dtype="fp8", mla_dtype="bf16", seed=4,
        plant_frac=0.05),
}


# ---------------------------------------------------------------- storage codecs
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f64_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float64 -> OCP e4m3fn codes (uint8): round to nearest even, saturate at +-448."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.minimum(np.abs(x), E4M3_MAX)
    code = np.zeros(a.shape, np.int64)
    sub = a < 2.0 ** -6
    # subnormals: m * 2^-9, m in 0..8 (m == 8 is the smallest normal, code 8)
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    nrm = ~sub
    if nrm.any():
        f, e = np.frexp(a[nrm])                # a = f * 2^e, f in [0.5, 1)
        m = np.rint(f * 16.0 - 8.0).astype(np.int64)   # 3-bit mantissa, RNE
        ee = (e - 1).astype(np.int64)
        carry = m == 8
        m[carry] = 0
        ee[carry] += 1
        code[nrm] = ((ee + 7) << 3) | m
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_fp8_rows(x: np.ndarray):
    """Quantise float64 [..., D] vectors: per-vector float32 scale amax/448 and e4m3fn codes."""
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / E4M3_MAX).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = f64_to_e4m3_codes(x / scale.astype(np.float64)[..., None])
    return codes, scale


def store(x64: np.ndarray, dtype: str):
    """Round float values to the storage type. Returns (stored array, scale or None)."""
    if dtype == "f32":
        return np.asarray(x64, dtype=np.float32), None
    if dtype == "bf16":
        return f32_to_bf16_bits(np.asarray(x64, dtype=np.float32)), None
    if dtype == "fp8":
        return quantize_fp8_rows(np.asarray(x64, dtype=np.float64))
    raise ValueError(dtype)


# ---------------------------------------------------------------- block draws
def _rng(seed, tid, layer, b, block):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, layer, b, block])))


def draw_rows(seed, tid, layer, b, r0, r1, row_elems, kind="normal"):
    """Rows [r0, r1) of a blocked float32 draw with ``row_elems`` values per row."""
    out = np.empty((max(r1 - r0, 0), row_elems), np.float32)
    if r1 <= r0:
        return out
    for blk in range(r0 // BLOCK_ROWS, (r1 - 1) // BLOCK_ROWS + 1):
        b0 = blk * BLOCK_ROWS
        g = _rng(seed, tid, layer, b, blk)
        if kind == "normal":
            vals = g.standard_normal((BLOCK_ROWS, row_elems), dtype=np.float32)
        else:
            vals = g.random((BLOCK_ROWS, row_elems), dtype=np.float32)
        lo, hi = max(r0, b0), min(r1, b0 + BLOCK_ROWS)
        out[lo - r0:hi - r0] = vals[lo - b0:hi - b0]
    return out


def rope_last_half(x: np.ndarray, pos: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate-half RoPE on the last D/2 dims of [..., rows, heads, D] float64 vectors.

    ``pos`` holds one absolute position per row. Pairs (i, i + D/4) inside the
    rope part are rotated by pos * theta^(-2i/(D/2)).
    """
    D = x.shape[-1]
    r = D // 2
    half = r // 2
    inv = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / r)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]          # [rows, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    y = x.astype(np.float64, copy=True)
    a = x[..., D - r:D - r + half].astype(np.float64)
    bb = x[..., D - r + half:].astype(np.float64)
    y[..., D - r:D - r + half] = a * c - bb * s
    y[..., D - r + half:] = bb * c + a * s
    return y


# ---------------------------------------------------------------- tensors
def index_q_rows(w: Workload, layer: int, b: int, t0: int, t1: int):
    """Index queries of rows [t0, t1): float64 values [rows, H, D] before storage rounding."""
    x = draw_rows(w.seed, TID_IDX_Q, layer, b, t0, t1, w.H * w.D).reshape(-1, w.H, w.D).astype(np.float64)
    if w.rope:
        x = rope_last_half(x, w.positions(t0, t1, True))
    return x


def index_w_rows(w: Workload, layer: int, b: int, t0: int, t1: int) -> np.ndarray:
    """Head weights U[0,1) float32 [rows, H]."""
    return draw_rows(w.seed, TID_IDX_W, layer, b, t0, t1, w.H, kind="uniform")


def _plant_direction(w: Workload, layer: int, b: int) -> np.ndarray:
    """Unit planting direction per key head, float64 [Hk, D], from the query of row 0."""
    q = index_q_rows(w, layer, b, 0, 1)[0]                         # [H, D]
    if w.Hk == w.H:
        v = q
    else:
        wt = index_w_rows(w, layer, b, 0, 1)[0].astype(np.float64)
        v = (wt[:, None] * q).sum(axis=0, keepdims=True)
    n = np.sqrt((v * v).sum(axis=-1, keepdims=True))
    return v / np.where(n > 0, n, 1.0)


def index_k_rows(w: Workload, layer: int, b: int, s0: int, s1: int):
    """Index keys of positions [s0, s1): float64 [rows, Hk, D] before storage rounding."""
    x = draw_rows(w.seed, TID_IDX_K, layer, b, s0, s1, w.Hk * w.D).reshape(-1, w.Hk, w.D).astype(np.float64)
    if w.rope:
        x = rope_last_half(x, w.positions(s0, s1, False))
    if w.plant_frac > 0:
        u = draw_rows(w.seed, TID_PLANT_POS, layer, b, s0, s1, 1, kind="uniform")[:, 0]
        g = draw_rows(w.seed, TID_PLANT_GAMMA, layer, b, s0, s1, 1, kind="uniform")[:, 0]
        sel = u < w.plant_frac
        if sel.any():
            gamma = 0.5 + g[sel].astype(np.float64)
            dirn = _plant_direction(w, layer, b)                   # [Hk, D]
            x[sel] = x[sel] + (gamma * math.sqrt(w.D))[:, None, None] * dirn[None]
    return x


def mla_q_rows(w: Workload, layer: int, b: int, t0: int, t1: int) -> np.ndarray:
    return draw_rows(w.seed, TID_MLA_Q, layer, b, t0, t1, w.Hm * w.row).reshape(-1, w.Hm, w.row)


def mla_kv_rows(w: Workload, layer: int, b: int, s0: int, s1: int) -> np.ndarray:
    return draw_rows(w.seed, TID_MLA_KV, layer, b, s0, s1, w.row)


# ---------------------------------------------------------------- whole tensors
def _pool():
    n = min(16, os.cpu_count() or 1)
    return ThreadPoolExecutor(max_workers=n)


def _blocks(n):
    return [(r, min(n, r + BLOCK_ROWS)) for r in range(0, n, BLOCK_ROWS)]


def build_layer_inputs(w: Workload, layer: int, with_index: bool, with_mla: bool = True):
    """Stored (host) inputs of one layer for all batch items.

    Returns a dict with 'mla_q' [B,T,Hm,row], 'kv' [B,S,row] (unless with_mla is
    False) and, for layers that carry an indexer, 'idx_q' [B,T,H,D], 'idx_k'
    [B,S,Hk,D], 'w' [B,T,H] and fp8 scales 'idx_q_scale' [B,T,H], 'idx_k_scale'
    [B,S,Hk].  Storage arrays: float32, uint16 (bf16 bits) or uint8 (e4m3fn codes).
    """
    mdt = np.float32 if w.mla_dtype == "f32" else np.uint16
    out = {}
    jobs = []
    if with_mla:
        out["mla_q"] = np.empty((w.B, w.T, w.Hm, w.row), mdt)
        out["kv"] = np.empty((w.B, w.S, w.row), mdt)

    def fill_mq(b, t0, t1):
        out["mla_q"][b, t0:t1] = store(mla_q_rows(w, layer, b, t0, t1), w.mla_dtype)[0]

    def fill_kv(b, s0, s1):
        out["kv"][b, s0:s1] = store(mla_kv_rows(w, layer, b, s0, s1), w.mla_dtype)[0]

    for b in range(w.B if with_mla else 0):
        jobs += [(fill_mq, b, r0, r1) for r0, r1 in _blocks(w.T)]
        jobs += [(fill_kv, b, r0, r1) for r0, r1 in _blocks(w.S)]
    if with_index:
        idt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[w.idx_dtype]
        out["idx_q"] = np.empty((w.B, w.T, w.H, w.D), idt)
        out["idx_k"] = np.empty((w.B, w.S, w.Hk, w.D), idt)
        out["w"] = np.empty((w.B, w.T, w.H), np.float32)
        if w.idx_dtype == "fp8":
            out["idx_q_scale"] = np.empty((w.B, w.T, w.H), np.float32)
            out["idx_k_scale"] = np.empty((w.B, w.S, w.Hk), np.float32)

        def fill_q(b, t0, t1):
            v, sc = store(index_q_rows(w, layer, b, t0, t1), w.idx_dtype)
            out["idx_q"][b, t0:t1] = v
            if sc is not None:
                out["idx_q_scale"][b, t0:t1] = sc
            out["w"][b, t0:t1] = index_w_rows(w, layer, b, t0, t1)

        def fill_k(b, s0, s1):
            v, sc = store(index_k_rows(w, layer, b, s0, s1), w.idx_dtype)
            out["idx_k"][b, s0:s1] = v
            if sc is not None:
                out["idx_k_scale"][b, s0:s1] = sc

        for b in range(w.B):
            jobs += [(fill_q, b, r0, r1) for r0, r1 in _blocks(w.T)]
            jobs += [(fill_k, b, r0, r1) for r0, r1 in _blocks(w.S)]
    with _pool() as ex:
        for f in [ex.submit(j[0], *j[1:]) for j in jobs]:
            f.result()
    return out


def layer_has_index(w: Workload, layer: int) -> bool:
    return w.layers[layer] == "F"


def build_inputs(w: Workload):
    """Stored inputs of every layer (index inputs only on full layers)."""
    return [build_layer_inputs(w, l, layer_has_index(w, l)) for l in range(w.n_layers)]


def scores_for_topk(seed: int, rows: int, n: int, kind: str = "normal") -> np.ndarray:
    """float32 [rows, n] score rows for exercising top-k alone.

    kinds: 'normal' (continuous), 'ties' (few distinct values, many exact
    ties), 'zeros' (mostly exact +0.0/-0.0 with a sprinkle of positives),
    'mixed' (normal values with planted duplicate runs and signed zeros).
    """
    g = _rng(seed, TID_SCORES, 0, 0, 0)
    if kind == "normal":
        return g.standard_normal((rows, n), dtype=np.float32)
    if kind == "ties":
        return (g.integers(0, 7, (rows, n)).astype(np.float32) - 3.0) * np.float32(0.25)
    if kind == "zeros":
        x = np.where(g.random((rows, n)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        pos = g.random((rows, n)) < 0.01
        x[pos] = g.random(int(pos.sum()), dtype=np.float32) + np.float32(1.0)
        return x
    if kind == "mixed":
        x = g.standard_normal((rows, n), dtype=np.float32)
        dup = g.random((rows, n)) < 0.3
        x[dup] = np.round(x[dup] * 4) / 4
        z = g.random((rows, n)) < 0.05
        x[z] = np.where(g.random(int(z.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
        return x.astype(np.float32)
    raise ValueError(kind)
