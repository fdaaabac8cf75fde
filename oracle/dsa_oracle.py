"""Plain, slow, float64 CPU oracle of the DSA indexer -> top-k -> sparse MLA path
with GLM-5.2 cross-layer IndexShare.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module.  It shares no code with the HIP library
and imports nothing from it.

What it follows (the pages do not print the formulas; readings are marked):
  * GLM-5.2 IndexShare page, section 1 "What DSA does before sharing": per query,
    a light indexer scores the prefix tokens, the top-k positions are kept, and
    the main attention runs only over those positions.
  * Same page, section 2 "What IndexShare changes", the layer-pattern figure and
    the "What is actually shared?" table: full layers compute and cache the top-k
    indices; shared layers reuse the nearest preceding full layer's indices (only
    the indices are shared) and still compute their own attention.
  * Megatron-Bridge GLM-5 DSA pull request, commit fixing top-k for short packed
    sequences: when fewer candidates than index_topk exist, take them all and pad
    to the fixed index_topk width with -1.
  * Same pull request, commit on the wrong-dimension-count parse: the MLA latent
    row is kv_lora_rank 512 + qk_rope_head_dim 64 = 576 values.
  * MaxText "add glm5.2 indexshare" pull request, description and review thread:
    per-layer full/shared list, F layers active, S layers reuse the donor.
  Reading (the pages do not print it): index score
      I[t, s] = sum_h w[t, h] * max(0, q[t, h, :] . k[s, g(h), :]),
  g(h) = h when there is one key head per query head, else 0.  Top-k ties go to
  the lower position and the kept positions are listed in ascending order.
  Sparse MLA is the absorbed form: keys are whole latent rows (Dc + Dr values),
  values are their first Dc values.

Parity pins live in tests/test_oracle_pins.py.  Parity against values printed on
the pages is unpinned: the pages print no score, index or attention values.
"""
from __future__ import annotations

import math

import numpy as np

# ------------------------------------------------------------------ input decoding


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: a bf16 is the top half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def _e4m3fn_table() -> np.ndarray:
    """Value of every OCP e4m3fn code: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; there is no
    infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    vals = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3FN = _e4m3fn_table()


def decode(stored: np.ndarray, dtype: str, scale: np.ndarray | None = None) -> np.ndarray:
    """Stored input -> float64.  fp8 values are multiplied by their per-vector scale."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(stored)
    if dtype == "fp8":
        v = E4M3FN[np.asarray(stored, dtype=np.uint8)]
        if scale is not None:
            v = v * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
        return v
    raise ValueError(dtype)


# ------------------------------------------------------------------ indexer score


def index_scores_loop(q: np.ndarray, k: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Index score by explicit loops (tiny inputs only).

    q [T, H, D], k [S, Hk, D], w [T, H] (float64) -> I [T, S].
    """
    T, H, D = q.shape
    S, Hk, _ = k.shape
    out = np.zeros((T, S))
    for t in range(T):
        for s in range(S):
            acc = 0.0
            for h in range(H):
                g = h if Hk == H else 0
                dot = 0.0
                for d in range(D):
                    dot += q[t, h, d] * k[s, g, d]
                acc += w[t, h] * max(dot, 0.0)
            out[t, s] = acc
    return out


def index_scores_row(q_row: np.ndarray, k: np.ndarray, w_row: np.ndarray,
                     key_start: int, key_end: int) -> np.ndarray:
    """Index scores of one query over its candidates [key_start, key_end).

    q_row [H, D], k [S, Hk, D], w_row [H] (float64) -> [key_end - key_start].
    """
    H = q_row.shape[0]
    kk = k[key_start:key_end]                                   # [n, Hk, D]
    if kk.shape[1] == H:
        # per head: keys of that head [n, D] times its query [D]
        dots = np.matmul(np.ascontiguousarray(kk.transpose(1, 0, 2)), q_row[:, :, None])[:, :, 0].T
    else:
        dots = kk[:, 0, :] @ q_row.T                            # [n, H]
    return np.maximum(dots, 0.0) @ w_row


def index_scores_rows(q_rows: np.ndarray, k: np.ndarray, w_rows: np.ndarray) -> np.ndarray:
    """Index scores of several queries of one batch item against the same keys.

    q_rows [R, H, D], k [n, Hk, D], w_rows [R, H] (float64) -> [R, n].  The same
    definition as index_scores_row, summed head by head: for head h the dot
    products of all R queries with all n keys of key head g(h), ReLU, times the
    head weight of each query.
    """
    R, H, _ = q_rows.shape
    Hk = k.shape[1]
    out = np.zeros((R, k.shape[0]))
    for h in range(H):
        g = h if Hk == H else 0
        dots = q_rows[:, h, :] @ k[:, g, :].T                   # [R, n]
        out += w_rows[:, h][:, None] * np.maximum(dots, 0.0)
    return out


def index_scores(q: np.ndarray, k: np.ndarray, w: np.ndarray,
                 key_start: np.ndarray, key_end: np.ndarray) -> np.ndarray:
    """q [B,T,H,D], k [B,S,Hk,D], w [B,T,H] -> I [B,T,S], NaN outside each candidate range."""
    B, T = q.shape[:2]
    S = k.shape[1]
    out = np.full((B, T, S), np.nan)
    for b in range(B):
        for t in range(T):
            ks, ke = int(key_start[b, t]), int(key_end[b, t])
            out[b, t, ks:ke] = index_scores_row(q[b, t], k[b], w[b, t], ks, ke)
    return out


def index_scores_backward_selected(q: np.ndarray, k: np.ndarray, w: np.ndarray, idx: np.ndarray,
                                   dI: np.ndarray):
    """Gradient of the index scores at the selected positions, by the chain rule through
    I[t, s] = sum_h w[t, h] max(0, q[t, h] . k[s, g(h)]) (section 1 of the IndexShare page;
    reading as in index_scores).  q [B,T,H,D] and k [B,S,Hk,D] are the dequantised inputs,
    w [B,T,H]; dI [B,T,kk] is a loss gradient with respect to I[b, t, idx[b, t, j]] (slots
    whose position lies outside [0, S) are ignored).  With s = q[t,h] . k[j,g(h)]:

        dw[t, h]      = sum_j dI_j max(0, s)
        dq[t, h]      = sum_j dI_j w[t, h] [s > 0] k[j, g(h)]
        dk[j, g(h)]  += dI_j w[t, h] [s > 0] q[t, h]

    The derivative of max(0, s) at s = 0 is taken as 0.  Returns (dq, dk, dw) float64."""
    B, T, H, D = q.shape
    S, Hk = k.shape[1], k.shape[2]
    g = np.arange(H) if Hk == H else np.zeros(H, np.int64)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dw = np.zeros(w.shape)
    for b in range(B):
        for t in range(T):
            sel = np.asarray(idx[b, t], dtype=np.int64)
            ok = (sel >= 0) & (sel < S)
            sel, gr = sel[ok], np.asarray(dI[b, t], dtype=np.float64)[ok]
            if sel.size == 0:
                continue
            kk = k[b][sel][:, g, :]                                   # [J, H, D]
            sc = np.einsum("hd,jhd->jh", q[b, t], kk)                 # [J, H]
            on = sc > 0
            dw[b, t] = (gr[:, None] * np.where(on, sc, 0.0)).sum(axis=0)
            coef = gr[:, None] * w[b, t][None, :] * on                # [J, H]
            dq[b, t] = np.einsum("jh,jhd->hd", coef, kk)
            contrib = coef[:, :, None] * q[b, t][None, :, :]          # [J, H, D]
            if Hk == H:
                np.add.at(dk[b], sel, contrib)
            else:
                np.add.at(dk[b], sel, contrib.sum(axis=1, keepdims=True))
    return dq, dk, dw


# ------------------------------------------------------------------ top-k


def topk_row(scores: np.ndarray, key_start: int, key_end: int, k: int):
    """Top-k of one row by a full stable sort.

    ``scores`` holds the candidates' scores in position order (length
    key_end - key_start; a longer array is cut to it).  Returns (indices int32
    [k], tau): the chosen absolute positions in ascending order followed by -1,
    and the k-th largest score (None when every candidate is taken).
    """
    n = max(key_end - key_start, 0)
    s = np.asarray(scores, dtype=np.float64)[:n]
    out = np.full(k, -1, np.int32)
    if n <= k:
        out[:n] = np.arange(key_start, key_end, dtype=np.int32)
        return out, None
    pos = np.arange(key_start, key_end, dtype=np.int64)
    order = np.lexsort((pos, -s))           # score descending, then position ascending
    keep = order[:k]
    tau = s[order[k - 1]]
    out[:] = np.sort(pos[keep]).astype(np.int32)
    return out, float(tau)


def topk(scores: np.ndarray, key_start: np.ndarray, key_end: np.ndarray, k: int):
    """scores [B,T,S] (absolute positions) -> (indices [B,T,k] int32, tau [B,T] with NaN where n <= k)."""
    B, T = scores.shape[:2]
    idx = np.full((B, T, k), -1, np.int32)
    tau = np.full((B, T), np.nan)
    for b in range(B):
        for t in range(T):
            ks, ke = int(key_start[b, t]), int(key_end[b, t])
            i, tt = topk_row(scores[b, t, ks:ke], ks, ke, k)
            idx[b, t] = i
            if tt is not None:
                tau[b, t] = tt
    return idx, tau


# ------------------------------------------------------------------ sparse MLA


def sparse_mla_row(q_row: np.ndarray, kv: np.ndarray, idx: np.ndarray, sm_scale: float, Dc: int):
    """Attention of one query over the listed latent rows (gather form).

    q_row [Hm, R], kv [S, R], idx [k] (entries outside [0, S) are skipped).
    Returns (o [Hm, Dc], lse [Hm]); an empty selection gives o = 0, lse = -inf.
    """
    S = kv.shape[0]
    sel = np.asarray(idx, dtype=np.int64)
    sel = sel[(sel >= 0) & (sel < S)]
    Hm = q_row.shape[0]
    if sel.size == 0:
        return np.zeros((Hm, Dc)), np.full(Hm, -np.inf)
    c = kv[sel]                                                 # [J, R]
    z = sm_scale * (q_row @ c.T)                                # [Hm, J]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e / l) @ c[:, :Dc]
    lse = (m + np.log(l))[:, 0]
    return o, lse


def sparse_mla_dense_masked_row(q_row: np.ndarray, kv: np.ndarray, idx: np.ndarray,
                                sm_scale: float, Dc: int):
    """Same attention in the dense-masked form: logits over all S rows, -inf off the selection.

    (The MaxText path carries the selection as an indexer mask over the prefix.)
    Each position counts once even if listed twice.
    """
    S = kv.shape[0]
    sel = np.asarray(idx, dtype=np.int64)
    sel = sel[(sel >= 0) & (sel < S)]
    Hm = q_row.shape[0]
    mask = np.zeros(S, bool)
    mask[sel] = True
    if not mask.any():
        return np.zeros((Hm, Dc)), np.full(Hm, -np.inf)
    z = sm_scale * (q_row @ kv.T)                               # [Hm, S]
    z = np.where(mask[None, :], z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ kv[:, :Dc], (m + np.log(l))[:, 0]


def sparse_mla(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, sm_scale: float, Dc: int):
    """q [B,T,Hm,R], kv [B,S,R], idx [B,T,k] -> (o [B,T,Hm,Dc], lse [B,T,Hm])."""
    B, T, Hm, _ = q.shape
    o = np.zeros((B, T, Hm, Dc))
    lse = np.zeros((B, T, Hm))
    for b in range(B):
        for t in range(T):
            o[b, t], lse[b, t] = sparse_mla_row(q[b, t], kv[b], idx[b, t], sm_scale, Dc)
    return o, lse


def sparse_mla_backward_row(q_row: np.ndarray, kv: np.ndarray, idx: np.ndarray, sm_scale: float, Dc: int,
                            dout_row: np.ndarray):
    """Gradient of one query's sparse attention (sparse_mla_row) for an output
    gradient dout_row [Hm, Dc], by the chain rule through the definition: the
    selection is a constant (no gradient flows through top-k), P = softmax(z) over the
    selected rows, z = sm_scale * q . c_j, o = sum_j P_j c_j[:Dc].

        dP_j = dout . c_j[:Dc]         D = dout . o = sum_j P_j dP_j
        dz_j = P_j (dP_j - D)
        dq   = sm_scale sum_j dz_j c_j
        dc_j = sm_scale dz_j q + [P_j dout, 0]   (summed over heads)

    Returns (dq_row [Hm, R], rows [J], dc [J, R]); an empty selection gives zeros."""
    S, R = kv.shape
    sel = np.asarray(idx, dtype=np.int64)
    sel = sel[(sel >= 0) & (sel < S)]
    Hm = q_row.shape[0]
    if sel.size == 0:
        return np.zeros((Hm, R)), sel, np.zeros((0, R))
    c = kv[sel]                                                 # [J, R]
    z = sm_scale * (q_row @ c.T)                                # [Hm, J]
    e = np.exp(z - z.max(axis=1, keepdims=True))
    P = e / e.sum(axis=1, keepdims=True)
    o = P @ c[:, :Dc]                                           # [Hm, Dc]
    dP = dout_row @ c[:, :Dc].T                                 # [Hm, J]
    D = (dout_row * o).sum(axis=1, keepdims=True)               # [Hm, 1]
    dz = P * (dP - D)
    dq = sm_scale * (dz @ c)                                    # [Hm, R]
    dc = sm_scale * (dz.T @ q_row)                              # [J, R]
    dc[:, :Dc] += P.T @ dout_row
    return dq, sel, dc


def sparse_mla_backward(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, sm_scale: float, Dc: int,
                        dout: np.ndarray):
    """q [B,T,Hm,R], kv [B,S,R], idx [B,T,k], dout [B,T,Hm,Dc] -> (dq [B,T,Hm,R], dkv [B,S,R]);
    a row selected by several queries (or listed twice) collects every contribution."""
    B, T = q.shape[:2]
    dq = np.zeros(q.shape)
    dkv = np.zeros(kv.shape)
    for b in range(B):
        for t in range(T):
            dq[b, t], sel, dc = sparse_mla_backward_row(q[b, t], kv[b], idx[b, t], sm_scale, Dc, dout[b, t])
            np.add.at(dkv[b], sel, dc)
    return dq, dkv


# ------------------------------------------------------------------ IndexShare


class NoDonorError(ValueError):
    """A shared layer has no preceding full layer and no valid cached indices."""


class StaleCacheError(ValueError):
    """Cached indices were produced for another call (tag or shape mismatch)."""


def parse_pattern(pattern: str, n_layers: int):
    """Repeat a full/shared pattern string such as "FSSS" over n_layers layers."""
    p = pattern.upper()
    if not p or set(p) - {"F", "S"}:
        raise ValueError(pattern)
    return ["full" if p[i % len(p)] == "F" else "shared" for i in range(n_layers)]


def donor_map(types, cache_valid: bool = False):
    """donor[l] = the nearest full layer j <= l.  A leading shared layer takes the
    cached indices (donor -1) if ``cache_valid``; otherwise it has no donor."""
    donors, last = [], None
    for l, ty in enumerate(types):
        if ty == "full":
            last = l
        elif ty != "shared":
            raise ValueError(ty)
        if last is None:
            if not cache_valid:
                raise NoDonorError(f"layer {l} is shared and has no preceding full layer")
            donors.append(-1)
        else:
            donors.append(last)
    return donors


def served_group_sizes(types):
    """Number of layers (itself included) that use each full layer's indices."""
    donors = donor_map(types)
    return [sum(1 for d in donors if d == l) for l, ty in enumerate(types) if ty == "full"]


def group_forward(layers, types, key_start, key_end, topk_k, sm_scale, Dc, cache=None, tag=0):
    """Whole layer group.

    ``layers[l]`` is a dict of float64 inputs: 'mla_q' [B,T,Hm,R], 'kv' [B,S,R]
    and, on full layers, 'idx_q' [B,T,H,D], 'idx_k' [B,S,Hk,D], 'w' [B,T,H].
    ``cache`` is None or a dict {'indices', 'tag'} carried from an earlier call.
    Returns dict(indices=[per layer], out=[...], lse=[...], donors=[...], cache=...).
    """
    donors = donor_map(types, cache_valid=cache is not None)
    if types and types[0] == "shared":
        if cache is None:
            raise NoDonorError("first layer is shared and there is no cached indices")
        if cache["tag"] != tag or cache["indices"].shape != (key_end.shape[0], key_end.shape[1], topk_k):
            raise StaleCacheError("cached indices belong to another call")
    cur = None if cache is None else cache["indices"]
    res = {"indices": [], "out": [], "lse": [], "donors": donors}
    for l, ty in enumerate(types):
        L = layers[l]
        if ty == "full":
            sc = index_scores(L["idx_q"], L["idx_k"], L["w"], key_start, key_end)
            cur, _ = topk(sc, key_start, key_end, topk_k)
        o, lse = sparse_mla(L["mla_q"], L["kv"], cur, sm_scale, Dc)
        res["indices"].append(cur)
        res["out"].append(o)
        res["lse"].append(lse)
    res["cache"] = {"indices": cur, "tag": tag}
    return res


def group_stats(types, key_start, key_end, *, H, D, Hk, idx_bytes, idx_scaled, topk_k,
                Hm, Dc, Dr, mla_bytes, S):
    """Analytic work of one group call (counts, not timings).

    indexer_flops  = 2*H*D per (query, candidate) pair, per full layer
    indexer_bytes  = index q + w (+ q scales) + index k of each item's prefix
                     (+ k scales) + fp32 scores written, per full layer
    topk_bytes     = fp32 scores read + int32 indices written, per full layer
    attn_flops     = 2*Hm*(2*Dc + Dr) per (query, selected row), per layer
    attn_bytes     = gathered rows + q read + out written, per layer
    """
    ks = np.asarray(key_start, np.int64)
    ke = np.asarray(key_end, np.int64)
    n = np.maximum(ke - ks, 0)
    rows = n.size
    B = ke.shape[0]
    sum_n = int(n.sum())
    sum_j = int(np.minimum(n, topk_k).sum())
    prefix = int(np.minimum(ke.max(axis=1), S).sum()) if rows else 0
    n_full = sum(1 for t in types if t == "full")
    n_sh = len(types) - n_full
    sc = 4 if idx_scaled else 0
    idx_b = rows * H * (D * idx_bytes + 4 + sc) + prefix * Hk * (D * idx_bytes + sc) + 4 * sum_n
    R = Dc + Dr
    return {
        "n_full": n_full,
        "n_shared": n_sh,
        "indexer_flops": float(n_full * 2 * H * D * sum_n),
        "indexer_bytes": float(n_full * idx_b),
        "topk_bytes": float(n_full * (4 * sum_n + 4 * rows * topk_k)),
        "attn_flops": float(len(types) * 2 * Hm * (2 * Dc + Dr) * sum_j),
        "attn_bytes": float(len(types) * (sum_j * R * mla_bytes + rows * Hm * R * mla_bytes
                                          + rows * Hm * Dc * mla_bytes)),
        "batch": B,
    }


# ------------------------------------------------------------------ decode-step preparation
# The steps a decode step applies to new index vectors before they are scored:
# Megatron-Bridge GLM-5 DSA pull request, commit on the indexer RoPE half swap (the
# rotated dims are the LAST qk_pos_emb_head_dim = D/2 of each index head), its config
# fix (rope_theta = 8e6), and fp8 e4m3 storage with one fp32 scale per vector.
# Reading: rotate-half pairs (i, i + D/4) inside the rope part turn by
# pos * theta^(-2i / (D/2)); the rotated vector is a float32 tensor (the value a
# projection in float32 would hold); fp8 storage takes scale = float32(amax / 448)
# (1 when amax is 0) and codes = nearest e4m3fn value of float32(y / scale), ties to
# the even code, magnitudes above 448 saturated; bf16 storage rounds to nearest even.


def rope_last_half(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE of the last D/2 dims of every vector of x [N, heads, D], float64."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    r = D // 2
    half = r // 2
    inv = float(theta) ** (-(2.0 * np.arange(half)) / r)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]      # [N, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = x[..., D - r:D - r + half]
    b = x[..., D - r + half:]
    y = x.copy()
    y[..., D - r:D - r + half] = a * c - b * s
    y[..., D - r + half:] = b * c + a * s
    return y


def encode_e4m3(v32: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3fn codes: the nearest finite e4m3fn value (ties to the even
    code, i.e. even mantissa), magnitudes above 448 saturated to 448."""
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    grid = E4M3FN[:127]                       # codes 0..126: the non-negative finite values, ascending
    a = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = grid[hi] - a
    d_lo = a - grid[lo]
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(take_lo, lo, hi).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 7)


def encode_bf16(v32: np.ndarray) -> np.ndarray:
    """float32 values (finite) -> bf16 bit patterns: keep the top 16 bits of the float32,
    rounding the dropped 16 bits to nearest, ties to an even kept part."""
    u = np.asarray(v32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    top = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((top & 1) == 1))
    return (top + up).astype(np.uint16)


def quantize_e4m3_f32(y32: np.ndarray):
    """float32 vectors [..., D] -> (e4m3fn codes, float32 scale per vector)."""
    y = np.asarray(y32, dtype=np.float32)
    amax = np.max(np.abs(y), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return encode_e4m3((y / scale[..., None]).astype(np.float32)), scale


def prep_index_vectors(x32: np.ndarray, pos: np.ndarray, theta: float, dtype: str):
    """New index vectors [N, heads, D] float32 -> stored values after RoPE:
    bf16 bit patterns (scale None) or (e4m3fn codes, scales [N, heads])."""
    y = rope_last_half(x32, pos, theta).astype(np.float32)
    if dtype == "bf16":
        return encode_bf16(y), None
    if dtype == "fp8":
        return quantize_e4m3_f32(y)
    raise ValueError(dtype)


def cache_append(k_cache, k_scale, kv_cache, k_new, pos, rows, theta, dtype, kv_new=None):
    """Decode-step append: returns new (k_cache, k_scale, kv_cache) with token n's prepared
    index key at row rows[n] and its latent row copied there; rows outside the cache are
    skipped.  Caches are flat over rows: k [rows, Hk, D], scales [rows, Hk], kv [rows, R]."""
    k_cache = np.array(k_cache, copy=True)
    k_scale = None if k_scale is None else np.array(k_scale, copy=True)
    kv_cache = None if kv_cache is None else np.array(kv_cache, copy=True)
    vals, sc = prep_index_vectors(k_new, pos, theta, dtype)
    for n, r in enumerate(np.asarray(rows, dtype=np.int64)):
        if not 0 <= r < k_cache.shape[0]:
            continue
        k_cache[r] = vals[n]
        if sc is not None:
            k_scale[r] = sc[n]
        if kv_cache is not None and kv_new is not None:
            kv_cache[r] = kv_new[n]
    return k_cache, k_scale, kv_cache
