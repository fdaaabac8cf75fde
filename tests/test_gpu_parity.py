"""GPU parity: each C-ABI entry point against the CPU oracle on the same seeded inputs.

Bars: top-k indices bit-exact (with the GPU's own inputs: exactly; through the
indexer: identical except inside the 1e-3 relative tie band around the k-th
score); attention max-abs-relative error <= 1e-5 (fp32) / 2e-2 (bf16); index
scores within 2e-5 * sum_h |w| sum_d |q k| of the float64 value (fp32
accumulation of exact products).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from dsa_indexer_top_lightning_amd import binding as b
from dsa_indexer_top_lightning_amd import synth
from helpers import ATTN_TOL, check_topk_row, decode_index, f32_dev, i32_dev, index_abs_bound, max_abs_rel, to_dev

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="t", B=1, T=64, S=64, pos0=0, layers="FSSS", H=32, D=128, Hk=32, topk=64, Hm=64, Dc=512,
                Dr=64, idx_dtype="bf16", mla_dtype="bf16", seed=7)
    base.update(kw)
    return synth.Workload(**base)


# ------------------------------------------------------------------ indexer

INDEXER_CASES = {
    "fp32_tiny": dict(B=1, T=256, S=256, H=4, D=32, Hk=4, idx_dtype="f32", mla_dtype="f32", Hm=8, Dc=64, Dr=16),
    "bf16_ragged": dict(B=2, T=70, S=150, pos0=80, rope=True),
    "bf16_shared_key": dict(B=2, T=70, S=150, pos0=80, Hk=1),
    "fp8_ragged": dict(B=2, T=70, S=150, pos0=80, idx_dtype="fp8"),
    "fp8_shared_key": dict(B=1, T=33, S=200, pos0=167, Hk=1, idx_dtype="fp8"),
    "bf16_decode": dict(B=3, T=1, S=300, pos0=299),
    "fp8_decode_planted": dict(B=2, T=1, S=700, pos0=699, idx_dtype="fp8", plant_frac=0.05),
    "bf16_generic_d64": dict(B=1, T=40, S=90, pos0=50, D=64, H=8, Hk=8),
    # decode streaming kernel: shared key head, 16 / 64 heads, several queries per item
    "bf16_decode_shared_key": dict(B=2, T=1, S=300, pos0=299, Hk=1),
    "fp8_decode_shared_key_h64": dict(B=2, T=1, S=257, pos0=256, H=64, Hk=1, idx_dtype="fp8"),
    "bf16_decode_h16_t3": dict(B=2, T=3, S=130, pos0=127, H=16, Hk=16),
    "fp8_decode_h64_t4": dict(B=1, T=4, S=1000, pos0=996, H=64, Hk=64, idx_dtype="fp8"),
    # between decode and prefill tiles
    "bf16_t8": dict(B=2, T=8, S=100, pos0=92),
    # prefill over its own prefix with a square 3 x 3 grid of 128 x 128 tiles (walked lower
    # triangle first) and a ragged last tile; fp8 as well (its own tile kernel)
    "bf16_square_prefill": dict(B=2, T=300, S=300, pos0=0),
    "fp8_square_prefill": dict(B=1, T=300, S=300, pos0=0, idx_dtype="fp8"),
}


@pytest.mark.parametrize("case", sorted(INDEXER_CASES))
@pytest.mark.parametrize("window", [False, True])
def test_indexer_scores_match_oracle(case, window):
    w = _wl(**INDEXER_CASES[case])
    L = synth.build_layer_inputs(w, 0, True)
    ke = w.key_end()
    ks = np.maximum(ke - 37, 0).astype(np.int32) if window else w.key_start()
    ld = w.S + 5
    q = to_dev(L["idx_q"], w.idx_dtype)
    k = to_dev(L["idx_k"], w.idx_dtype)
    qs = f32_dev(L["idx_q_scale"]) if w.idx_dtype == "fp8" else None
    kss = f32_dev(L["idx_k_scale"]) if w.idx_dtype == "fp8" else None
    scores = torch.full((w.B, w.T, ld), float("nan"), device="cuda")
    b.indexer_scores(q, k, f32_dev(L["w"]), scores, q_scale=qs, k_scale=kss, key_start=i32_dev(ks),
                     key_end=i32_dev(ke))
    got = scores.cpu().numpy()
    q64, k64, w64 = decode_index(L, w)
    for bb in range(w.B):
        ref = O.index_scores(q64[bb:bb + 1], k64[bb:bb + 1], w64[bb:bb + 1], ks[bb:bb + 1], ke[bb:bb + 1])[0]
        bound = 2e-5 * index_abs_bound(q64[bb], k64[bb], w64[bb], w.Hk) + 1e-30
        mask = ~np.isnan(ref)
        g = got[bb, :, :w.S]
        assert np.isnan(g[~mask]).all(), "cells outside the candidate ranges were written"
        assert np.isnan(got[bb, :, w.S:]).all()
        err = np.abs(g[mask] - ref[mask])
        assert (err <= bound[mask]).all(), f"max err {err.max()} vs bound {bound[mask][np.argmax(err)]}"


# ------------------------------------------------------------------ top-k

TOPK_CASES = [
    # (rows B x T, s_cap, topk, kind)
    ((2, 40), 300, 32, "normal"),
    ((1, 64), 5000, 2048, "normal"),
    ((1, 64), 5000, 2048, "ties"),
    ((2, 16), 3000, 100, "zeros"),
    ((1, 48), 4096, 2048, "mixed"),
    ((1, 6), 40000, 2048, "mixed"),      # few long rows: chunked over workgroups
    ((3, 1), 33000, 2048, "normal"),
    ((2, 5), 100000, 2048, "ties"),
    ((1, 3), 70001, 2048, "zeros"),
    ((1, 7), 20000, 512, "mixed"),
    ((4, 1), 1 << 20, 2048, "normal"),   # 1M-key rows
    ((1, 512), 40000, 2048, "normal"),   # many rows longer than the LDS key cache: two reads per row
    ((1, 520), 70001, 1000, "mixed"),    # odd row length (unaligned rows), ties at the k-th key
    ((2, 300), 50001, 2048, "ties"),     # the k-th key's digit holds too many keys: HBM passes
    ((1, 512), 36000, 2048, "zeros"),
    ((1, 512), 300000, 2048, "ties"),    # many rows longer than the two-read path: radix passes over HBM
]


@pytest.mark.parametrize("rows,s_cap,k,kind", TOPK_CASES)
def test_topk_is_bit_exact(rows, s_cap, k, kind):
    B, T = rows
    sc = synth.scores_for_topk(s_cap + B * T + k, B * T, s_cap, kind).reshape(B, T, s_cap)
    rng = np.random.default_rng(s_cap + k)
    ke = rng.integers(0, s_cap + 1, (B, T)).astype(np.int32)
    ke[0, 0] = s_cap
    ke[0, -1] = min(k, s_cap)             # n == k
    if T > 2:
        ke[0, 1] = min(k + 1, s_cap)      # n == k + 1
    ks = np.minimum(rng.integers(0, 50, (B, T)), ke).astype(np.int32)
    ks[0, 0] = 0
    out = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
    nws = b.workspace_bytes(b.make_shape(B, T, s_cap, topk=k), b.OP_TOPK)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)                        # the split path must not rely on a cleared workspace
    b.topk_select(f32_dev(sc), out, s_cap, key_start=i32_dev(ks), key_end=i32_dev(ke), workspace=ws)
    got = out.cpu().numpy()
    ref, _ = O.topk(sc.astype(np.float64), ks, ke, k)
    assert np.array_equal(got, ref)


def test_topk_short_prefix_example_on_gpu():
    # 256 candidates, index_topk 2048: 256 ascending positions then 1792 x -1
    sc = synth.scores_for_topk(3, 1, 256, "normal").reshape(1, 1, 256)
    out = torch.zeros((1, 1, 2048), dtype=torch.int32, device="cuda")
    b.topk_select(f32_dev(sc), out, 256)
    got = out.cpu().numpy()[0, 0]
    assert np.array_equal(got[:256], np.arange(256)) and (got[256:] == -1).all()


def test_empty_prefix_and_calls_without_rows():
    # A prefix of length 0: every top-k row is padding only (also through the fused indexer ->
    # top-k), and the attention of a selection with no valid entry is 0 with lse = -inf (the
    # oracle's empty-selection values).  Calls with no query rows succeed and write nothing.
    k, H, D, Hm = 16, 32, 128, 64
    ref_idx, _ = O.topk(np.zeros((1, 3, 0)), np.zeros((1, 3), np.int32), np.zeros((1, 3), np.int32), k)
    assert (ref_idx == -1).all()
    out = torch.full((1, 3, k), -7, dtype=torch.int32, device="cuda")
    b.topk_select(torch.zeros((1, 3, 1), device="cuda"), out, 0)
    assert np.array_equal(out.cpu().numpy(), ref_idx)

    q = torch.randn((1, 3, H, D), device="cuda").to(torch.bfloat16)
    kk = torch.empty((1, 0, H, D), dtype=torch.bfloat16, device="cuda")
    w = torch.rand((1, 3, H), device="cuda")
    nws = b.workspace_bytes(b.make_shape(1, 3, 0, H=H, D=D, Hk=H, topk=k), b.OP_INDEXER_TOPK)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    out.fill_(-7)
    b.indexer_topk(q, kk, w, out, workspace=ws)
    assert np.array_equal(out.cpu().numpy(), ref_idx)

    km = 256  # 4 tiles of 64 slots: two query rows split their selection over workgroups
    rq = np.random.default_rng(5).standard_normal((Hm, 576))
    o_ref, lse_ref = O.sparse_mla_row(rq, np.zeros((0, 576)), np.full(km, -1), 0.05, 512)
    assert not o_ref.any() and np.isneginf(lse_ref).all()
    for T in (2, 1100):  # selection split over workgroups (then merged), one workgroup per query
        mq = torch.randn((1, T, Hm, 576), device="cuda").to(torch.bfloat16)
        kv = torch.empty((1, 0, 576), dtype=torch.bfloat16, device="cuda")
        idx = torch.full((1, T, km), -1, dtype=torch.int32, device="cuda")
        o = torch.full((1, T, Hm, 512), 7.0, device="cuda").to(torch.bfloat16)
        lse = torch.full((1, T, Hm), 7.0, device="cuda")
        shape = b.make_shape(1, T, 0, topk=km, Hm=Hm, Dc=512, Dr=64)
        mws = torch.empty(max(b.workspace_bytes(shape, b.OP_SPARSE_MLA), 1), dtype=torch.uint8, device="cuda")
        b.sparse_mla_attention(mq, kv, idx, 0.05, o, lse, Dc=512, workspace=mws)
        assert not o.float().cpu().numpy().any() and np.isneginf(lse.cpu().numpy()).all(), T

    # no query rows: nothing is written, the calls succeed
    out0 = torch.empty((1, 0, k), dtype=torch.int32, device="cuda")
    b.topk_select(torch.zeros((1, 0, 100), device="cuda"), out0, 100)
    b.indexer_scores(torch.empty((1, 0, H, D), dtype=torch.bfloat16, device="cuda"),
                     torch.randn((1, 100, H, D), device="cuda").to(torch.bfloat16),
                     torch.empty((1, 0, H), device="cuda"), torch.empty((1, 0, 100), device="cuda"))
    shape0 = b.make_shape(1, 0, 100, topk=k, Hm=Hm, Dc=512, Dr=64)
    mws0 = torch.empty(max(b.workspace_bytes(shape0, b.OP_SPARSE_MLA), 1), dtype=torch.uint8, device="cuda")
    b.sparse_mla_attention(torch.empty((1, 0, Hm, 576), dtype=torch.bfloat16, device="cuda"),
                           torch.randn((1, 100, 576), device="cuda").to(torch.bfloat16),
                           torch.empty((1, 0, k), dtype=torch.int32, device="cuda"), 0.05,
                           torch.empty((1, 0, Hm, 512), dtype=torch.bfloat16, device="cuda"), Dc=512,
                           workspace=mws0)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ sparse MLA

def _mla_inputs(w, layer=0):
    L = synth.build_layer_inputs(w, layer, False)
    return L["mla_q"], L["kv"]


def _random_indices(rng, B, T, S, k, holes=False):
    idx = np.full((B, T, k), -1, np.int32)
    for bb in range(B):
        for t in range(T):
            n = int(rng.integers(0, min(k, S) + 1)) if t % 5 else min(k, S)
            idx[bb, t, :n] = np.sort(rng.choice(S, n, replace=False))
            if holes and n > 4:
                idx[bb, t, 1] = -1
                idx[bb, t, 3] = S + 5          # out of range: skipped
    idx[0, 0] = -1                             # empty row
    return idx


MLA_CASES = {
    "fp32_generic": dict(B=1, T=30, S=256, Hm=8, Dc=64, Dr=16, topk=32, mla_dtype="f32", idx_dtype="f32"),
    "bf16_mfma": dict(B=2, T=20, S=600, topk=256),
    "bf16_mfma_h128": dict(B=1, T=9, S=700, topk=192, Hm=128),
    "bf16_decode_split": dict(B=3, T=1, S=3000, topk=2048),
    # k not a multiple of the 64-row tile, rows that fill all k slots: the last tile's lanes
    # past k must not count (prefill, and a decode split whose last split is a partial tile)
    "bf16_mfma_ragged_topk": dict(B=2, T=20, S=600, topk=100),
    "bf16_decode_split_ragged_topk": dict(B=3, T=1, S=3000, topk=2000),
    "bf16_generic_small_heads": dict(B=1, T=12, S=200, topk=64, Hm=16, Dc=128, Dr=32),
}


@pytest.mark.parametrize("case", sorted(MLA_CASES))
def test_sparse_mla_matches_oracle(case):
    w = _wl(**MLA_CASES[case])
    q, kv = _mla_inputs(w)
    rng = np.random.default_rng(11)
    idx = _random_indices(rng, w.B, w.T, w.S, w.topk, holes=True)
    R = w.Dc + w.Dr
    out = torch.full((w.B, w.T, w.Hm, w.Dc), float("nan"), device="cuda",
                     dtype=torch.float32 if w.mla_dtype == "f32" else torch.bfloat16)
    lse = torch.full((w.B, w.T, w.Hm), float("nan"), device="cuda")
    shape = b.make_shape(w.B, w.T, w.S, topk=w.topk, Hm=w.Hm, Dc=w.Dc, Dr=w.Dr)
    ws = torch.empty(max(b.workspace_bytes(shape, b.OP_SPARSE_MLA), 1), dtype=torch.uint8, device="cuda")
    b.sparse_mla_attention(to_dev(q, w.mla_dtype), to_dev(kv, w.mla_dtype), i32_dev(idx), w.sm_scale, out, lse,
                           Dc=w.Dc, workspace=ws)
    got = out.float().cpu().numpy()
    gl = lse.cpu().numpy()
    q64, kv64 = O.decode(q, w.mla_dtype), O.decode(kv, w.mla_dtype)
    ref, rl = O.sparse_mla(q64, kv64, idx, w.sm_scale, w.Dc)
    tol = ATTN_TOL[w.mla_dtype]
    assert max_abs_rel(got, ref) <= tol
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    assert np.max(np.abs(gl[fin] - rl[fin])) / np.max(np.abs(rl[fin])) <= tol
    assert not got[0, 0].any()                                   # empty selection -> 0


def test_sparse_mla_full_selection_equals_dense_causal():
    # top-k >= prefix: the indexer degenerates to dense causal attention
    w = _wl(B=1, T=48, S=48, topk=64)
    q, kv = _mla_inputs(w)
    idx = np.full((1, 48, 64), -1, np.int32)
    for t in range(48):
        idx[0, t, :t + 1] = np.arange(t + 1)
    out = torch.empty((1, 48, 64, 512), device="cuda", dtype=torch.bfloat16)
    shape = b.make_shape(1, 48, 48, topk=64, Hm=64, Dc=512, Dr=64)
    ws = torch.empty(max(b.workspace_bytes(shape, b.OP_SPARSE_MLA), 1), dtype=torch.uint8, device="cuda")
    b.sparse_mla_attention(to_dev(q, "bf16"), to_dev(kv, "bf16"), i32_dev(idx), w.sm_scale, out, Dc=512,
                           workspace=ws)
    q64, kv64 = O.decode(q, "bf16"), O.decode(kv, "bf16")
    qq = torch.from_numpy(q64[0]).permute(1, 0, 2)[None]
    kk = torch.from_numpy(kv64[0])[None, None].expand(1, 64, 48, 576)
    vv = torch.from_numpy(np.ascontiguousarray(kv64[0][:, :512]))[None, None].expand(1, 64, 48, 512)
    dense = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=w.sm_scale)
    ref = dense[0].permute(1, 0, 2).numpy()
    assert max_abs_rel(out.float().cpu().numpy()[0], ref) <= ATTN_TOL["bf16"]


# ------------------------------------------------------------------ group

def _upload_group(w, inputs):
    dev = []
    for l, L in enumerate(inputs):
        d = {"q": to_dev(L["mla_q"], w.mla_dtype), "kv": to_dev(L["kv"], w.mla_dtype),
             "out": torch.empty((w.B, w.T, w.Hm, w.Dc), device="cuda",
                                dtype=torch.float32 if w.mla_dtype == "f32" else torch.bfloat16),
             "lse": torch.empty((w.B, w.T, w.Hm), device="cuda")}
        if "idx_q" in L:
            d["index"] = {"q": to_dev(L["idx_q"], w.idx_dtype), "k": to_dev(L["idx_k"], w.idx_dtype),
                          "w": f32_dev(L["w"])}
            if w.idx_dtype == "fp8":
                d["index"]["q_scale"] = f32_dev(L["idx_q_scale"])
                d["index"]["k_scale"] = f32_dev(L["idx_k_scale"])
        dev.append(d)
    return dev


def _run_group(w, dev, ke_dev, ks_dev=None, cache=None, tag=1, types=None):
    types = types or ["full" if c == "F" else "shared" for c in w.layers]
    shape = b.make_shape(w.B, w.T, w.S, H=w.H, D=w.D, Hk=w.Hk, topk=w.topk, Hm=w.Hm, Dc=w.Dc, Dr=w.Dr,
                         key_start=ks_dev, key_end=ke_dev, key_start_host=w.key_start() if ks_dev is not None
                         else None, key_end_host=w.key_end())
    ws = torch.empty(max(b.workspace_bytes(shape, b.OP_GROUP), 1), dtype=torch.uint8, device="cuda")
    cache = cache or b.IndexCache(w.B, w.T, w.topk)
    mdt = b.F32 if w.mla_dtype == "f32" else b.BF16
    stats = b.group_forward(shape, mdt, types, dev, w.sm_scale, cache, tag, ws)
    # the call's own counters are the analytic ones of its shape and key ranges
    idt = {"f32": b.F32, "bf16": b.BF16, "fp8": b.FP8_E4M3}[w.idx_dtype]
    ref = b.group_stats_compute(shape, idt, mdt, types, w.key_start() if ks_dev is not None else None, w.key_end())
    for key in ("n_full", "n_shared", "indexer_flops", "indexer_bytes", "topk_bytes", "attn_flops", "attn_bytes"):
        assert getattr(stats, key) == getattr(ref, key), key
    assert stats.n_launches >= len(types)
    return cache, stats


def _check_group(w, inputs, dev, cache_idx_per_layer, rows):
    """Compare indices (tie band) and per-layer attention on the given (b, t) rows.

    Attention is checked on every row against the oracle re-run with the GPU's own
    indices of the row's donor (already validated by the tie-band rule), so a swap
    inside the band does not hide an attention error and no row is left out."""
    ke, ks = w.key_end(), w.key_start()
    donors = O.donor_map(["full" if c == "F" else "shared" for c in w.layers])
    for l in sorted(set(donors)):
        q64, k64, w64 = decode_index(inputs[l], w)
        for (bb, t) in rows:
            s_row = O.index_scores_row(q64[bb, t], k64[bb], w64[bb, t], int(ks[bb, t]), int(ke[bb, t]))
            r, tau = O.topk_row(s_row, int(ks[bb, t]), int(ke[bb, t]), w.topk)
            check_topk_row(cache_idx_per_layer[l][bb, t], r, s_row, int(ks[bb, t]), tau)
    for l, L in enumerate(inputs):
        got = dev[l]["out"].float().cpu().numpy()
        kv64 = O.decode(L["kv"], w.mla_dtype)
        g = np.stack([got[bb, t] for bb, t in rows])
        ref = np.stack([O.sparse_mla_row(O.decode(L["mla_q"][bb, t], w.mla_dtype), kv64[bb],
                                         cache_idx_per_layer[donors[l]][bb, t], w.sm_scale, w.Dc)[0]
                        for bb, t in rows])
        assert max_abs_rel(g, ref) <= ATTN_TOL[w.mla_dtype], f"layer {l}"


def test_group_tiny_fp32_workload_all_rows():
    w = synth.WORKLOADS["tiny_prefill256_fp32"]
    inputs = synth.build_inputs(w)
    dev = _upload_group(w, inputs)
    cache, stats = _run_group(w, dev, i32_dev(w.key_end()))
    assert (stats.n_full, stats.n_shared) == (1, 3)
    idx = cache.indices.cpu().numpy()
    rows = [(0, t) for t in range(w.T)]
    _check_group(w, inputs, dev, {0: idx}, rows)
    # whole-tensor comparison against the oracle group (all rows matched exactly above)
    layers64 = []
    for L in inputs:
        d = {"mla_q": O.decode(L["mla_q"], "f32"), "kv": O.decode(L["kv"], "f32")}
        if "idx_q" in L:
            d.update(idx_q=O.decode(L["idx_q"], "f32"), idx_k=O.decode(L["idx_k"], "f32"), w=L["w"].astype(float))
        layers64.append(d)
    ref = O.group_forward(layers64, ["full", "shared", "shared", "shared"], w.key_start(), w.key_end(), w.topk,
                          w.sm_scale, w.Dc)
    if np.array_equal(ref["indices"][0], idx):
        for l in range(4):
            assert max_abs_rel(dev[l]["out"].cpu().numpy(), ref["out"][l]) <= ATTN_TOL["f32"]


@pytest.mark.parametrize("idx_dtype,Hk", [("bf16", 32), ("fp8", 32), ("bf16", 1)])
def test_group_mid_size_all_rows(idx_dtype, Hk):
    w = _wl(B=2, T=300, S=700, pos0=400, topk=256, idx_dtype=idx_dtype, Hk=Hk, layers="FFSSFS")
    inputs = synth.build_inputs(w)
    dev = _upload_group(w, inputs)
    cache, stats = _run_group(w, dev, i32_dev(w.key_end()))
    assert (stats.n_full, stats.n_shared) == (3, 3)
    # the cache ends with the last full layer's (layer 4) indices; donors 0 and 1 are
    # recomputed by single-full-layer calls on their inputs (same kernels, same bytes)
    per_layer = {4: cache.indices.cpu().numpy()}
    rows = [(bb, t) for bb in range(w.B) for t in range(w.T)]
    for donor in (0, 1):
        c2, _ = _run_group(w, [dev[donor]], i32_dev(w.key_end()), types=["full"])
        per_layer[donor] = c2.indices.cpu().numpy()
    _check_group(w, inputs, dev, per_layer, rows)


def test_group_cache_reuse_across_calls_and_errors():
    w = _wl(B=1, T=100, S=100, topk=32, layers="FS")
    inputs = synth.build_inputs(w)
    dev = _upload_group(w, inputs)
    ke = i32_dev(w.key_end())
    cache, _ = _run_group(w, dev, ke, tag=42)
    first = dev[1]["out"].clone()
    assert cache.valid and cache.c.donor_layer == 0 and cache.c.tag == 42
    # a later call starting on a shared layer reuses the handle
    dev2 = _upload_group(w, inputs[1:])
    _run_group(w, dev2, ke, cache=cache, tag=42, types=["shared"])
    assert torch.equal(dev2[0]["out"], first)
    with pytest.raises(b.DsaError) as e:
        _run_group(w, dev2, ke, cache=cache, tag=43, types=["shared"])
    assert e.value.status == 4
    with pytest.raises(b.DsaError) as e:
        _run_group(w, dev2, ke, cache=b.IndexCache(1, 100, 32), tag=42, types=["shared"])
    assert e.value.status == 3


def test_group_is_deterministic_and_shared_layers_match_standalone():
    w = _wl(B=1, T=200, S=400, pos0=200, topk=128)
    inputs = synth.build_inputs(w)
    dev = _upload_group(w, inputs)
    ke = i32_dev(w.key_end())
    cache, _ = _run_group(w, dev, ke)
    outs = [d["out"].clone() for d in dev]
    idx = cache.indices.clone()
    cache2, _ = _run_group(w, dev, ke)
    assert torch.equal(cache2.indices, idx)
    for l in range(4):
        assert torch.equal(dev[l]["out"], outs[l])
    # shared layer l == standalone attention with the donor's indices, bit for bit
    shape = b.make_shape(w.B, w.T, w.S, topk=w.topk, Hm=w.Hm, Dc=w.Dc, Dr=w.Dr)
    mws = torch.empty(max(b.workspace_bytes(shape, b.OP_SPARSE_MLA), 1), dtype=torch.uint8, device="cuda")
    for l in range(1, 4):
        o = torch.empty_like(outs[l])
        b.sparse_mla_attention(dev[l]["q"], dev[l]["kv"], idx, w.sm_scale, o, Dc=512, workspace=mws)
        assert torch.equal(o, outs[l])


def test_group_packed_varlen_sampled_rows():
    # packed variable-length batch: per-query [start of own sequence, position] ranges,
    # sequences from 1 token to longer than index_topk (many rows padded with -1)
    w = synth.WORKLOADS["packed_varlen_bf16"]
    inputs = synth.build_inputs(w)
    dev = _upload_group(w, inputs)
    cache, stats = _run_group(w, dev, i32_dev(w.key_end()), ks_dev=i32_dev(w.key_start()))
    assert (stats.n_full, stats.n_shared) == (1, 2)
    idx = cache.indices.cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(w.seqlens)])
    ts = set()
    for i, n in enumerate(w.seqlens):
        ts |= {int(cu[i]), int(cu[i] + n - 1), int(cu[i] + n // 2)}
    ts |= set(np.random.default_rng(1).integers(0, w.T, 12).tolist())
    rows = [(0, t) for t in sorted(ts)]
    _check_group(w, inputs, dev, {0: idx}, rows)
    ks, ke = w.key_start()[0], w.key_end()[0]
    for _, t in rows:   # every kept index inside the row's own sequence, -1 padding after
        n = min(int(ke[t] - ks[t]), w.topk)
        r = idx[0, t]
        assert ((r[:n] >= ks[t]) & (r[:n] < ke[t])).all() and (r[n:] == -1).all()


def test_group_decode_graph_capture_replays_match_eager():
    # a decode step captured once as a HIP graph and replayed: chunked top-k over 20,000-key
    # rows and split sparse MLA with its combine pass; every replay (with eager work and a
    # synchronisation between replays) must reproduce the eager results bit for bit
    w = _wl(B=4, T=1, S=20000, pos0=19999, layers="FSSF", topk=2048)
    inputs = synth.build_inputs(w)
    dev = _upload_group(w, inputs)
    types = ["full" if c == "F" else "shared" for c in w.layers]
    ke = i32_dev(w.key_end())
    shape = b.make_shape(w.B, w.T, w.S, H=w.H, D=w.D, Hk=w.Hk, topk=w.topk, Hm=w.Hm, Dc=w.Dc, Dr=w.Dr,
                         key_end=ke)
    ws = torch.empty(max(b.workspace_bytes(shape, b.OP_GROUP), 1), dtype=torch.uint8, device="cuda")
    cache = b.IndexCache(w.B, w.T, w.topk)
    b.group_forward(shape, b.BF16, types, dev, w.sm_scale, cache, 1, ws)
    torch.cuda.synchronize()
    eager = [d["out"].clone() for d in dev]
    eager_idx = cache.indices.clone()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            b.group_forward(shape, b.BF16, types, dev, w.sm_scale, cache, 1, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for d in dev:
            d["out"].fill_(float(rep + 1))
        cache.indices.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache.indices, eager_idx), f"replay {rep}: indices"
        for l, d in enumerate(dev):
            assert torch.equal(d["out"], eager[l]), f"replay {rep}: layer {l}"


def test_group_prefill4k_full_size_sampled_rows():
    w = synth.WORKLOADS["prefill4k_bf16"]
    inputs = synth.build_inputs(w)
    dev = _upload_group(w, inputs)
    cache, stats = _run_group(w, dev, i32_dev(w.key_end()))
    idx = cache.indices.cpu().numpy()
    # every 32nd row, both sides of every 128-row tile boundary, and the select-all / top-k edge
    ts = set(range(0, 4096, 32)) | {0, 1, 2, 2046, 2047, 2048, 2049, 4095}
    for x in range(128, 4096, 128):
        ts |= {x - 1, x}
    _check_group(w, inputs, dev, {0: idx}, [(0, t) for t in sorted(ts)])


@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_sparse_mla_running_max_moves(direction):
    # logits grow (or shrink) by several log2 units per 64-row tile, so the running
    # max of the online softmax is raised mid-row (rising) or fixed by the first tile
    rng = np.random.default_rng(21)
    T, S, Hm, R = 3, 640, 64, 576
    u = rng.standard_normal(R)
    u /= np.linalg.norm(u)
    gain = rng.uniform(1.0, 3.0, (T, Hm))
    q = 0.3 * rng.standard_normal((1, T, Hm, R)) + gain[None, :, :, None] * u
    ramp = np.arange(S) / 64.0 if direction == "rising" else (S - 1 - np.arange(S)) / 64.0
    kv = 0.5 * rng.standard_normal((1, S, R)) + 24.0 * ramp[None, :, None] * u
    qb = synth.f32_to_bf16_bits(q.astype(np.float32))
    kvb = synth.f32_to_bf16_bits(kv.astype(np.float32))
    idx = np.broadcast_to(np.arange(S, dtype=np.int32), (1, T, S)).copy()   # tiles in position order
    sm = 1.0 / 24.0
    out = torch.empty((1, T, Hm, 512), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((1, T, Hm), device="cuda")
    shape = b.make_shape(1, T, S, topk=S, Hm=Hm, Dc=512, Dr=64)
    ws = torch.empty(max(b.workspace_bytes(shape, b.OP_SPARSE_MLA), 1), dtype=torch.uint8, device="cuda")
    b.sparse_mla_attention(to_dev(qb, "bf16"), to_dev(kvb, "bf16"), i32_dev(idx), sm, out, lse, Dc=512,
                           workspace=ws)
    ref, rl = O.sparse_mla(O.decode(qb, "bf16"), O.decode(kvb, "bf16"), idx, sm, 512)
    assert max_abs_rel(out.float().cpu().numpy(), ref) <= ATTN_TOL["bf16"]
    assert np.max(np.abs(lse.cpu().numpy() - rl)) / np.max(np.abs(rl)) <= ATTN_TOL["bf16"]
