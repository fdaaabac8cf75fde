"""The large workloads at full size through the C ABI, checked against the oracle.

  * 32K-token decode of 64 sequences over an 8-layer F,F,F,S,S,S,F,S group: every
    sequence, every donor's indices, every layer's attention;
  * a 4096-query fp8 chunk at positions 126976..131071 over a 131072-token prefix:
    64 query rows on both sides of every 128-row tile boundary, and a full-width
    slab of index scores (those 64 rows x all 131072 keys) compared cell by cell;
  * 1M-token decode of 4 sequences with planted keys: every sequence;
  * the 4096-token prefill: a 128-row x 4096-key slab of index scores cell by cell.

Indices follow the tie-band rule; attention is compared on every checked row against
the oracle re-run with the GPU's own (tie-band validated) indices of the row's donor,
to the bf16 max-abs-relative bar.  The oracle works key block by key block, each block
decoded once for all checked rows of its batch item, in a few threads.
"""
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from dsa_indexer_top_lightning_amd import binding as b
from dsa_indexer_top_lightning_amd import synth
from helpers import ATTN_TOL, check_topk_row, f32_dev, i32_dev, max_abs_rel, to_dev

pytestmark = pytest.mark.gpu

KEY_BLOCK = 8192
THREADS = 12
SCORE_REL = 2e-5          # index-score bar: |g - o| <= 2e-5 * sum_h |w| sum_d |q k|


def _say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def _upload(w, L):
    d = {"q": to_dev(L["mla_q"], w.mla_dtype), "kv": to_dev(L["kv"], w.mla_dtype),
         "out": torch.empty((w.B, w.T, w.Hm, w.Dc), device="cuda", dtype=torch.bfloat16),
         "lse": torch.empty((w.B, w.T, w.Hm), device="cuda")}
    if "idx_q" in L:
        d["index"] = {"q": to_dev(L["idx_q"], w.idx_dtype), "k": to_dev(L["idx_k"], w.idx_dtype),
                      "w": f32_dev(L["w"])}
        if w.idx_dtype == "fp8":
            d["index"]["q_scale"] = f32_dev(L["idx_q_scale"])
            d["index"]["k_scale"] = f32_dev(L["idx_k_scale"])
    return d


def _oracle_rows(w, L, bb, ts, ke, bound=False, threads=THREADS):
    """Oracle index scores of rows ts of item bb over [0, ke[t]) (float64, one array per row), and
    with ``bound`` the per-cell scale sum_h |w| sum_d |q k| of their fp32 accumulation error.
    Each key block is decoded once and scored for every row that reaches it."""
    qsc = L.get("idx_q_scale")
    q = O.decode(L["idx_q"][bb, ts], w.idx_dtype, None if qsc is None else qsc[bb, ts])     # [R, H, D]
    wr = L["w"][bb, ts].astype(np.float64)
    kend = [int(ke[bb, t]) for t in ts]
    sc = [np.empty(n) for n in kend]
    bd = [np.empty(n) for n in kend] if bound else None
    ksc = L.get("idx_k_scale")

    def block(s0):
        s1 = min(max(kend), s0 + KEY_BLOCK)
        kb = O.decode(L["idx_k"][bb, s0:s1], w.idx_dtype, None if ksc is None else ksc[bb, s0:s1])
        live = [i for i in range(len(ts)) if kend[i] > s0]
        blk = O.index_scores_rows(q[live], kb, wr[live])
        # sum_h |w| max(0, |q|.|k|) = sum_h |w| sum_d |q k|: the scale of each cell's rounding error
        bb_ = O.index_scores_rows(np.abs(q[live]), np.abs(kb), np.abs(wr[live])) if bound else None
        for j, i in enumerate(live):
            e = min(kend[i], s1)
            sc[i][s0:e] = blk[j, :e - s0]
            if bound:
                bd[i][s0:e] = bb_[j, :e - s0]

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(block, range(0, max(kend), KEY_BLOCK)))
    return sc, bd


def _run(w, rows, slab=None):
    """Generate, upload and run the whole group (once per distinct donor, so that every donor's
    indices can be read back); the oracle's scores, indices and k-th score of the checked rows are
    formed per full layer while its inputs are on the host.  ``slab`` = rows of item 0 whose
    index scores of layer 0 are also computed by dsa_indexer_scores and returned."""
    types = ["full" if c == "F" else "shared" for c in w.layers]
    ke_h = w.key_end()
    items = sorted({bb for bb, _ in rows})
    dev, kv_keep, mq_keep, ref = [], [], [], {}
    slab_out = None
    for l in range(w.n_layers):
        L = synth.build_layer_inputs(w, l, types[l] == "full")
        dev.append(_upload(w, L))
        kv_keep.append(L["kv"])
        mq_keep.append({(bb, t): L["mla_q"][bb, t].copy() for bb, t in rows})
        if types[l] == "full":
            n_item = min(len(items), THREADS)   # items side by side, key blocks inside each

            def item(bb):
                ts = [t for b2, t in rows if b2 == bb]
                sc, _ = _oracle_rows(w, L, bb, ts, ke_h, threads=max(1, THREADS // n_item))
                return {(bb, t): (sc[i],) + O.topk_row(sc[i], 0, int(ke_h[bb, t]), w.topk)
                        for i, t in enumerate(ts)}
            with ThreadPoolExecutor(n_item) as ex:
                for part in ex.map(item, items):
                    ref.update({(l,) + key: v for key, v in part.items()})
            if l == 0 and slab is not None:
                slab_out = _slab(w, L, dev[0]["index"], slab)
        del L
        _say(f"{w.name}: layer {l} generated, uploaded{' and scored by the oracle' if types[l] == 'full' else ''}")
    shape = b.make_shape(w.B, w.T, w.S, H=w.H, D=w.D, Hk=w.Hk, topk=w.topk, Hm=w.Hm, Dc=w.Dc, Dr=w.Dr,
                         key_end=i32_dev(ke_h), key_end_host=ke_h)
    ws = torch.empty(b.workspace_bytes(shape, b.OP_GROUP), dtype=torch.uint8, device="cuda")
    donors = O.donor_map(types)
    per_donor = {}
    for d in sorted(set(donors)):
        cache = b.IndexCache(w.B, w.T, w.topk)
        last = max(l for l in range(w.n_layers) if donors[l] == d)
        b.group_forward(shape, b.BF16, types[:last + 1], dev[:last + 1], w.sm_scale, cache, 1, ws)
        per_donor[d] = cache.indices.cpu().numpy()
        _say(f"{w.name}: group through layer {last} done (donor {d})")
    torch.cuda.synchronize()
    outs = [d["out"].float().cpu().numpy() for d in dev]
    return donors, outs, kv_keep, mq_keep, ref, per_donor, slab_out


def _slab(w, L, I, ts):
    """dsa_indexer_scores of layer 0 on the device; rows ts of item 0 copied back, and the oracle's
    scores and error scales of those rows."""
    ld = w.S
    scores = torch.full((w.B, w.T, ld), float("nan"), device="cuda")
    ke_h = w.key_end()
    b.indexer_scores(I["q"], I["k"], I["w"], scores, q_scale=I.get("q_scale"), k_scale=I.get("k_scale"),
                     key_end=i32_dev(ke_h))
    got = scores[0, ts].cpu().numpy()
    del scores
    sc, bd = _oracle_rows(w, L, 0, ts, ke_h, bound=True)
    return got, sc, bd, [int(ke_h[0, t]) for t in ts]


def _check(w, rows, slab=None):
    donors, outs, kv_keep, mq_keep, ref, per_donor, slab_out = _run(w, rows, slab)
    for d in per_donor:
        for (bb, t) in rows:
            sc, r, tau = ref[(d, bb, t)]
            check_topk_row(per_donor[d][bb, t], r, sc, 0, tau)
        _say(f"{w.name}: donor {d}: indices of {len(rows)} rows checked")
    for l in range(w.n_layers):
        g, o = [], []
        for (bb, t) in rows:
            idx = per_donor[donors[l]][bb, t]
            sel = idx[idx >= 0]
            kv_rows = O.decode(kv_keep[l][bb][sel], w.mla_dtype)
            q = O.decode(mq_keep[l][(bb, t)], w.mla_dtype)
            o.append(O.sparse_mla_row(q, kv_rows, np.arange(len(sel)), w.sm_scale, w.Dc)[0])
            g.append(outs[l][bb, t])
        assert max_abs_rel(np.stack(g), np.stack(o)) <= ATTN_TOL["bf16"], f"layer {l}"
    _say(f"{w.name}: attention of {len(rows)} rows x {w.n_layers} layers checked")
    if slab_out is not None:
        got, sc, bd, kend = slab_out
        for i in range(len(slab)):
            n = kend[i]
            err = np.abs(got[i, :n] - sc[i])
            assert (err <= SCORE_REL * bd[i] + 1e-30).all(), f"slab row {slab[i]}: max err {err.max()}"
            assert np.isnan(got[i, n:]).all(), f"slab row {slab[i]}: cells past the causal end written"
        _say(f"{w.name}: index scores of {len(slab)} rows x {w.S} keys checked cell by cell")


def test_decode32k_b64_bf16_every_sequence():
    w = synth.WORKLOADS["decode32k_b64_bf16"]
    _check(w, [(bb, 0) for bb in range(w.B)])


def _tile_boundary_rows(T, tile=128):
    ts = {0, T - 1}
    for x in range(tile, T, tile):
        ts |= {x - 1, x}
    return sorted(ts)


def test_chunk128k_fp8_tile_boundary_rows_and_score_slab():
    w = synth.WORKLOADS["chunk128k_fp8"]
    ts = _tile_boundary_rows(w.T)
    assert len(ts) == 64
    _check(w, [(0, t) for t in ts], slab=ts)


def test_decode1m_b4_fp8_planted_every_sequence():
    w = synth.WORKLOADS["decode1m_b4_fp8"]
    _check(w, [(bb, 0) for bb in range(w.B)])


def test_prefill4k_bf16_score_slab_cell_by_cell():
    # 128 query rows across the 2048 boundary (select-all rows below it, top-k rows above) and
    # across a 128-row tile boundary, all 4096 keys of each
    w = synth.WORKLOADS["prefill4k_bf16"]
    L = synth.build_layer_inputs(w, 0, True)
    I = _upload(w, L)["index"]
    ts = list(range(1984, 2112))
    got, sc, bd, kend = _slab(w, L, I, ts)
    for i, t in enumerate(ts):
        n = kend[i]
        err = np.abs(got[i, :n] - sc[i])
        assert (err <= SCORE_REL * bd[i] + 1e-30).all(), f"row {t}: max err {err.max()}"
        assert np.isnan(got[i, n:]).all()
