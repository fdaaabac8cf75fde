"""dsa_indexer_topk (indexer -> top-k without the score matrix) on the GPU.

The call's contract is bit-identical indices to dsa_indexer_scores followed by
dsa_topk_select on the same inputs; every test checks that on every row.  The first
B*T*s_cap*4 bytes of the workspace are the score buffer of the fall-back rows (nothing
else writes them), so each test also checks WHICH rows fell back:
  * random keys: none (the sampled threshold keeps between topk and 12288 candidates);
  * all-zero head weights: every key ties, more candidates than slots -> every row;
  * sampled positions made to dominate: fewer candidates than topk -> every row;
  * a mix of both in one call, rows with fewer keys than topk, windows starting past 0;
for the fp8 prefill tile kernel and the bf16 / fp8 decode stream kernel, at several sample
strides, and against the oracle (tie band) on a few rows.  At full size: the 4096-query fp8
chunk over 131072 keys and the 1M-key fp8 decode of 4 sequences, every row.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle as O
from dsa_indexer_top_lightning_amd import binding as b
from dsa_indexer_top_lightning_amd import synth
from helpers import check_topk_row, f32_dev, i32_dev, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def _inputs(w):
    L = synth.build_layer_inputs(w, 0, True, with_mla=False)
    return L


def _upload(w, L):
    I = {"q": to_dev(L["idx_q"], w.idx_dtype), "k": to_dev(L["idx_k"], w.idx_dtype), "w": f32_dev(L["w"])}
    if w.idx_dtype == "fp8":
        I["q_scale"] = f32_dev(L["idx_q_scale"])
        I["k_scale"] = f32_dev(L["idx_k_scale"])
    return I


def _run(w, I, ks=None, ke=None, stride=0):
    """Unfused reference and fused indices (int32 [B,T,topk]) and the rows that fell back."""
    B, T, S, K = w.B, w.T, w.S, w.topk
    kd = None if ke is None else i32_dev(ke)
    sd = None if ks is None else i32_dev(ks)
    extra = dict(q_scale=I.get("q_scale"), k_scale=I.get("k_scale"), key_start=sd, key_end=kd)
    shape = b.make_shape(B, T, S, H=w.H, D=w.D, Hk=w.Hk, topk=K, key_start=sd, key_end=kd)
    ws = torch.full((b.workspace_bytes(shape, b.OP_INDEXER_TOPK),), 0xFF, dtype=torch.uint8, device="cuda")
    got = torch.full((B, T, K), -7, dtype=torch.int32, device="cuda")
    b.indexer_topk(I["q"], I["k"], I["w"], got, sample_stride=stride, workspace=ws, **extra)
    torch.cuda.synchronize()
    fell = (ws[:B * T * S * 4].view(torch.int32).view(B * T, S) != -1).any(dim=1).cpu().numpy()
    del ws
    scores = torch.empty((B, T, S), device="cuda")
    b.indexer_scores(I["q"], I["k"], I["w"], scores, **extra)
    ref = torch.empty((B, T, K), dtype=torch.int32, device="cuda")
    tws = torch.empty((max(1, b.workspace_bytes(shape, b.OP_TOPK)),), dtype=torch.uint8, device="cuda")
    b.topk_select(scores, ref, S, key_start=sd, key_end=kd, workspace=tws)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy(), fell


def _same(ref, got, what):
    bad = np.argwhere((ref != got).any(-1))
    assert bad.size == 0, f"{what}: rows {bad[:8].tolist()} differ from the unfused call"


def _oracle_rows(w, L, ks, ke, rows):
    """Oracle scores (float64, over [key_start, key_end)) and top-k of the given rows; only each
    row's own key range is decoded."""
    qsc, ksc = L.get("idx_q_scale"), L.get("idx_k_scale")
    for bb, t in rows:
        a, e = int(ks[bb, t]), int(ke[bb, t])
        q = O.decode(L["idx_q"][bb, t], w.idx_dtype, None if qsc is None else qsc[bb, t])
        k = O.decode(L["idx_k"][bb, a:e], w.idx_dtype, None if ksc is None else ksc[bb, a:e])
        sc = O.index_scores_row(q, k, L["w"][bb, t].astype(np.float64), 0, e - a)
        yield (bb, t), sc, O.topk_row(sc, a, e, w.topk)


PREFILL = synth.WORKLOADS["chunk128k_fp8"].with_(name="chunk20k_fp8", T=300, S=20000, pos0=19700, topk=512)


def _ranges(w):
    ke = w.key_end()
    return np.zeros_like(ke), ke


@pytest.mark.parametrize("stride", [0, 16, 4096])
def test_prefill_fp8_random_keys(stride):
    # 300 queries = 2 full 128-row tiles and a ragged one; 20000 keys = 78 key tiles and a tail
    w = PREFILL
    L = _inputs(w)
    ks, ke = _ranges(w)
    ref, got, fell = _run(w, _upload(w, L), ks, ke, stride)
    _same(ref, got, f"stride {stride}")
    if stride in (0, 16):
        assert not fell.any(), f"{int(fell.sum())} rows fell back"
    else:
        # 5 samples per row, fewer than the threshold's rank (37): every key is a candidate,
        # more than 12288 of them, so every row falls back
        assert fell.all()
    for key, sc, (r, tau) in _oracle_rows(w, L, ks, ke, [(0, 0), (0, 127), (0, 128), (0, 299)]):
        check_topk_row(got[key], r, sc, 0, tau)


def test_prefill_fp8_fallback_rows_mixed_with_candidate_rows():
    w = PREFILL
    L = _inputs(w)
    ks, ke = _ranges(w)
    # rows 5, 130 and 299: zero head weights (all scores 0: every key ties, too many candidates)
    for t in (5, 130, 299):
        L["w"][0, t] = 0.0
    # rows 0..3 see fewer keys than topk (select-all rows), row 200 a window starting at 7000
    ke[0, :4] = [1, 200, 511, 512]
    ks[0, 200] = 7000
    I = _upload(w, L)
    ref, got, fell = _run(w, I, ks, ke)
    _same(ref, got, "mixed")
    assert set(np.flatnonzero(fell)) == {5, 130, 299}
    assert (got[0, 5] == np.arange(512)).all()       # ties go to the lowest positions
    for key, sc, (r, tau) in _oracle_rows(w, L, ks, ke, [(0, 0), (0, 3), (0, 200), (0, 201)]):
        check_topk_row(got[key], r, sc, int(ks[key]), tau)


def test_prefill_fp8_dominant_samples_fall_back():
    # keys at multiples of the default stride 64 score ~100x higher: the threshold is set among
    # them, about r of them reach it (r < topk), every row falls back
    w = PREFILL
    L = _inputs(w)
    L["idx_k_scale"][0, ::64] *= 100.0
    ks, ke = _ranges(w)
    ref, got, fell = _run(w, _upload(w, L), ks, ke)
    _same(ref, got, "dominant samples")
    assert fell.all()


# bf16 rows are longer than the select's bitmap (131072 keys: kept positions sorted instead),
# fp8 rows shorter (emitted from the bitmap)
DECODE = {
    "bf16": synth.WORKLOADS["decode32k_b64_bf16"].with_(name="decode160k_b4_bf16_h16", B=4, S=160000, pos0=159999,
                                                       H=16, Hk=16),
    "fp8": synth.WORKLOADS["decode1m_b4_fp8"].with_(name="decode100k_b4_fp8", S=100000, pos0=99999),
}


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_decode_stream(dt):
    w = DECODE[dt]
    L = _inputs(w)
    ks, ke = _ranges(w)
    ke[1, 0] = 50001                      # a shorter row (bitmap emit in both cases)
    ks[2, 0] = 30000                      # a window
    L["w"][3, 0] = 0.0                    # every key ties: falls back
    ref, got, fell = _run(w, _upload(w, L), ks, ke)
    _same(ref, got, dt)
    assert list(fell) == [False, False, False, True]
    for key, sc, (r, tau) in _oracle_rows(w, L, ks, ke, [(0, 0), (1, 0), (2, 0)]):
        check_topk_row(got[key], r, sc, int(ks[key]), tau)


def test_prefill_fp8_two_batch_items_ragged_ranges():
    # two batch items, 200 queries (a ragged second query tile), 6000 keys (a ragged last key
    # tile): the head-major key scales and row weights are laid out per batch item and padded to
    # whole tiles; item 1 gets windows that start past 0 and rows whose range ends in the second
    # key tile
    w = PREFILL.with_(name="chunk6k_fp8_b2", B=2, T=200, S=6000, pos0=5800, topk=256)
    L = _inputs(w)
    ks, ke = _ranges(w)
    ks[1, :50] = 1000 + 7 * np.arange(50)
    ks[1, 150:] = 4400
    ke[1, 120:130] = 300
    ref, got, fell = _run(w, _upload(w, L), ks, ke)
    _same(ref, got, "two batch items")
    assert not fell.any(), f"{int(fell.sum())} rows fell back"
    for key, sc, (r, tau) in _oracle_rows(w, L, ks, ke, [(0, 0), (0, 199), (1, 0), (1, 125), (1, 199)]):
        check_topk_row(got[key], r, sc, int(ks[key]), tau)


@pytest.mark.parametrize("name", ["chunk128k_fp8", "decode1m_b4_fp8"])
def test_full_size_every_row(name):
    w = synth.WORKLOADS[name]
    L = _inputs(w)
    _say(f"{name}: inputs generated")
    ks, ke = _ranges(w)
    ref, got, fell = _run(w, _upload(w, L), ks, ke)
    _say(f"{name}: {int(fell.sum())} of {fell.size} rows fell back")
    _same(ref, got, name)
    assert fell.sum() <= fell.size // 100
