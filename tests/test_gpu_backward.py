"""GPU parity of the backward calls (dsa_sparse_mla_backward, dsa_index_backward) against
the oracle.

The GPU takes the forward's own results (output, log-sum-exp) from dsa_sparse_mla_attention
on the same inputs; the oracle recomputes everything in float64 from the stored inputs.
Bars as for the forward: max-abs-relative error <= 1e-5 (fp32) and <= 2e-2 (bf16) per
gradient tensor.  The latent-row gradient collects its contributions with fp32 atomics
in no fixed order, which the fp32 bar covers.  The index-score backward computes with
exact products and fp32 sums, so all of its gradients are held to 1e-5 for every input
type; slots whose score lies within rounding of the ReLU kink get no gradient in the
test (the two sides could take different branches there).
"""
import numpy as np
import pytest
import torch

import oracle as O
from dsa_indexer_top_lightning_amd import binding as b
from helpers import max_abs_rel

pytestmark = pytest.mark.gpu


def _inputs(rng, B, T, S, Hm, Dc, Dr, k, dtype):
    R = Dc + Dr
    q = rng.standard_normal((B, T, Hm, R)).astype(np.float32)
    kv = rng.standard_normal((B, S, R)).astype(np.float32)
    dout = rng.standard_normal((B, T, Hm, Dc)).astype(np.float32)
    idx = np.full((B, T, k), -1, np.int32)
    for bb in range(B):
        for t in range(T):
            n = int(rng.integers(0, k + 1)) if t % 3 else k
            idx[bb, t, :n] = np.sort(rng.choice(S, size=min(n, S), replace=False))[:n]
    if T > 1 and k > 2:
        idx[0, 1, 1] = idx[0, 1, 0]        # a row listed twice
    if dtype == "bf16":
        q, kv, dout = [torch.from_numpy(x).to(torch.bfloat16) for x in (q, kv, dout)]
        host = [x.to(torch.float64).numpy() for x in (q, kv, dout)]
    else:
        q, kv, dout = [torch.from_numpy(x) for x in (q, kv, dout)]
        host = [x.to(torch.float64).numpy() for x in (q, kv, dout)]
    return q, kv, dout, idx, host


def _run(q, kv, dout, idx, Dc, scale, dtype):
    B, T, Hm, R = q.shape
    S = kv.shape[1]
    qd, kvd, dd = q.cuda(), kv.cuda(), dout.cuda()
    idd = torch.from_numpy(idx).cuda()
    out = torch.empty(B, T, Hm, Dc, dtype=qd.dtype, device="cuda")
    lse = torch.empty(B, T, Hm, device="cuda")
    shape = b.make_shape(B, T, S, topk=idx.shape[-1], Hm=Hm, Dc=Dc, Dr=R - Dc)
    ws = torch.empty(max(b.workspace_bytes(shape, b.OP_SPARSE_MLA), 1), dtype=torch.uint8, device="cuda")
    b.sparse_mla_attention(qd, kvd, idd, scale, out, lse, Dc=Dc, workspace=ws)
    dq = torch.full((B, T, Hm, R), float("nan"), device="cuda")
    dkv = torch.full((B, S, R), float("nan"), device="cuda")   # the call must clear it
    nws = b.workspace_bytes(shape, b.OP_SPARSE_MLA_BWD)
    bws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda") if nws else None  # stale contents
    b.sparse_mla_backward(qd, kvd, idd, scale, out, lse, dd, dq, dkv, Dc=Dc, workspace=bws)
    torch.cuda.synchronize()
    return dq.cpu().numpy().astype(np.float64), dkv.cpu().numpy().astype(np.float64)


CASES = {
    # name: (B, T, S, Hm, Dc, Dr, k, dtype, tol)
    "fp32_small": (2, 5, 40, 8, 64, 16, 12, "f32", 1e-5),
    "fp32_odd_heads": (1, 4, 30, 3, 40, 8, 9, "f32", 1e-5),
    # bf16 with 512 + 64 dims and heads in groups of 64: the matrix-core kernels; with
    # 8 k >= S the latent-row gradient is formed per 64-row tile (dense path), else per slot
    "bf16_mla_dims": (1, 24, 300, 64, 512, 64, 64, "bf16", 2e-2),
    "bf16_decode": (3, 1, 5000, 64, 512, 64, 2048, "bf16", 2e-2),
    # per-slot path: two head groups, a partial last tile (200 = 3 x 64 + 8 slots), 40 queries
    "bf16_two_head_groups": (2, 20, 3000, 128, 512, 64, 200, "bf16", 2e-2),
    # 512 query rows: each workgroup walks 2 tiles of its selection (with fewer rows the
    # selection is split to one tile per workgroup)
    "bf16_two_tiles_per_workgroup": (1, 512, 2000, 64, 512, 64, 256, "bf16", 2e-2),
    # dense path with two head groups, 300 queries in 10 query chunks (the last one ragged) and a
    # 1200-row tail tile
    "bf16_dense_two_groups_chunks": (1, 300, 1200, 128, 512, 64, 256, "bf16", 2e-2),
    # 32 heads: the vector kernel
    "bf16_32_heads": (1, 8, 300, 32, 512, 64, 64, "bf16", 2e-2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_mla_backward_matches_oracle(name):
    B, T, S, Hm, Dc, Dr, k, dtype, tol = CASES[name]
    rng = np.random.default_rng(100 + list(CASES).index(name))
    scale = 1.0 / np.sqrt(Dc + Dr)
    q, kv, dout, idx, (qh, kvh, dh) = _inputs(rng, B, T, S, Hm, Dc, Dr, k, dtype)
    dq, dkv = _run(q, kv, dout, idx, Dc, float(np.float32(scale)), dtype)
    rq, rkv = O.sparse_mla_backward(qh, kvh, idx, float(np.float32(scale)), Dc, dh)
    assert max_abs_rel(dq, rq) <= tol, max_abs_rel(dq, rq)
    assert max_abs_rel(dkv, rkv) <= tol, max_abs_rel(dkv, rkv)
    untouched = np.ones((B, S), bool)
    for bb in range(B):
        sel = idx[bb][idx[bb] >= 0]
        untouched[bb, sel] = False
    assert np.all(dkv[untouched] == 0.0)     # rows nobody selected: exactly zero


@pytest.mark.parametrize("B,T,S,Hm,Dc,Dr,k,dtype", [(1, 3, 16, 8, 64, 16, 4, "f32"),
                                                      (1, 3, 100, 64, 512, 64, 64, "bf16"),      # matrix cores
                                                      (2, 1, 3000, 64, 512, 64, 2048, "bf16")])  # ... split
def test_sparse_mla_backward_empty_selections(B, T, S, Hm, Dc, Dr, k, dtype):
    rng = np.random.default_rng(5)
    q, kv, dout, idx, _ = _inputs(rng, B, T, S, Hm, Dc, Dr, k, dtype)
    idx[:] = -1
    dq, dkv = _run(q, kv, dout, idx, Dc, 0.1, dtype)
    assert np.all(dq == 0) and np.all(dkv == 0)


# ------------------------------------------------------------------ index score backward

def _index_inputs(rng, B, T, S, H, D, Hk, k, dtype):
    """Stored device inputs and their dequantised float64 values (oracle side)."""
    if dtype == "fp8":
        def codes(shape):
            c = rng.integers(0, 126, shape).astype(np.uint8) | (rng.integers(0, 2, shape).astype(np.uint8) << 7)
            return c
        qc, kc = codes((B, T, H, D)), codes((B, S, Hk, D))
        qs = (rng.random((B, T, H)) * 0.02 + 0.001).astype(np.float32)
        ks = (rng.random((B, S, Hk)) * 0.02 + 0.001).astype(np.float32)
        qh = O.decode(qc, "fp8", qs)
        kh = O.decode(kc, "fp8", ks)
        dev = (torch.from_numpy(qc).cuda().view(torch.float8_e4m3fn), torch.from_numpy(kc).cuda().view(torch.float8_e4m3fn),
               torch.from_numpy(qs).cuda(), torch.from_numpy(ks).cuda())
    else:
        q = torch.from_numpy(rng.standard_normal((B, T, H, D)).astype(np.float32))
        kk = torch.from_numpy(rng.standard_normal((B, S, Hk, D)).astype(np.float32))
        if dtype == "bf16":
            q, kk = q.to(torch.bfloat16), kk.to(torch.bfloat16)
        qh, kh = q.to(torch.float64).numpy(), kk.to(torch.float64).numpy()
        dev = (q.cuda(), kk.cuda(), None, None)
    w = rng.random((B, T, H)).astype(np.float32)
    idx = np.full((B, T, k), -1, np.int32)
    for bb in range(B):
        for t in range(T):
            n = int(rng.integers(1, k + 1)) if t % 2 else k
            idx[bb, t, :n] = rng.choice(S, size=n, replace=False)
    if T > 1 and k > 2:
        idx[0, 1, 1] = idx[0, 1, 0]        # a key listed twice
    dI = rng.standard_normal((B, T, k)).astype(np.float32)
    # a score within rounding of 0 could take the other ReLU branch on the GPU: give
    # such slots no gradient, so that both sides agree on every branch that counts
    g = np.arange(H) if Hk == H else np.zeros(H, int)
    for bb in range(B):
        for t in range(T):
            for j in range(k):
                e = idx[bb, t, j]
                if e < 0:
                    continue
                prod = qh[bb, t] * kh[bb, e][g]
                if np.any(np.abs(prod.sum(axis=1)) <= 1e-4 * np.abs(prod).sum(axis=1)):
                    dI[bb, t, j] = 0.0
    return dev, qh, kh, w, idx, dI


INDEX_BWD_CASES = {
    # name: (B, T, S, H, D, Hk, k, dtype, dense): dense = the matrix-core path (bf16 / fp8,
    # D = 128, 8 k >= S), else the vector kernel
    "fp32_small": (2, 5, 60, 4, 32, 4, 10, "f32", False),
    "bf16_heads": (1, 6, 300, 32, 128, 32, 64, "bf16", True),
    "bf16_shared_key": (1, 6, 300, 32, 128, 1, 64, "bf16", True),
    "fp8_heads": (1, 5, 200, 32, 128, 32, 48, "fp8", True),
    "fp8_shared_key": (2, 3, 200, 32, 128, 1, 48, "fp8", True),
    "bf16_decode": (3, 1, 3000, 32, 128, 32, 2048, "bf16", True),
    # 300 queries = 2 full 128-query workgroups and a ragged one, 2000 keys = 31 key tiles
    # and a 16-key tail, 512 slots per row
    "bf16_dense_tiles": (1, 300, 2000, 32, 128, 32, 512, "bf16", True),
    "fp8_dense_shared_key": (2, 130, 1000, 32, 128, 1, 256, "fp8", True),
    # 8 x 64 < 5000 keys: the vector kernel
    "bf16_sparse": (1, 4, 5000, 32, 128, 32, 64, "bf16", False),
    "fp8_sparse_shared_key": (1, 3, 3000, 32, 128, 1, 96, "fp8", False),
}


@pytest.mark.parametrize("name", list(INDEX_BWD_CASES))
def test_index_backward_matches_oracle(name):
    B, T, S, H, D, Hk, k, dtype, dense = INDEX_BWD_CASES[name]
    rng = np.random.default_rng(200 + list(INDEX_BWD_CASES).index(name))
    (qd, kd, qsd, ksd), qh, kh, w, idx, dI = _index_inputs(rng, B, T, S, H, D, Hk, k, dtype)
    dq = torch.full((B, T, H, D), float("nan"), device="cuda")
    dk = torch.full((B, S, Hk, D), float("nan"), device="cuda")
    dw = torch.full((B, T, H), float("nan"), device="cuda")
    shape = b.make_shape(B, T, S, H=H, D=D, Hk=Hk, topk=k)
    nws = b.workspace_bytes(shape, b.OP_INDEX_BWD)
    assert (nws > 0) == dense
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda") if nws else None  # stale contents
    b.index_backward(qd, kd, torch.from_numpy(w).cuda(), torch.from_numpy(idx).cuda(), torch.from_numpy(dI).cuda(),
                     dq, dk, dw, q_scale=qsd, k_scale=ksd, workspace=ws)
    torch.cuda.synchronize()
    rq, rk, rw = O.index_scores_backward_selected(qh, kh, w.astype(np.float64), idx, dI.astype(np.float64))
    for got, ref in ((dq, rq), (dk, rk), (dw, rw)):
        g = got.cpu().numpy().astype(np.float64)
        assert max_abs_rel(g, ref) <= 1e-5, (max_abs_rel(g, ref), got.shape)
    sel = np.zeros((B, S), bool)
    for bb in range(B):
        sel[bb, idx[bb][idx[bb] >= 0]] = True
    assert np.all(dk.cpu().numpy()[~sel] == 0.0)     # keys nobody selected: exactly zero


# ------------------------------------------------------------------ full size (4K prefill)

def _prefill_selection(rng, T, k):
    """The 4K prefill's selection structure: query t takes every key <= t while t + 1 <= k, then k of
    its t + 1 keys; ascending, -1 padded."""
    idx = np.full((1, T, k), -1, np.int32)
    for t in range(T):
        if t + 1 <= k:
            idx[0, t, :t + 1] = np.arange(t + 1)
        else:
            idx[0, t] = np.sort(rng.choice(t + 1, size=k, replace=False))
    return idx


def _selecting(idx, j):
    """Rows (queries) of batch item 0 whose selection names key j, and how many slots do."""
    hits = (idx[0] == j).sum(axis=1)
    return np.flatnonzero(hits), hits


SAMPLED_QUERIES = [0, 1, 63, 64, 2046, 2047, 2048, 3001, 4095]
SAMPLED_KEYS = [4090, 4032, 3990]   # selected by the last queries only: a few to a few dozen each


def test_prefill4k_full_size_sparse_mla_backward_sampled():
    # the shape bench.py --backward times on the 4K prefill: 4096 queries over 4096 keys, 64
    # heads, 512 + 64 latent dims, topk 2048 (the dense latent-row path and the per-tile dq)
    T, S, Hm, Dc, Dr, k = 4096, 4096, 64, 512, 64, 2048
    R = Dc + Dr
    rng = np.random.default_rng(4096)
    idx = _prefill_selection(rng, T, k)
    q = torch.from_numpy(rng.standard_normal((1, T, Hm, R), dtype=np.float32)).to(torch.bfloat16)
    kv = torch.from_numpy(rng.standard_normal((1, S, R), dtype=np.float32)).to(torch.bfloat16)
    dout = torch.from_numpy(rng.standard_normal((1, T, Hm, Dc), dtype=np.float32)).to(torch.bfloat16)
    shape = b.make_shape(1, T, S, topk=k, Hm=Hm, Dc=Dc, Dr=Dr)
    assert b.workspace_bytes(shape, b.OP_SPARSE_MLA_BWD) > 0
    scale = float(np.float32(1.0 / np.sqrt(R)))
    dq, dkv = _run(q, kv, dout, idx, Dc, scale, "bf16")
    kvh = kv.to(torch.float64).numpy()[0]
    qh = lambda t: q[0, t].to(torch.float64).numpy()
    dh = lambda t: dout[0, t].to(torch.float64).numpy()
    for t in SAMPLED_QUERIES:
        rq, _, _ = O.sparse_mla_backward_row(qh(t), kvh, idx[0, t], scale, Dc, dh(t))
        assert max_abs_rel(dq[0, t], rq) <= 2e-2, (t, max_abs_rel(dq[0, t], rq))
    for j in SAMPLED_KEYS:
        ts, _ = _selecting(idx, j)
        ref = np.zeros(R)
        for t in ts:
            _, rows, dc = O.sparse_mla_backward_row(qh(t), kvh, idx[0, t], scale, Dc, dh(t))
            ref += dc[rows == j].sum(axis=0)
        assert len(ts) > 0
        assert max_abs_rel(dkv[0, j], ref) <= 2e-2, (j, len(ts), max_abs_rel(dkv[0, j], ref))


def test_prefill4k_full_size_index_backward_sampled():
    # the 4K prefill's index heads: 32 per-head bf16 keys of 128 dims (the dense matrix-core path)
    T, S, H, D, k = 4096, 4096, 32, 128, 2048
    rng = np.random.default_rng(4097)
    idx = _prefill_selection(rng, T, k)
    q = torch.from_numpy(rng.standard_normal((1, T, H, D), dtype=np.float32)).to(torch.bfloat16)
    kk = torch.from_numpy(rng.standard_normal((1, S, H, D), dtype=np.float32)).to(torch.bfloat16)
    w = rng.random((1, T, H)).astype(np.float32)
    dI = rng.standard_normal((1, T, k)).astype(np.float32)
    qh, kh = q.to(torch.float64).numpy(), kk.to(torch.float64).numpy()
    rows = sorted(set(SAMPLED_QUERIES) | {int(t) for j in SAMPLED_KEYS for t in _selecting(idx, j)[0]})
    # slots of the checked rows whose score lies within rounding of the ReLU kink get no gradient
    for t in rows:
        sel = idx[0, t]
        valid = sel >= 0
        prod = qh[0, t][None, :, :] * kh[0, sel[valid]]            # [slots, H, D]
        near = np.any(np.abs(prod.sum(axis=2)) <= 1e-4 * np.abs(prod).sum(axis=2), axis=1)
        dI[0, t, np.flatnonzero(valid)[near]] = 0.0
    shape = b.make_shape(1, T, S, H=H, D=D, Hk=H, topk=k)
    nws = b.workspace_bytes(shape, b.OP_INDEX_BWD)
    assert nws > 0
    dq = torch.full((1, T, H, D), float("nan"), device="cuda")
    dk = torch.full((1, S, H, D), float("nan"), device="cuda")
    dw = torch.full((1, T, H), float("nan"), device="cuda")
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    b.index_backward(q.cuda(), kk.cuda(), torch.from_numpy(w).cuda(), torch.from_numpy(idx).cuda(),
                     torch.from_numpy(dI).cuda(), dq, dk, dw, workspace=ws)
    torch.cuda.synchronize()
    dq, dk, dw = (x.cpu().numpy().astype(np.float64) for x in (dq, dk, dw))
    r = np.asarray(rows)
    rq, rk, rw = O.index_scores_backward_selected(qh[:, r], kh, w[:, r].astype(np.float64), idx[:, r],
                                                  dI[:, r].astype(np.float64))
    for i, t in enumerate(rows):
        if t in SAMPLED_QUERIES:
            assert max_abs_rel(dq[0, t], rq[0, i]) <= 1e-5, (t, max_abs_rel(dq[0, t], rq[0, i]))
            assert max_abs_rel(dw[0, t], rw[0, i]) <= 1e-5, (t, max_abs_rel(dw[0, t], rw[0, i]))
    for j in SAMPLED_KEYS:   # every query that names j is among the rows given to the oracle
        assert max_abs_rel(dk[0, j], rk[0, j]) <= 1e-5, (j, max_abs_rel(dk[0, j], rk[0, j]))
