"""GPU parity of the sparse MLA backward (dsa_sparse_mla_backward) against the oracle.

The GPU takes the forward's own results (output, log-sum-exp) from dsa_sparse_mla_attention
on the same inputs; the oracle recomputes everything in float64 from the stored inputs.
Bars as for the forward: max-abs-relative error <= 1e-5 (fp32) and <= 2e-2 (bf16) per
gradient tensor.  The latent-row gradient collects its contributions with fp32 atomics
in no fixed order, which the fp32 bar covers.
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
    b.sparse_mla_backward(qd, kvd, idd, scale, out, lse, dd, dq, dkv, Dc=Dc)
    torch.cuda.synchronize()
    return dq.cpu().numpy().astype(np.float64), dkv.cpu().numpy().astype(np.float64)


CASES = {
    # name: (B, T, S, Hm, Dc, Dr, k, dtype, tol)
    "fp32_small": (2, 5, 40, 8, 64, 16, 12, "f32", 1e-5),
    "fp32_odd_heads": (1, 4, 30, 3, 40, 8, 9, "f32", 1e-5),
    "bf16_mla_dims": (1, 24, 300, 64, 512, 64, 64, "bf16", 2e-2),
    "bf16_decode": (3, 1, 5000, 64, 512, 64, 2048, "bf16", 2e-2),
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


def test_sparse_mla_backward_empty_selections():
    B, T, S, Hm, Dc, Dr = 1, 3, 16, 8, 64, 16
    rng = np.random.default_rng(5)
    q, kv, dout, idx, _ = _inputs(rng, B, T, S, Hm, Dc, Dr, 4, "f32")
    idx[:] = -1
    dq, dkv = _run(q, kv, dout, idx, Dc, 0.1, "f32")
    assert np.all(dq == 0) and np.all(dkv == 0)
