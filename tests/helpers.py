"""Shared test helpers: device upload of stored synthetic inputs and comparison rules."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from dsa_indexer_top_lightning_amd import synth

TIE_BAND = 1e-3          # relative band around the k-th score (index parity rule)
ATTN_TOL = {"f32": 1e-5, "bf16": 2e-2}


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Stored host array -> device tensor of the matching torch dtype."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).cuda().view(torch.float8_e4m3fn)
    raise ValueError(dtype)


def f32_dev(arr) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def i32_dev(arr) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).cuda()


def decode_index(L: dict, w: synth.Workload):
    """float64 index q, k, w of a layer's stored inputs (oracle side)."""
    q = O.decode(L["idx_q"], w.idx_dtype, L.get("idx_q_scale"))
    k = O.decode(L["idx_k"], w.idx_dtype, L.get("idx_k_scale"))
    return q, k, L["w"].astype(np.float64)


def index_abs_bound(q64, k64, w64, Hk):
    """Sum_h |w| * sum_d |q k| per (t, s): scale of the fp32 accumulation error of one score."""
    aq, ak = np.abs(q64), np.abs(k64)
    if Hk == q64.shape[-2]:
        per_head = np.einsum("thd,shd->tsh", aq, ak)
    else:
        per_head = np.einsum("thd,sd->tsh", aq, ak[:, 0, :])
    return (per_head * np.abs(w64)[:, None, :]).sum(-1)


def max_abs_rel(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / den) if den > 0 else float(np.max(np.abs(got)))


def check_topk_row(gpu: np.ndarray, ref: np.ndarray, scores_row: np.ndarray, key_start: int, tau):
    """Index parity for one row: identical, or differing only inside the tie band.

    ``scores_row`` are the oracle's scores of the row's candidates in position order.
    Returns True when the row is byte-identical to the oracle's.
    """
    nref = int((ref >= 0).sum())
    ngpu = int((gpu >= 0).sum())
    assert ngpu == nref, f"valid count {ngpu} != {nref}"
    assert (gpu[ngpu:] == -1).all(), "tail must be -1"
    v = gpu[:ngpu]
    assert (np.diff(v) > 0).all(), "valid indices must be ascending and unique"
    if np.array_equal(gpu, ref):
        return True
    assert tau is not None, "rows with n <= topk must match exactly"
    band = TIE_BAND * abs(tau)
    diff = np.setxor1d(v, ref[:nref])
    sc = scores_row[diff - key_start]
    assert np.all(np.abs(sc - tau) <= band), \
        f"differing positions {diff[:8]} have scores {sc[:8]} outside the band around tau={tau}"
    return False
