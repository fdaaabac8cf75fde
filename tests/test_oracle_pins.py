"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a hand-worked value, a library routine
(torch on the CPU), brute force, or an identity of the mathematics, chosen so
that a dropped term, a wrong sign or index, or a transposed operand fails one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- decoding

def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref, equal_nan=True)


def test_e4m3fn_table_matches_torch_and_format_facts():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.E4M3FN, ref, equal_nan=True)
    assert O.E4M3FN[0x7E] == 448.0 and O.E4M3FN[0xFE] == -448.0
    assert O.E4M3FN[0x01] == 2.0 ** -9 and O.E4M3FN[0x38] == 1.0
    assert np.isnan(O.E4M3FN[0x7F]) and np.isnan(O.E4M3FN[0xFF])
    assert np.isfinite(np.delete(O.E4M3FN, [0x7F, 0xFF])).all()


def test_fp8_decode_applies_per_vector_scale():
    codes = np.array([[0x38, 0x40], [0xB8, 0x00]], np.uint8)      # [[1, 2], [-1, 0]]
    sc = np.array([0.5, 3.0], np.float32)
    assert np.array_equal(O.decode(codes, "fp8", sc), [[0.5, 1.0], [-3.0, 0.0]])


# ---------------------------------------------------------------- index score

def test_index_score_hand_example_per_head_keys():
    g = _gold("index_score_hand.json")
    q = np.array(g["q"], float)[None]                 # [1, H=2, D=3]
    k = np.array(g["k_per_head"], float)              # [S=3, Hk=2, D=3]
    w = np.array(g["w"], float)[None]
    assert np.array_equal(O.index_scores_loop(q, k, w)[0], g["expected_per_head"])
    assert np.array_equal(O.index_scores_row(q[0], k, w[0], 0, 3), g["expected_per_head"])
    # a sub-range returns the same positions' scores
    assert np.array_equal(O.index_scores_row(q[0], k, w[0], 1, 3), g["expected_per_head"][1:])


def test_index_score_hand_example_shared_key():
    g = _gold("index_score_hand.json")
    q = np.array(g["q"], float)[None]
    k = np.array(g["k_shared"], float)[:, None, :]    # [S=3, Hk=1, D=3]
    w = np.array(g["w"], float)[None]
    assert np.array_equal(O.index_scores_loop(q, k, w)[0], g["expected_shared"])
    assert np.array_equal(O.index_scores_row(q[0], k, w[0], 0, 3), g["expected_shared"])


def _rand_index(rng, T=5, S=7, H=3, D=4, Hk=None):
    Hk = H if Hk is None else Hk
    return rng.standard_normal((T, H, D)), rng.standard_normal((S, Hk, D)), rng.random((T, H))


@pytest.mark.parametrize("hk_one", [False, True])
def test_index_score_loop_equals_vectorised(hk_one):
    rng = np.random.default_rng(11)
    q, k, w = _rand_index(rng, Hk=1 if hk_one else None)
    ref = O.index_scores_loop(q, k, w)
    ks = np.zeros((1, 5), np.int32)
    ke = np.full((1, 5), 7, np.int32)
    got = O.index_scores(q[None], k[None], w[None], ks, ke)[0]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_index_score_relu_identities_catch_sign_and_index_errors():
    # relu(x) + relu(-x) = |x| and relu(x) - relu(-x) = x, summed with the head weights.
    rng = np.random.default_rng(12)
    q, k, w = _rand_index(rng, T=3, S=6, H=4, D=5)
    pos = O.index_scores_loop(q, k, w)
    neg = O.index_scores_loop(-q, k, w)
    dots = np.stack([q[:, h, :] @ k[:, h, :].T for h in range(4)], axis=-1)   # [T, S, H]
    np.testing.assert_allclose(pos - neg, (dots * w[:, None, :]).sum(-1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(pos + neg, (np.abs(dots) * w[:, None, :]).sum(-1), rtol=1e-12, atol=1e-12)


def test_index_score_special_cases():
    rng = np.random.default_rng(13)
    q, k, w = _rand_index(rng)
    assert not O.index_scores_loop(q, k, np.zeros_like(w)).any()
    assert not O.index_scores_loop(np.zeros_like(q), k, w).any()
    assert np.array_equal(O.index_scores_loop(q, k, 2 * w), 2 * O.index_scores_loop(q, k, w))
    # one-hot: q[t,h] = e_h, k[s,h] = c_s * e_h  =>  I[t,s] = sum_h w[t,h] * max(c_s, 0)
    H = D = 3
    q1 = np.broadcast_to(np.eye(H, D), (2, H, D)).copy()
    c = np.array([2.0, -1.0, 0.5, 0.0])
    k1 = c[:, None, None] * np.eye(H, D)[None]
    w1 = np.array([[1.0, 2.0, 3.0], [0.0, 1.0, 0.0]])
    exp = np.outer(w1.sum(1), np.maximum(c, 0))
    assert np.array_equal(O.index_scores_loop(q1, k1, w1), exp)


def test_index_score_shared_key_equals_replicated_keys():
    rng = np.random.default_rng(14)
    q, k1, w = _rand_index(rng, Hk=1)
    kH = np.repeat(k1, 3, axis=1)
    a = O.index_scores_row(q[2], k1, w[2], 0, 7)
    b = O.index_scores_row(q[2], kH, w[2], 0, 7)
    np.testing.assert_allclose(a, b, rtol=1e-15, atol=0)
    assert np.array_equal(O.index_scores_loop(q, k1, w), O.index_scores_loop(q, kH, w))


# ---------------------------------------------------------------- top-k

def _brute_topk(scores, ks, k):
    """The unique k-subset whose every member beats every non-member on (score desc, position asc)."""
    n = len(scores)
    if n <= k:
        return list(range(ks, ks + n))
    found = []
    for sub in itertools.combinations(range(n), k):
        inside = set(sub)
        ok = all((scores[x] > scores[y]) or (scores[x] == scores[y] and x < y)
                 for x in inside for y in range(n) if y not in inside)
        if ok:
            found.append(sub)
    assert len(found) == 1
    return [ks + i for i in found[0]]


def test_topk_matches_brute_force_with_ties_and_signed_zeros():
    rng = np.random.default_rng(21)
    values = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.0])
    for trial in range(300):
        n = int(rng.integers(0, 10))
        k = int(rng.integers(1, 5))
        ks = int(rng.integers(0, 3))
        s = values[rng.integers(0, len(values), n)]
        idx, tau = O.topk_row(s, ks, ks + n, k)
        exp = _brute_topk(list(s), ks, k)
        assert list(idx[:len(exp)]) == exp
        assert (idx[len(exp):] == -1).all()
        if n > k:
            assert tau == sorted(s, reverse=True)[k - 1]


def test_topk_short_prefix_pads_with_minus_one():
    g = _gold("short_prefix_pad.json")
    rng = np.random.default_rng(22)
    n, k = g["prefix_len"], g["index_topk"]
    idx, tau = O.topk_row(rng.standard_normal(n), 0, n, k)
    assert tau is None and idx.shape == (k,)
    assert (idx >= 0).sum() == g["expected_valid"] and (idx == -1).sum() == g["expected_pad"]
    assert list(idx[:4]) == g["expected_first_positions"]
    assert idx[g["expected_valid"] - 1] == g["expected_last_valid_position"]


def test_topk_matches_torch_topk_as_sets_on_continuous_scores():
    rng = np.random.default_rng(23)
    for n, k in [(100, 7), (5000, 2048), (3000, 1)]:
        s = rng.standard_normal(n)
        idx, _ = O.topk_row(s, 0, n, k)
        ref = torch.topk(torch.from_numpy(s), k).indices.numpy()
        assert set(idx.tolist()) == set(ref.tolist())
        assert (np.diff(idx) > 0).all()


def test_topk_invariant_under_increasing_transform_and_offset():
    rng = np.random.default_rng(24)
    s = np.round(rng.standard_normal(500) * 3) / 3        # many ties
    a, _ = O.topk_row(s, 10, 510, 64)
    b, _ = O.topk_row(np.exp(s) * 3 + 1, 10, 510, 64)
    assert np.array_equal(a, b)
    assert a.min() >= 10 and a.max() < 510


def test_topk_all_equal_takes_lowest_positions():
    s = np.where(np.arange(40) % 2 == 0, 0.0, -0.0)
    idx, tau = O.topk_row(s, 5, 45, 8)
    assert list(idx) == list(range(5, 13)) and tau == 0.0


# ---------------------------------------------------------------- sparse MLA

def _sdpa_causal(q, kv, Dc, scale):
    """Dense causal attention by torch's library routine, float64."""
    T, Hm, R = q.shape
    S = kv.shape[0]
    qq = torch.from_numpy(q).permute(1, 0, 2)[None]                 # [1, Hm, T, R]
    kk = torch.from_numpy(kv)[None, None].expand(1, Hm, S, R)
    vv = torch.from_numpy(np.ascontiguousarray(kv[:, :Dc]))[None, None].expand(1, Hm, S, Dc)
    pos = np.arange(T)[:, None] + (S - T)
    mask = torch.from_numpy(np.arange(S)[None, :] <= pos)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_sparse_mla_with_topk_ge_prefix_equals_dense_causal_attention():
    rng = np.random.default_rng(31)
    T = S = 12
    Hm, Dc, Dr, k = 3, 6, 2, 16
    q = rng.standard_normal((T, Hm, Dc + Dr))
    kv = rng.standard_normal((S, Dc + Dr))
    sc = rng.standard_normal((T, S))
    scale = 1 / math.sqrt(Dc + Dr)
    o = np.zeros((T, Hm, Dc))
    for t in range(T):
        idx, tau = O.topk_row(sc[t, :t + 1], 0, t + 1, k)
        assert tau is None
        o[t] = O.sparse_mla_row(q[t], kv, idx, scale, Dc)[0]
    np.testing.assert_allclose(o, _sdpa_causal(q, kv, Dc, scale), rtol=1e-12, atol=1e-13)


def test_sparse_mla_decode_row_equals_dense_attention_over_prefix():
    rng = np.random.default_rng(32)
    S, Hm, Dc, Dr = 20, 4, 8, 4
    q = rng.standard_normal((1, Hm, Dc + Dr))
    kv = rng.standard_normal((S, Dc + Dr))
    idx = np.concatenate([np.arange(S), -np.ones(12)]).astype(np.int32)
    o, _ = O.sparse_mla_row(q[0], kv, idx, 0.3, Dc)
    np.testing.assert_allclose(o, _sdpa_causal(q, kv, Dc, 0.3)[0], rtol=1e-12, atol=1e-13)


def test_sparse_mla_closed_forms():
    rng = np.random.default_rng(33)
    S, Hm, Dc, Dr = 30, 2, 5, 3
    kv = rng.standard_normal((S, Dc + Dr))
    idx = np.array([3, 7, 11, 29, -1, -1], np.int32)
    o, lse = O.sparse_mla_row(np.zeros((Hm, Dc + Dr)), kv, idx, 0.7, Dc)
    np.testing.assert_allclose(o, np.broadcast_to(kv[[3, 7, 11, 29], :Dc].mean(0), (Hm, Dc)), rtol=1e-13)
    np.testing.assert_allclose(lse, math.log(4), rtol=1e-14)
    q = rng.standard_normal((Hm, Dc + Dr))
    o1, lse1 = O.sparse_mla_row(q, kv, np.array([17, -1], np.int32), 0.7, Dc)
    assert np.array_equal(o1, np.broadcast_to(kv[17, :Dc], (Hm, Dc)))
    np.testing.assert_allclose(lse1, 0.7 * (q @ kv[17]), rtol=1e-14)
    o0, l0 = O.sparse_mla_row(q, kv, np.full(4, -1, np.int32), 0.7, Dc)
    assert not o0.any() and np.isneginf(l0).all()


def test_sparse_mla_order_free_and_gather_equals_dense_masked():
    rng = np.random.default_rng(34)
    S, Hm, Dc, Dr = 50, 3, 7, 2
    kv = rng.standard_normal((S, Dc + Dr))
    q = rng.standard_normal((Hm, Dc + Dr))
    idx = rng.choice(S, 20, replace=False).astype(np.int32)
    a, la = O.sparse_mla_row(q, kv, idx, 0.4, Dc)
    b, lb = O.sparse_mla_row(q, kv, rng.permutation(idx), 0.4, Dc)
    c, lc = O.sparse_mla_dense_masked_row(q, kv, idx, 0.4, Dc)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(a, c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(la, lc, rtol=1e-14)


# ---------------------------------------------------------------- IndexShare

def test_pattern_fsss_over_78_layers():
    g = _gold("indexshare_patterns.json")["fsss_78"]
    types = O.parse_pattern(g["pattern"], g["n_layers"])
    full = [i for i, t in enumerate(types) if t == "full"]
    shared = [i for i, t in enumerate(types) if t == "shared"]
    assert len(full) == g["n_full"] and len(shared) == g["n_shared"]
    assert full[:4] == g["first_full_layers"] and shared[:6] == g["first_shared_layers"]
    assert round(100 * len(shared) / g["n_layers"], 1) == g["pruned_percent_1dp"]
    assert O.served_group_sizes(types) == g["served_group_sizes"]


def test_donors_follow_indexer_types_not_layer_modulo():
    g = _gold("indexshare_patterns.json")["public_config_prefix"]
    assert O.donor_map(g["indexer_types"]) == g["donors"]
    with pytest.raises(O.NoDonorError):
        O.donor_map(["shared", "full"])
    assert O.donor_map(["shared", "full"], cache_valid=True) == [-1, 1]


def _tiny_group(rng, types, B=2, T=9, S=9, H=2, D=4, Hm=2, Dc=4, Dr=2):
    layers = []
    for ty in types:
        L = {"mla_q": rng.standard_normal((B, T, Hm, Dc + Dr)), "kv": rng.standard_normal((B, S, Dc + Dr))}
        if ty == "full":
            L.update(idx_q=rng.standard_normal((B, T, H, D)), idx_k=rng.standard_normal((B, S, H, D)),
                     w=rng.random((B, T, H)))
        layers.append(L)
    ke = np.broadcast_to(np.arange(1, T + 1) + (S - T), (B, T)).astype(np.int32)
    return layers, np.zeros_like(ke), ke


def test_group_shared_layers_reuse_donor_indices_byte_for_byte():
    rng = np.random.default_rng(41)
    types = ["full", "full", "full", "shared", "shared", "shared", "full", "shared"]
    layers, ks, ke = _tiny_group(rng, types)
    res = O.group_forward(layers, types, ks, ke, 4, 0.5, 4)
    for l, d in enumerate(res["donors"]):
        assert res["indices"][l].tobytes() == res["indices"][d].tobytes()
    # each layer's attention uses its own q and kv with the donor's indices
    for l in range(len(types)):
        o, _ = O.sparse_mla(layers[l]["mla_q"], layers[l]["kv"], res["indices"][res["donors"][l]], 0.5, 4)
        assert np.array_equal(o, res["out"][l])


def test_group_all_full_with_copied_index_inputs_equals_fsss():
    rng = np.random.default_rng(42)
    fsss = ["full", "shared", "shared", "shared"]
    layers, ks, ke = _tiny_group(rng, fsss)
    for l in range(1, 4):
        layers[l].update({k: layers[0][k] for k in ("idx_q", "idx_k", "w")})
    a = O.group_forward(layers, fsss, ks, ke, 4, 0.5, 4)
    b = O.group_forward(layers, ["full"] * 4, ks, ke, 4, 0.5, 4)
    for l in range(4):
        assert np.array_equal(a["out"][l], b["out"][l]) and np.array_equal(a["indices"][l], b["indices"][l])
    kw = dict(H=2, D=4, Hk=2, idx_bytes=4, idx_scaled=False, topk_k=4, Hm=2, Dc=4, Dr=2, mla_bytes=4, S=9)
    sa, sb = O.group_stats(fsss, ks, ke, **kw), O.group_stats(["full"] * 4, ks, ke, **kw)
    for key in sa:
        if key in ("indexer_flops", "indexer_bytes", "topk_bytes"):
            assert sb[key] == 4 * sa[key]
        elif key in ("n_full", "n_shared"):
            continue
        else:
            assert sa[key] == sb[key]


def test_group_cached_handle_rules():
    rng = np.random.default_rng(43)
    layers, ks, ke = _tiny_group(rng, ["full", "shared"])
    first = O.group_forward(layers, ["full", "shared"], ks, ke, 4, 0.5, 4, tag=7)
    with pytest.raises(O.NoDonorError):
        O.group_forward(layers[1:], ["shared"], ks, ke, 4, 0.5, 4)
    with pytest.raises(O.StaleCacheError):
        O.group_forward(layers[1:], ["shared"], ks, ke, 4, 0.5, 4, cache=first["cache"], tag=8)
    again = O.group_forward(layers[1:], ["shared"], ks, ke, 4, 0.5, 4, cache=first["cache"], tag=7)
    assert np.array_equal(again["out"][0], first["out"][1])


def test_group_stats_closed_forms_causal_prefill():
    T, k = 100, 16
    ke = np.arange(1, T + 1, dtype=np.int32)[None]
    ks = np.zeros_like(ke)
    st = O.group_stats(["full", "shared", "shared", "shared"], ks, ke, H=4, D=8, Hk=4, idx_bytes=2,
                       idx_scaled=False, topk_k=k, Hm=2, Dc=8, Dr=4, mla_bytes=2, S=T)
    sum_n = T * (T + 1) // 2
    sum_j = k * (k + 1) // 2 + (T - k) * k
    assert st["indexer_flops"] == 2 * 4 * 8 * sum_n
    assert st["attn_flops"] == 4 * 2 * 2 * (2 * 8 + 4) * sum_j
    assert st["topk_bytes"] == 4 * sum_n + 4 * T * k
    assert (st["n_full"], st["n_shared"]) == (1, 3)
