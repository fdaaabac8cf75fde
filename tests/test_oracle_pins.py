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
    assert np.array_equal(O.index_scores_rows(q, k, w)[0], g["expected_per_head"])
    # a sub-range returns the same positions' scores
    assert np.array_equal(O.index_scores_row(q[0], k, w[0], 1, 3), g["expected_per_head"][1:])


def test_index_score_hand_example_shared_key():
    g = _gold("index_score_hand.json")
    q = np.array(g["q"], float)[None]
    k = np.array(g["k_shared"], float)[:, None, :]    # [S=3, Hk=1, D=3]
    w = np.array(g["w"], float)[None]
    assert np.array_equal(O.index_scores_loop(q, k, w)[0], g["expected_shared"])
    assert np.array_equal(O.index_scores_row(q[0], k, w[0], 0, 3), g["expected_shared"])
    assert np.array_equal(O.index_scores_rows(q, k, w)[0], g["expected_shared"])


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
    np.testing.assert_allclose(O.index_scores_rows(q, k, w), ref, rtol=1e-12, atol=1e-14)


def test_index_score_relu_identities_catch_sign_and_index_errors():
    # relu(x) + relu(-x) = |x| and relu(x) - relu(-x) = x, summed with the head weights.
    rng = np.random.default_rng(12)
    q, k, w = _rand_index(rng, T=3, S=6, H=4, D=5)
    pos = O.index_scores_loop(q, k, w)
    neg = O.index_scores_loop(-q, k, w)
    for f in (O.index_scores_rows,):      # the batched form obeys the same identities
        np.testing.assert_allclose(f(q, k, w) - f(-q, k, w), pos - neg, rtol=1e-12, atol=1e-12)
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


def test_batched_topk_with_key_start_offsets_matches_brute_force():
    # the batched call slices each row to [key_start, key_end) of absolute positions;
    # every row is checked against brute force over that row's own candidates
    rng = np.random.default_rng(25)
    values = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.0])
    B, T, S, k = 3, 7, 12, 4
    sc = values[rng.integers(0, len(values), (B, T, S))]
    ke = rng.integers(0, S + 1, (B, T)).astype(np.int32)
    ks = np.minimum(rng.integers(0, 6, (B, T)), ke).astype(np.int32)
    ks[0, 0], ke[0, 0] = 5, 12                 # n = 7 > k, candidates start at 5
    ks[1, 2], ke[1, 2] = 9, 12                 # n = 3 < k: all kept, then -1
    idx, tau = O.topk(sc, ks, ke, k)
    for bb in range(B):
        for t in range(T):
            a, z = int(ks[bb, t]), int(ke[bb, t])
            exp = _brute_topk(list(sc[bb, t, a:z]), a, k)
            assert list(idx[bb, t, :len(exp)]) == exp, (bb, t)
            assert (idx[bb, t, len(exp):] == -1).all()
            if z - a > k:
                assert tau[bb, t] == sorted(sc[bb, t, a:z], reverse=True)[k - 1]
            else:
                assert np.isnan(tau[bb, t])
    assert list(idx[0, 0]) == _brute_topk(list(sc[0, 0, 5:12]), 5, k) and idx[0, 0].min() >= 5


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


def test_group_stats_bytes_hand_counted():
    # two items, two queries each; item 0 reads keys [0, 7), item 1 keys [0, 10)
    ks = np.array([[0, 2], [1, 0]])
    ke = np.array([[3, 7], [10, 5]])            # n = 3, 5, 9, 5: sum 22; min(n, 3) summed: 12
    kw = dict(H=2, D=8, Hk=2, topk_k=3, Hm=2, Dc=4, Dr=2, S=10)
    bf = O.group_stats(["full", "shared", "shared"], ks, ke, idx_bytes=2, idx_scaled=False, mla_bytes=2, **kw)
    # index q 4 rows x 2 heads x 8 x 2 B = 128, w 4 x 2 x 4 B = 32, keys (7 + 10) x 2 x 8 x 2 B = 544,
    # scores written 22 x 4 B = 88
    assert bf["indexer_bytes"] == 128 + 32 + 544 + 88
    # per layer: 12 gathered rows x 6 x 2 B = 144, q 4 x 2 x 6 x 2 B = 96, out 4 x 2 x 4 x 2 B = 64
    assert bf["attn_bytes"] == 3 * (144 + 96 + 64)
    assert bf["topk_bytes"] == 22 * 4 + 4 * 3 * 4
    f8 = O.group_stats(["full", "full"], ks, ke, idx_bytes=1, idx_scaled=True, mla_bytes=4, **kw)
    # fp8: q 64 B, w 32, q scales 4 x 2 x 4 = 32, keys 272, key scales 17 x 2 x 4 = 136, scores 88
    assert f8["indexer_bytes"] == 2 * (64 + 32 + 32 + 272 + 136 + 88)
    assert f8["attn_bytes"] == 2 * (12 * 6 * 4 + 4 * 2 * 6 * 4 + 4 * 2 * 4 * 4)


# ------------------------------------------------------------------ decode-step preparation

def test_e4m3_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if not np.isnan(O.E4M3FN[c])], np.uint8)
    vals = O.E4M3FN[codes].astype(np.float32)
    got = O.encode_e4m3(vals)
    zero = vals == 0                          # -0.0 and +0.0 keep their sign bit
    assert np.array_equal(got[~zero], codes[~zero])
    assert np.array_equal(got[zero], codes[zero])


def test_e4m3_encoder_matches_torch_cast_in_range():
    # library routine: torch's float32 -> float8_e4m3fn cast (round to nearest even) on
    # random values, exact midpoints between neighbouring codes and subnormals, |x| <= 464
    rng = np.random.default_rng(4)
    vals = np.concatenate([
        rng.standard_normal(20000) * 40.0,
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000),
        (O.E4M3FN[0:126] + O.E4M3FN[1:127]) / 2.0,          # midpoints
        -(O.E4M3FN[0:126] + O.E4M3FN[1:127]) / 2.0,
        np.array([464.0, -464.0, 448.0]),
    ]).astype(np.float32)
    vals = vals[np.abs(vals) <= 464.0]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_e4m3(vals), ref)


def test_e4m3_encoder_saturates_and_flushes():
    v = np.array([449.0, 500.0, 1e30, -1e30, 2.0 ** -10, -(2.0 ** -10), 1.5 * 2.0 ** -10], np.float32)
    assert O.encode_e4m3(v).tolist() == [126, 126, 126, 254, 0, 128, 1]


def test_bf16_encoder_matches_torch_cast():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 3,
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 65504.0], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.encode_bf16(v), ref)


def test_rope_rotates_the_last_half_by_position():
    # unit vector on the first rope dim (index D - D/2) at position p: it turns into the
    # pair (D - D/2, D - D/4) by angle p (the pair's frequency is theta^0 = 1); the first
    # half of the vector is untouched
    D, p = 8, 3
    x = np.zeros((1, 1, D))
    x[0, 0, 4] = 1.0
    x[0, 0, 0] = 7.0
    y = O.rope_last_half(x, np.array([p]), 1.0e4)[0, 0]
    assert y[0] == 7.0 and np.allclose(y[1:4], 0)
    assert np.isclose(y[4], math.cos(p)) and np.isclose(y[6], math.sin(p))
    assert np.allclose(y[[5, 7]], 0)
    # second pair turns with frequency theta^(-2/(D/2)) = theta^-0.5
    x2 = np.zeros((1, 1, D))
    x2[0, 0, 7] = 1.0
    y2 = O.rope_last_half(x2, np.array([p]), 1.0e4)[0, 0]
    a = p * 1.0e4 ** -0.5
    assert np.isclose(y2[7], math.cos(a)) and np.isclose(y2[5], -math.sin(a))


def test_rope_invariants():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((5, 3, 16))
    k = rng.standard_normal((5, 3, 16))
    pos = np.array([0, 1, 17, 1000, 1048575])
    assert np.allclose(O.rope_last_half(q, np.zeros(5), 8e6), q)                   # position 0
    rq = O.rope_last_half(q, pos, 8e6)
    assert np.allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1))   # rotations
    # relative positions: q at m + d and k at n + d score like q at m and k at n
    d = 12345
    s0 = (O.rope_last_half(q, pos, 8e6) * O.rope_last_half(k, pos[::-1], 8e6)).sum(-1)
    s1 = (O.rope_last_half(q, pos + d, 8e6) * O.rope_last_half(k, pos[::-1] + d, 8e6)).sum(-1)
    assert np.allclose(s0, s1)


def test_fp32_quantisation_maps_the_largest_entry_to_448():
    rng = np.random.default_rng(7)
    y = (rng.standard_normal((10, 4, 128)) * rng.uniform(0.01, 100, (10, 4, 1))).astype(np.float32)
    y[3, 2] = 0.0
    codes, scale = O.quantize_e4m3_f32(y)
    amax_pos = np.argmax(np.abs(y), axis=-1)
    top = np.take_along_axis(codes, amax_pos[..., None], axis=-1)[..., 0] & 0x7F   # [10, 4]
    nonzero = np.ones((10, 4), bool)
    nonzero[3, 2] = False
    assert (top[nonzero] == 126).all()                            # |y| = amax encodes as 448
    assert scale[3, 2] == 1.0 and not codes[3, 2].any()
    err = np.abs(O.E4M3FN[codes] * scale[..., None] - y)
    step = np.maximum(np.abs(y), 2.0 ** -6 * scale[..., None]) * 2.0 ** -4 + 1e-30
    assert (err <= step * (1 + 1e-6)).all()                       # half an e4m3 step, 3-bit mantissa


def test_cache_append_writes_rows_and_skips_outside():
    rng = np.random.default_rng(8)
    N, Hk, D, R, rows_total = 3, 2, 16, 8, 6
    kc = np.zeros((rows_total, Hk, D), np.uint8)
    sc = np.ones((rows_total, Hk), np.float32)
    kv = np.zeros((rows_total, R), np.uint16)
    k_new = rng.standard_normal((N, Hk, D)).astype(np.float32)
    kv_new = rng.integers(0, 65535, (N, R)).astype(np.uint16)
    rows = np.array([4, -1, 6])                                    # -1 and 6 are outside
    k2, s2, kv2 = O.cache_append(kc, sc, kv, k_new, np.array([5, 6, 7]), rows, 8e6, "fp8", kv_new)
    codes, scales = O.prep_index_vectors(k_new, np.array([5, 6, 7]), 8e6, "fp8")
    assert np.array_equal(k2[4], codes[0]) and np.array_equal(s2[4], scales[0]) and np.array_equal(kv2[4], kv_new[0])
    untouched = [0, 1, 2, 3, 5]
    assert not k2[untouched].any() and (s2[untouched] == 1).all() and not kv2[untouched].any()


# ---------------------------------------------------------------- sparse MLA backward

def _sdpa_causal_grads(q, kv, Dc, scale, dout):
    """Gradients of dense causal attention w.r.t. q and the latent rows (keys = whole
    rows, values = their first Dc values) by torch autograd through its library
    attention routine, float64."""
    T, Hm, R = q.shape
    S = kv.shape[0]
    qt = torch.from_numpy(q).clone().requires_grad_(True)
    kvt = torch.from_numpy(kv).clone().requires_grad_(True)
    qq = qt.permute(1, 0, 2)[None]
    kk = kvt[None, None].expand(1, Hm, S, R)
    vv = kvt[:, :Dc][None, None].expand(1, Hm, S, Dc)
    pos = np.arange(T)[:, None] + (S - T)
    mask = torch.from_numpy(np.arange(S)[None, :] <= pos)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
    (o[0].permute(1, 0, 2) * torch.from_numpy(dout)).sum().backward()
    return qt.grad.numpy(), kvt.grad.numpy()


@pytest.mark.parametrize("T,S", [(10, 10), (3, 17)])
def test_sparse_mla_backward_with_topk_ge_prefix_equals_dense_causal_autograd(T, S):
    rng = np.random.default_rng(71 + T)
    Hm, Dc, Dr, k = 3, 6, 2, 32
    q = rng.standard_normal((1, T, Hm, Dc + Dr))
    kv = rng.standard_normal((1, S, Dc + Dr))
    dout = rng.standard_normal((1, T, Hm, Dc))
    scale = 0.37
    idx = np.full((1, T, k), -1, np.int64)
    for t in range(T):
        p = S - T + t
        idx[0, t, :p + 1] = np.arange(p + 1)
    dq, dkv = O.sparse_mla_backward(q, kv, idx, scale, Dc, dout)
    rq, rkv = _sdpa_causal_grads(q[0], kv[0], Dc, scale, dout[0])
    np.testing.assert_allclose(dq[0], rq, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkv[0], rkv, rtol=1e-11, atol=1e-12)


def test_sparse_mla_backward_matches_central_differences():
    """Scattered selections with -1 holes and a row listed twice: every gradient entry
    against a central difference of the forward oracle's loss sum(o * dout)."""
    rng = np.random.default_rng(73)
    B, T, S, Hm, Dc, Dr, k = 2, 2, 7, 2, 4, 2, 5
    q = rng.standard_normal((B, T, Hm, Dc + Dr))
    kv = rng.standard_normal((B, S, Dc + Dr))
    dout = rng.standard_normal((B, T, Hm, Dc))
    idx = np.array([[[0, 3, -1, 6, 2], [5, 5, 1, -1, -1]], [[4, -1, -1, -1, -1], [6, 0, 1, 2, 3]]])
    scale = 0.6
    dq, dkv = O.sparse_mla_backward(q, kv, idx, scale, Dc, dout)

    def loss(qq, kk):
        return float((O.sparse_mla(qq, kk, idx, scale, Dc)[0] * dout).sum())

    eps = 1e-6
    num_q = np.zeros_like(q)
    for i in np.ndindex(q.shape):
        a, b = q.copy(), q.copy()
        a[i] += eps
        b[i] -= eps
        num_q[i] = (loss(a, kv) - loss(b, kv)) / (2 * eps)
    num_kv = np.zeros_like(kv)
    for i in np.ndindex(kv.shape):
        a, b = kv.copy(), kv.copy()
        a[i] += eps
        b[i] -= eps
        num_kv[i] = (loss(q, a) - loss(q, b)) / (2 * eps)
    np.testing.assert_allclose(dq, num_q, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dkv, num_kv, rtol=1e-6, atol=1e-8)
    assert np.all(dkv[0, 1] != 0) and np.all(dkv[1, 5] == 0)   # row 1 of item 0 selected, row 5 of item 1 not


def test_sparse_mla_backward_single_row_and_empty_selection():
    """|J| = 1: P = 1, so dz = 0: no query gradient, and the row's gradient is the sum
    of the heads' output gradients in its value part and 0 in its rope part.  An empty
    selection contributes nothing."""
    rng = np.random.default_rng(74)
    Hm, Dc, Dr, S = 3, 5, 3, 6
    q = rng.standard_normal((1, 2, Hm, Dc + Dr))
    kv = rng.standard_normal((1, S, Dc + Dr))
    dout = rng.standard_normal((1, 2, Hm, Dc))
    idx = np.array([[[4, -1], [-1, -1]]])
    dq, dkv = O.sparse_mla_backward(q, kv, idx, 0.5, Dc, dout)
    assert np.allclose(dq, 0, atol=1e-14)
    want = np.zeros((S, Dc + Dr))
    want[4, :Dc] = dout[0, 0].sum(axis=0)
    np.testing.assert_allclose(dkv[0], want, atol=1e-14)


# ---------------------------------------------------------------- index score backward

def _index_loss(q, k, w, idx, dI):
    """sum over selected slots of dI * I at the slot's position, from the forward oracle."""
    B, T = q.shape[:2]
    S = k.shape[1]
    I = O.index_scores(q, k, w, np.zeros((B, T), np.int64), np.full((B, T), S, np.int64))
    tot = 0.0
    for b in range(B):
        for t in range(T):
            for j, s in enumerate(idx[b, t]):
                if 0 <= s < S:
                    tot += dI[b, t, j] * I[b, t, s]
    return tot


@pytest.mark.parametrize("Hk", [3, 1])
def test_index_backward_matches_central_differences(Hk):
    """Every gradient entry against a central difference of the forward oracle; scores are
    kept away from the ReLU kink so that the difference quotient is that of one branch."""
    rng = np.random.default_rng(81 + Hk)
    B, T, S, H, D, kk = 2, 2, 6, 3, 4, 4
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, S, Hk, D))
    w = rng.random((B, T, H))
    idx = np.array([[[0, 5, -1, 2], [3, 3, 1, 4]], [[5, -1, -1, -1], [1, 0, 2, 3]]])
    dI = rng.standard_normal((B, T, kk))
    g = np.arange(H) if Hk == H else np.zeros(H, int)
    for b in range(B):
        for t in range(T):
            for s in range(S):
                for h in range(H):
                    while abs(q[b, t, h] @ k[b, s, g[h]]) < 0.05:
                        k[b, s, g[h]] += 0.1
    dq, dk, dw = O.index_scores_backward_selected(q, k, w, idx, dI)
    eps = 1e-6
    for arr, grad in ((q, dq), (k, dk), (w, dw)):
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            a0 = arr[i]
            arr[i] = a0 + eps
            lp = _index_loss(q, k, w, idx, dI)
            arr[i] = a0 - eps
            lm = _index_loss(q, k, w, idx, dI)
            arr[i] = a0
            num[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_index_backward_closed_forms():
    """w = 0: no q or k gradient, dw = sum_j dI_j max(0, s); a single selected key with
    all scores positive: dq = dI w k, dk = dI sum_h w_h q_h (shared key)."""
    rng = np.random.default_rng(83)
    q = np.abs(rng.standard_normal((1, 1, 4, 8)))
    k = np.abs(rng.standard_normal((1, 5, 1, 8)))
    w = rng.random((1, 1, 4))
    idx = np.array([[[2, -1]]])
    dI = np.array([[[0.7, 5.0]]])
    dq, dk, dw = O.index_scores_backward_selected(q, k, np.zeros_like(w), idx, dI)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dw[0, 0], 0.7 * (q[0, 0] @ k[0, 2, 0]), rtol=1e-14)
    dq, dk, dw = O.index_scores_backward_selected(q, k, w, idx, dI)
    np.testing.assert_allclose(dq[0, 0], 0.7 * w[0, 0][:, None] * k[0, 2, 0][None, :], rtol=1e-14)
    want = np.zeros((5, 1, 8))
    want[2, 0] = 0.7 * (w[0, 0][:, None] * q[0, 0]).sum(axis=0)
    np.testing.assert_allclose(dk[0], want, rtol=1e-14)
