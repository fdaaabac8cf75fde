"""The seeded input generator: storage codecs against torch's, block regeneration."""
import numpy as np
import pytest
import torch

from dsa_indexer_top_lightning_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.integers(0, 2**31, 100000, dtype=np.uint32)).view(np.float32)])
    x = x[np.isfinite(x)]
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_encoder_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(2)
    # every representable value, every midpoint between neighbours, and random values
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = np.sort(vals[np.isfinite(vals)])
    mids = (fin[1:] + fin[:-1]) / 2
    x = np.concatenate([fin, mids, rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01])
    x = x.astype(np.float32)
    ours = synth.f64_to_e4m3_codes(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch maps -0.0 to 0x80 and keeps signs of zero; so do we
    assert np.array_equal(ours, ref)


def test_fp8_quantisation_saturates_and_scales():
    x = np.array([[448.0 * 3, -1.0, 0.0, 2.0]])
    codes, sc = synth.quantize_fp8_rows(x)
    assert sc.dtype == np.float32 and np.isclose(sc[0], 3.0)
    back = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * sc[:, None]
    assert np.abs(back - x).max() <= 3.0 * 16            # within half an ulp of the top binade
    zc, zs = synth.quantize_fp8_rows(np.zeros((2, 8)))
    assert (zc == 0).all() and (zs == 1.0).all()


def test_blocks_regenerate_identically_and_slices_agree():
    w = synth.WORKLOADS["prefill4k_bf16"].with_(T=5000, S=5000)
    a = synth.index_k_rows(w, 0, 0, 4000, 4200)
    b = synth.index_k_rows(w, 0, 0, 0, 5000)[4000:4200]
    assert np.array_equal(a, b)
    c = synth.mla_kv_rows(w, 2, 0, 4095, 4097)
    assert np.array_equal(c, synth.mla_kv_rows(w, 2, 0, 0, 5000)[4095:4097])
    assert not np.array_equal(synth.mla_kv_rows(w, 1, 0, 0, 4), synth.mla_kv_rows(w, 2, 0, 0, 4))


def test_rope_touches_only_last_half_and_keeps_norms():
    w = synth.WORKLOADS["prefill4k_bf16"].with_(T=64, S=64)
    x = synth.draw_rows(w.seed, synth.TID_IDX_Q, 0, 0, 0, 64, w.H * w.D).reshape(64, w.H, w.D).astype(np.float64)
    y = synth.rope_last_half(x, np.arange(64))
    assert np.array_equal(x[..., :64], y[..., :64])
    np.testing.assert_allclose(np.linalg.norm(x[..., 64:], axis=-1), np.linalg.norm(y[..., 64:], axis=-1), rtol=1e-12)
    assert np.array_equal(x[0], y[0])                    # position 0 is not rotated


def test_planted_keys_fraction_and_direction():
    w = synth.WORKLOADS["decode1m_b4_fp8"].with_(S=20000, pos0=19999)
    k = synth.index_k_rows(w, 0, 1, 0, 20000)
    base = synth.draw_rows(w.seed, synth.TID_IDX_K, 0, 1, 0, 20000, w.Hk * w.D).reshape(-1, w.Hk, w.D)
    moved = np.abs(k - base).max(axis=(1, 2)) > 0
    assert 0.04 < moved.mean() < 0.06
    q = synth.index_q_rows(w, 0, 1, 0, 1)[0]
    u = q / np.linalg.norm(q, axis=-1, keepdims=True)
    proj = ((k - base)[moved] * u[None]).sum(-1) / np.sqrt(w.D)      # = gamma per (key, head)
    assert proj.min() >= 0.5 - 1e-9 and proj.max() <= 1.5 + 1e-9


def test_workload_key_ranges():
    w = synth.WORKLOADS["chunk128k_fp8"]
    ke = w.key_end()
    assert ke.shape == (1, 4096) and ke[0, 0] == 126977 and ke[0, -1] == 131072
    d = synth.WORKLOADS["decode32k_b64_bf16"].key_end()
    assert d.shape == (64, 1) and (d == 32768).all()


def test_packed_batch_key_ranges_and_positions():
    w = synth.WORKLOADS["packed_varlen_bf16"]
    ks, ke = w.key_start()[0].astype(np.int64), w.key_end()[0].astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(w.seqlens)])
    for i, n in enumerate(w.seqlens):
        o = cu[i]
        assert (ks[o:o + n] == o).all()                          # range starts at its sequence
        assert np.array_equal(ke[o:o + n], np.arange(o + 1, o + n + 1))   # causal inside it
        assert np.array_equal(w.positions(o, o + n, True), np.arange(n))  # RoPE restarts
    assert (ke - ks >= 1).all() and ke[-1] == w.S
    assert ((ke - ks) < w.topk).sum() > w.T // 3                  # many rows pad with -1
    assert {1, w.topk, w.topk + 1} <= set(int(x) for x in w.seqlens)


def test_packed_batch_shape_is_checked():
    with pytest.raises(ValueError):
        synth.WORKLOADS["packed_varlen_bf16"].with_(B=2)
