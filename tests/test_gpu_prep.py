"""GPU parity of the decode-step preparation calls (dsa_index_prep, dsa_latent_append)
against the oracle's prep_index_vectors / cache_append.

Both sides form the RoPE angle and the rotation in float64 and round once to float32,
so they differ only where the two float64 libraries' pow / sin / cos differ in the
last bits.  Bars: dims outside the rotated half, position 0 and small positions are
bit-exact; at other positions a bf16 value lies within one bf16 ulp of the oracle's
float64 value, an fp8 scale within one float32 ulp of the oracle's, and each decoded
code within half an e4m3 step (in scaled units) of the oracle's float64 value divided
by the kernel's scale.  Both slacks also allow for an angle that the two libraries
round differently (a few float64 ulps of pos * inv).  Latent rows are copied
bit-exactly and cache rows that no new token names stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle as O
from dsa_indexer_top_lightning_amd import binding as b

pytestmark = pytest.mark.gpu

THETA = 8.0e6
POSITIONS = [0, 1, 5, 777, 4095, 131071, 1048575, 2]
SMALL_POS = 5          # positions up to this are compared bit-exactly


def _x(rng, n, heads, D):
    x = rng.standard_normal((n, heads, D)).astype(np.float32)
    x[0, 0] = 0.0                                   # all-zero vector: scale 1, codes 0
    if n > 1:
        x[1, -1] *= np.float32(3.0e3)               # large magnitudes
    return x


def _pos(n):
    return np.array([POSITIONS[i % len(POSITIONS)] for i in range(n)], dtype=np.int32)


def _angle_slack(x, pos):
    """Per element: a bound on what differently rounded float64 angles (a few ulps of
    pos * inv) can move a rotated value: |d angle| * (|a| + |b|) of its pair."""
    D = x.shape[-1]
    r, half = D // 2, D // 4
    a = np.abs(x[..., D - r:D - r + half].astype(np.float64))
    bb = np.abs(x[..., D - r + half:].astype(np.float64))
    dang = 8.0 * 2.0 ** -52 * (1.0 + np.asarray(pos, dtype=np.float64))[:, None, None]
    s = np.zeros(x.shape, dtype=np.float64)
    s[..., D - r:D - r + half] = dang * (a + bb)
    s[..., D - r + half:] = dang * (a + bb)
    return s


def _bf16_ulp(v):
    v = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(v)) - 7)


def _e4m3_half_step(v):
    a = np.minimum(np.abs(v), 448.0)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * 2.0 ** (e - 3)                     # subnormals share the 2^-9 step of binade -6


def _check_bf16(got_bits, x, pos):
    want_bits, _ = O.prep_index_vectors(x, pos, THETA, "bf16")
    y64 = O.rope_last_half(x, pos, THETA)
    D = x.shape[-1]
    small = np.asarray(pos) <= SMALL_POS
    np.testing.assert_array_equal(got_bits[small], want_bits[small])
    np.testing.assert_array_equal(got_bits[..., :D - D // 2], want_bits[..., :D - D // 2])
    got = O.decode_bf16(got_bits).astype(np.float64)
    tol = _bf16_ulp(y64) + _angle_slack(x, pos)
    err = np.abs(got - y64)
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3f}"
    mism = np.mean(got_bits != want_bits)
    assert mism < 0.01, mism


def _check_fp8(got_codes, got_scale, x, pos):
    want_codes, want_scale = O.prep_index_vectors(x, pos, THETA, "fp8")
    y64 = O.rope_last_half(x, pos, THETA)
    small = np.asarray(pos) <= SMALL_POS
    np.testing.assert_array_equal(got_codes[small], want_codes[small])
    np.testing.assert_array_equal(got_scale[small], want_scale[small])
    lo = np.nextafter(want_scale, np.float32(0))
    hi = np.nextafter(want_scale, np.float32(np.inf))
    assert np.all((got_scale >= lo) & (got_scale <= hi))
    zero = ~np.any(x != 0, axis=-1)
    assert np.all(got_scale[zero] == 1.0) and np.all(got_codes[zero] == 0)
    s = got_scale.astype(np.float64)[..., None]
    v = y64 / s
    dec = O.E4M3FN[got_codes].astype(np.float64)
    tol = _e4m3_half_step(v) * (1 + 1e-6) + 1e-6 * np.abs(v) + _angle_slack(x, pos) / s
    err = np.abs(dec - np.clip(v, -448.0, 448.0))
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3f}"
    assert np.all(np.max(np.abs(dec), axis=-1)[~zero] == 448.0)     # the amax element maps to 448
    assert np.mean(got_codes != want_codes) < 0.01


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("n,heads,D", [(5, 32, 128), (9, 1, 128), (3, 4, 1024), (17, 3, 4), (8, 16, 32)])
def test_index_prep_queries(dtype, n, heads, D):
    rng = np.random.default_rng(1000 + n * 7 + heads + D)
    x = _x(rng, n, heads, D)
    pos = _pos(n)
    xd = torch.from_numpy(x).cuda()
    pd = torch.from_numpy(pos).cuda()
    if dtype == "bf16":
        out = torch.full((n, heads, D), 0x7FC1, dtype=torch.int16, device="cuda")
        b.index_prep(xd, pd, out, rope_theta=THETA)
        torch.cuda.synchronize()
        _check_bf16(out.cpu().numpy().view(np.uint16), x, pos)
    else:
        out = torch.full((n, heads, D), 0x55, dtype=torch.uint8, device="cuda")
        sc = torch.full((n, heads), -1.0, dtype=torch.float32, device="cuda")
        b.index_prep(xd, pd, out, sc, rope_theta=THETA)
        torch.cuda.synchronize()
        _check_fp8(out.cpu().numpy(), sc.cpu().numpy(), x, pos)


def test_index_prep_long_context_positions():
    """Every position of a 1M-token context in one call (4 key heads of D = 128, bf16)."""
    rng = np.random.default_rng(77)
    n = 1 << 20
    pos = rng.permutation(n).astype(np.int32)[:4096]
    x = rng.standard_normal((pos.size, 1, 128)).astype(np.float32)
    out = torch.empty((pos.size, 1, 128), dtype=torch.int16, device="cuda")
    b.index_prep(torch.from_numpy(x).cuda(), torch.from_numpy(pos).cuda(), out, rope_theta=THETA)
    torch.cuda.synchronize()
    _check_bf16(out.cpu().numpy().view(np.uint16), x, pos)


@pytest.mark.parametrize("dtype,Hk", [("bf16", 32), ("bf16", 1), ("fp8", 1), ("fp8", 32)])
def test_decode_cache_append(dtype, Hk):
    """A decode step of B streams appends its new index keys and latent rows at
    row b * s_cap + pos[b]; streams past the cache (row >= n_rows) or with a negative
    row are skipped, every other row keeps its contents."""
    rng = np.random.default_rng(31 + Hk)
    B, s_cap, D, R = 7, 300, 128, 576
    n_rows = (B - 1) * s_cap                        # the last stream's row lies past the cache
    pos = np.array([0, 5, 299, 17, 128, 200, 3], dtype=np.int32)
    rows = np.arange(B, dtype=np.int64) * s_cap + pos
    rows[3] = -1                                    # stream 3 inactive
    x = _x(rng, B, Hk, D)
    kv_new = torch.randn(B, R, dtype=torch.bfloat16)
    kv_cache0 = torch.randn(n_rows, R, dtype=torch.bfloat16)
    if dtype == "bf16":
        k0 = rng.integers(0, 1 << 16, size=(n_rows, Hk, D), dtype=np.uint16)
        s0 = None
    else:
        k0 = rng.integers(0, 256, size=(n_rows, Hk, D), dtype=np.uint8)
        s0 = rng.random((n_rows, Hk), dtype=np.float32)
    want_k, want_s, want_kv = O.cache_append(k0, s0, kv_cache0.view(torch.int16).numpy(), x, pos, rows, THETA,
                                             dtype, kv_new=kv_new.view(torch.int16).numpy())

    kd = torch.from_numpy(k0.view(np.int16) if dtype == "bf16" else k0).cuda()
    sd = None if s0 is None else torch.from_numpy(s0).cuda()
    kvd = kv_cache0.cuda()
    rows_d = torch.from_numpy(rows).cuda()
    b.index_prep(torch.from_numpy(x).cuda(), torch.from_numpy(pos).cuda(), kd, sd, rows=rows_d, rope_theta=THETA)
    b.latent_append(kv_new.cuda(), rows_d, kvd)
    torch.cuda.synchronize()

    got_k = kd.cpu().numpy().view(np.uint16 if dtype == "bf16" else np.uint8)
    np.testing.assert_array_equal(kvd.cpu().view(torch.int16).numpy(), want_kv)
    hit = np.array([0 <= r < n_rows for r in rows])
    written = rows[hit]
    untouched = np.ones(n_rows, dtype=bool)
    untouched[written] = False
    np.testing.assert_array_equal(got_k[untouched], want_k[untouched])
    if dtype == "bf16":
        _check_bf16(got_k[written], x[hit], pos[hit])
    else:
        got_s = sd.cpu().numpy()
        np.testing.assert_array_equal(got_s[untouched], want_s[untouched])
        _check_fp8(got_k[written], got_s[written], x[hit], pos[hit])


def test_latent_append_f32_rows():
    rng = np.random.default_rng(5)
    n, R, n_rows = 33, 68, 100
    new = torch.from_numpy(rng.standard_normal((n, R)).astype(np.float32))
    cache0 = torch.from_numpy(rng.standard_normal((n_rows, R)).astype(np.float32))
    rows = torch.from_numpy(rng.permutation(n_rows + 20)[:n].astype(np.int64) - 10)   # some out of range
    want = cache0.clone()
    for i, r in enumerate(rows.tolist()):
        if 0 <= r < n_rows:
            want[r] = new[i]
    got = cache0.cuda()
    b.latent_append(new.cuda(), rows.cuda(), got)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), want)
