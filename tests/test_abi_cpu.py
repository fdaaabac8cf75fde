"""The C-ABI library on a host without a GPU: symbols, status strings, host-side
validation (every error returns before anything is enqueued), workspace sizing and
analytic stats.  No compute call is made here."""
import ctypes as C

import numpy as np
import pytest

import oracle as O
from dsa_indexer_top_lightning_amd import binding as b


@pytest.fixture(scope="module")
def L():
    return b.lib()


def test_library_exports_every_declared_symbol(L):
    names = b.header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert L.dsa_abi_version() == 4


def test_status_strings(L):
    for code, name in b.STATUS.items():
        assert L.dsa_status_string(code).decode() == name


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _shape(**kw):
    base = dict(B=1, T=4, s_cap=16, H=4, D=32, Hk=4, topk=8, Hm=8, Dc=64, Dr=16)
    base.update(kw)
    return b.Shape(base["B"], base["T"], base["s_cap"], base["H"], base["D"], base["Hk"], base["topk"],
                   base["Hm"], base["Dc"], base["Dr"], None, None)


def _idx(L, shape, dt=b.BF16, q=FAKE, qs=None, k=FAKE, ks=None, w=FAKE, sc=FAKE, ld=None):
    return L.dsa_indexer_scores(C.byref(shape), dt, q, qs, k, ks, w, sc, shape.s_cap if ld is None else ld, None)


@pytest.mark.parametrize("kw,dt,expect", [
    (dict(Hk=2), b.BF16, 1),
    (dict(D=24), b.BF16, 2),
    (dict(D=512), b.BF16, 2),
    (dict(H=200, Hk=200), b.BF16, 2),
    (dict(B=-1), b.BF16, 1),
    (dict(), 7, 1),
])
def test_indexer_shape_errors(L, kw, dt, expect):
    assert _idx(L, _shape(**kw), dt=dt) == expect
    assert L.dsa_last_error().decode()


def test_indexer_pointer_errors(L):
    s = _shape()
    assert _idx(L, s, q=None) == 1
    assert _idx(L, s, dt=b.FP8_E4M3) == 1            # fp8 without scales
    assert _idx(L, s, ld=15) == 1                     # ld < s_cap
    assert _idx(L, s, sc=None) == 1
    assert _idx(L, _shape(B=0), q=None, k=None, w=None, sc=None) == 0   # empty problem: nothing to do


def test_topk_errors(L):
    s = _shape(topk=0)
    assert L.dsa_topk_select(C.byref(s), FAKE, 16, FAKE, None, 0, None) == 1
    s = _shape()
    assert L.dsa_topk_select(C.byref(s), FAKE, 8, FAKE, None, 0, None) == 1
    assert L.dsa_topk_select(C.byref(s), FAKE, 16, None, None, 0, None) == 1
    assert L.dsa_topk_select(None, FAKE, 16, FAKE, None, 0, None) == 1


def test_sparse_mla_errors(L):
    s = _shape()
    f = L.dsa_sparse_mla_attention
    assert f(C.byref(s), b.FP8_E4M3, FAKE, FAKE, FAKE, 1.0, FAKE, None, None, 0, None) == 2
    assert f(C.byref(_shape(Dc=60)), b.BF16, FAKE, FAKE, FAKE, 1.0, FAKE, None, None, 0, None) == 2
    assert f(C.byref(_shape(Dc=1024, Dr=64)), b.BF16, FAKE, FAKE, FAKE, 1.0, FAKE, None, None, 0, None) == 2
    assert f(C.byref(s), b.BF16, None, FAKE, FAKE, 1.0, FAKE, None, None, 0, None) == 1
    assert f(C.byref(s), b.BF16, FAKE, FAKE, None, 1.0, FAKE, None, None, 0, None) == 1
    # decode-sized bf16 problem needs a split workspace
    d = _shape(B=2, T=1, s_cap=4096, topk=2048, Hm=64, Dc=512, Dr=64)
    need = L.dsa_workspace_bytes(C.byref(d), b.OP_SPARSE_MLA)
    assert need > 0
    assert f(C.byref(d), b.BF16, FAKE, FAKE, FAKE, 1.0, FAKE, None, FAKE, need - 1, None) == 5


def _group(L, shape, types, layers, cache, tag=0, ws=FAKE, ws_bytes=None, stats=None):
    n = len(types)
    tarr = (C.c_int * n)(*types)
    arr = (b.LayerIO * n)(*layers)
    if ws_bytes is None:
        ws_bytes = L.dsa_workspace_bytes(C.byref(shape), b.OP_GROUP)
    return L.dsa_group_forward(C.byref(shape), b.BF16, n, tarr, arr, 0.1, C.byref(cache), tag, ws, ws_bytes,
                               None, None if stats is None else C.byref(stats), None)


def _io(with_index):
    io = b.IndexIO(b.BF16, FAKE, None, FAKE, None, FAKE)
    keep = [io]
    return b.LayerIO(C.pointer(io) if with_index else None, FAKE, FAKE, FAKE, None), keep


def test_group_no_donor_and_stale_cache(L):
    s = _shape()
    sh, k1 = _io(False)
    cache = b.TopkCache(FAKE, 0, 0, 0, 0, -1, 0)
    assert _group(L, s, [b.SHARED, b.SHARED], [sh, sh], cache) == 3                 # NO_DONOR
    assert "SHARED" in L.dsa_last_error().decode()
    cache = b.TopkCache(FAKE, 1, 4, 8, 1, 0, 5)
    assert _group(L, s, [b.SHARED], [sh], cache, tag=6) == 4                        # tag mismatch
    cache = b.TopkCache(FAKE, 1, 3, 8, 1, 0, 6)
    assert _group(L, s, [b.SHARED], [sh], cache, tag=6) == 4                        # T mismatch
    cache = b.TopkCache(FAKE, 1, 4, 16, 1, 0, 6)
    assert _group(L, s, [b.SHARED], [sh], cache, tag=6) == 4                        # topk mismatch


def test_group_argument_errors(L):
    s = _shape()
    sh, k1 = _io(False)
    fu, k2 = _io(True)
    cache = b.TopkCache(FAKE, 0, 0, 0, 0, -1, 0)
    assert _group(L, s, [b.FULL, b.SHARED], [sh, sh], cache) == 1                   # full layer without index
    assert _group(L, s, [b.FULL, 9], [fu, sh], cache) == 1                          # bad type
    assert _group(L, s, [b.FULL], [fu], cache, ws_bytes=16) == 5                    # workspace too small
    nocache = b.TopkCache(None, 0, 0, 0, 0, -1, 0)
    assert _group(L, s, [b.FULL], [fu], nocache) == 1
    assert L.dsa_group_forward(C.byref(s), b.BF16, 1, None, None, 0.1, C.byref(cache), 0, FAKE, 1 << 20,
                               None, None, None) == 1
    # nothing was enqueued and the handle was not touched
    assert cache.valid == 0 and cache.donor_layer == -1


def test_sparse_mla_rejects_bad_softmax_scale(L):
    d = _shape(B=1, T=1, s_cap=64, topk=64, Hm=64, Dc=512, Dr=64)
    f = L.dsa_sparse_mla_attention
    for bad in (0.0, -0.5, float("inf"), float("nan")):
        assert f(C.byref(d), b.BF16, FAKE, FAKE, FAKE, bad, FAKE, None, None, 0, None) == 1
        assert "sm_scale" in b.last_error()


def test_topk_workspace_only_for_few_long_rows(L):
    # few rows over a long prefix are chunked over workgroups and need histogram space
    long_rows = _shape(B=4, T=1, s_cap=1 << 20, topk=2048)
    need = L.dsa_workspace_bytes(C.byref(long_rows), b.OP_TOPK)
    assert need >= 4 * 3 * 2048 * 4
    assert L.dsa_topk_select(C.byref(long_rows), FAKE, 1 << 20, FAKE, None, 0, None) == 5
    assert L.dsa_topk_select(C.byref(long_rows), FAKE, 1 << 20, FAKE, FAKE, need - 1, None) == 5
    # many rows, or short rows, take one workgroup per row and no workspace
    assert L.dsa_workspace_bytes(C.byref(_shape(B=1, T=4096, s_cap=4096, topk=2048)), b.OP_TOPK) == 0
    assert L.dsa_workspace_bytes(C.byref(_shape(B=1, T=512, s_cap=1 << 17, topk=2048)), b.OP_TOPK) == 0


def _itk(L, shape, dt=b.BF16, out=FAKE, stride=0, ws=FAKE, ws_bytes=1 << 40, qs=None, ks=None):
    return L.dsa_indexer_topk(C.byref(shape), dt, FAKE, qs, FAKE, ks, FAKE, out, stride, ws, ws_bytes, None)


def test_indexer_topk_errors(L):
    assert _itk(L, _shape(topk=0)) == 1
    assert _itk(L, _shape(D=24)) == 2
    assert _itk(L, _shape(), dt=b.FP8_E4M3) == 1            # fp8 without scales
    assert _itk(L, _shape(), out=None) == 1
    for bad in (-1, 1, 15, (1 << 20) + 1):
        assert _itk(L, _shape(), stride=bad) == 1
        assert "sample_stride" in b.last_error()
    s = _shape()
    need = L.dsa_workspace_bytes(C.byref(s), b.OP_INDEXER_TOPK)
    assert need > 0
    assert _itk(L, s, ws_bytes=need - 1) == 5
    assert _itk(L, s, ws=None, ws_bytes=need) == 5
    assert L.dsa_indexer_topk(C.byref(_shape(B=0)), b.BF16, None, None, None, None, None, None, 0, None, 0, None) == 0


def test_indexer_topk_workspace_layout(L):
    # a 4096-query chunk over a 131072-key prefix (fp8 and one key head per query head can fuse):
    # score buffer for fall-back rows, no top-k histograms (many rows), samples sized for
    # stride 16, four per-row words, 12288 candidate positions and values per row, then the
    # head-major key scales [32][S] and row weights [32][rows] of the fp8 tile kernel
    rows, S = 4096, 131072
    s = _shape(B=1, T=rows, s_cap=S, H=32, D=128, Hk=32, topk=2048, Hm=64, Dc=512, Dr=64)
    want = rows * S * 4 + rows * (S // 16) * 4 + 4 * rows * 4 + 2 * rows * 12288 * 4 + 32 * S * 4 + 32 * rows * 4
    assert L.dsa_workspace_bytes(C.byref(s), b.OP_INDEXER_TOPK) == want
    # a group over rows this long runs the fused call in the same workspace
    assert L.dsa_workspace_bytes(C.byref(s), b.OP_GROUP) >= want
    # D = 64 has no sampling kernel: the unfused pair (scores + top-k workspace) only
    s64 = _shape(B=1, T=rows, s_cap=S, H=32, D=64, Hk=32, topk=2048)
    assert L.dsa_workspace_bytes(C.byref(s64), b.OP_INDEXER_TOPK) == rows * S * 4
    # shorter prefixes do not fuse inside a group: its workspace is the unfused one
    sh = _shape(B=1, T=4096, s_cap=4096, H=32, D=128, Hk=32, topk=2048, Hm=64, Dc=512, Dr=64)
    assert L.dsa_workspace_bytes(C.byref(sh), b.OP_GROUP) < L.dsa_workspace_bytes(C.byref(sh), b.OP_INDEXER_TOPK)


def test_group_stats_count_the_fused_full_layers(L):
    # prefill chunks over >= 65536 keys on the fp8 tile kernel run fused; bf16 prefill, short
    # prefixes and decode rows do not
    types = (C.c_int * 4)(b.FULL, b.SHARED, b.FULL, b.SHARED)
    chunk = _shape(B=1, T=4096, s_cap=131072, H=32, D=128, Hk=32, topk=2048, Hm=64, Dc=512, Dr=64)
    for shape, dt, want in [(chunk, b.FP8_E4M3, 2), (chunk, b.BF16, 0),
                            (_shape(B=1, T=4096, s_cap=4096, H=32, D=128, Hk=32, topk=2048), b.FP8_E4M3, 0),
                            (_shape(B=4, T=1, s_cap=1 << 20, H=32, D=128, Hk=32, topk=2048), b.FP8_E4M3, 0)]:
        st = b.GroupStats()
        assert L.dsa_group_stats_compute(C.byref(shape), dt, b.BF16, 4, types, None, None, C.byref(st)) == 0
        assert (st.n_full, st.n_fused) == (2, want)


def test_workspace_sizes(L):
    s = _shape(B=1, T=4096, s_cap=4096, topk=2048, Hm=64, Dc=512, Dr=64)
    assert L.dsa_workspace_bytes(C.byref(s), b.OP_GROUP) >= 4096 * 4096 * 4
    assert L.dsa_workspace_bytes(C.byref(s), b.OP_INDEXER) == 0
    assert L.dsa_workspace_bytes(None, b.OP_GROUP) == 0


@pytest.mark.parametrize("types", [["full", "shared", "shared", "shared"],
                                   ["full", "full", "full", "shared", "shared", "shared", "full", "shared"],
                                   ["full"] * 4])
@pytest.mark.parametrize("idx_dt,mla_dt", [("bf16", "bf16"), ("fp8", "bf16"), ("f32", "f32")])
def test_group_stats_match_oracle_counts(types, idx_dt, mla_dt):
    rng = np.random.default_rng(5)
    B, T, S = 3, 50, 300
    ke = rng.integers(1, S + 1, (B, T)).astype(np.int32)
    ks = np.minimum(rng.integers(0, 40, (B, T)), ke - 1).astype(np.int32)
    shape = b.Shape(B, T, S, 32, 128, 32, 64, 64, 512, 64, None, None)
    code = {"f32": b.F32, "bf16": b.BF16, "fp8": b.FP8_E4M3}
    st = b.group_stats_compute(shape, code[idx_dt], code[mla_dt], types, ks, ke)
    e = {"f32": 4, "bf16": 2, "fp8": 1}
    ref = O.group_stats(types, ks, ke, H=32, D=128, Hk=32, idx_bytes=e[idx_dt], idx_scaled=idx_dt == "fp8",
                        topk_k=64, Hm=64, Dc=512, Dr=64, mla_bytes=e[mla_dt], S=S)
    assert (st.n_full, st.n_shared) == (ref["n_full"], ref["n_shared"])
    for key in ("indexer_flops", "indexer_bytes", "topk_bytes", "attn_flops", "attn_bytes"):
        assert getattr(st, key) == pytest.approx(ref[key], rel=1e-12), key


def test_index_prep_and_latent_append_validation(L):
    f = L.dsa_index_prep
    ok = dict(n=2, heads=4, D=128, theta=8e6, dt=b.FP8_E4M3, x=FAKE, pos=FAKE, rows=None, n_rows=2, out=FAKE,
              scale=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["n"], a["heads"], a["D"], a["theta"], a["dt"], a["x"], a["pos"], a["rows"], a["n_rows"],
                 a["out"], a["scale"], None)

    assert call(D=130) == 1 and call(D=0) == 1 and call(D=2048) == 1
    assert call(theta=0.0) == 1 and call(theta=float("nan")) == 1
    assert call(dt=b.F32) == 1
    assert call(scale=None) == 1                        # fp8 needs scales
    assert call(x=None) == 1 and call(pos=None) == 1 and call(out=None) == 1
    assert call(n_rows=1) == 1                          # rows NULL: n_rows >= n
    assert call(heads=0) == 1 and call(n=-1) == 1
    assert call(n=0, x=None, pos=None, out=None, scale=None) == 0     # nothing to do
    g = L.dsa_latent_append
    assert g(2, 0, b.BF16, FAKE, FAKE, 10, FAKE, None) == 1
    assert g(2, 4, b.BF16, FAKE, FAKE, 10, FAKE, None) == 2          # 8-byte rows
    assert g(2, 576, b.FP8_E4M3, FAKE, FAKE, 10, FAKE, None) == 1
    assert g(2, 576, b.BF16, None, FAKE, 10, FAKE, None) == 1
    assert g(0, 576, b.BF16, None, None, 0, None, None) == 0


def test_backward_validation(L):
    shape = _shape(topk=8)
    # sparse MLA backward: bad scale, unsupported head count, NULL pointers
    f = L.dsa_sparse_mla_backward
    args = lambda sh, sc=0.1, dq=FAKE, ws=None, nws=0: f(C.byref(sh), b.BF16, FAKE, FAKE, FAKE, sc, FAKE, FAKE, FAKE,
                                                         dq, FAKE, ws, nws, None)
    assert args(shape, sc=0.0) == 1
    assert args(shape, dq=None) == 1
    assert args(_shape(topk=8, Hm=96)) == 2             # more than 64 heads, not in groups of 64
    # the matrix-core shape (bf16, 512 + 64, heads in groups of 64) needs its workspace: D per
    # (query, head), then P, dz' and dz' transposed per (query, slot rounded up to 64, head)
    mma = _shape(B=2, T=3, topk=100, Hm=128, Dc=512, Dr=64, s_cap=1000)
    need = L.dsa_workspace_bytes(C.byref(mma), b.OP_SPARSE_MLA_BWD)
    assert need == 6 * 128 * 4 + 3 * (6 * 128 * 128 * 2)   # both multiples of 256; slots 100 -> 128
    assert args(mma) == 5
    assert args(mma, ws=FAKE, nws=need - 1) == 5
    assert L.dsa_workspace_bytes(C.byref(_shape(topk=8)), b.OP_SPARSE_MLA_BWD) == 0   # vector kernel
    # dense selections (8 topk >= s_cap): D and dz' as before, then a multiplicity per (query,
    # latent row) (rows of s_cap rounded up to 64) and a byte per (query, 64-row tile)
    dn = _shape(B=2, T=3, topk=100, Hm=128, Dc=512, Dr=64, s_cap=700)
    assert L.dsa_workspace_bytes(C.byref(dn), b.OP_SPARSE_MLA_BWD) == \
        6 * 128 * 4 + 6 * 128 * 128 * 2 + 6 * 704 * 4 + 256
    # index backward: unsupported heads, NULL pointers, fp8 without scales
    g = L.dsa_index_backward
    call = lambda sh, dt=b.BF16, qs=None, dI=FAKE, ws=None, nws=0: g(C.byref(sh), dt, FAKE, qs, FAKE, FAKE, FAKE,
                                                                     FAKE, dI, FAKE, FAKE, FAKE, ws, nws, None)
    assert call(shape, dI=None) == 1
    assert call(shape, dt=b.FP8_E4M3) == 1
    assert call(_shape(topk=8, H=128, Hk=128)) == 2
    # dense selections (D = 128, 8 topk >= s_cap): the workspace holds dI as a [row][key] fp32
    # matrix with rows of s_cap rounded up to 64 keys, then a byte per 64 x 64 block
    dense = _shape(B=2, T=3, topk=100, H=8, D=128, Hk=8, s_cap=700)
    need = L.dsa_workspace_bytes(C.byref(dense), b.OP_INDEX_BWD)
    assert need == (6 * 704 * 4 + 255) // 256 * 256 + 256      # 2 x 1 x 11 = 22 occupancy bytes
    assert call(dense) == 5
    assert call(dense, ws=FAKE, nws=need - 1) == 5
    assert L.dsa_workspace_bytes(C.byref(_shape(B=2, T=3, topk=100, H=8, D=128, Hk=8, s_cap=801)),
                                 b.OP_INDEX_BWD) == 0         # 8 x 100 < 801: the sparse kernel
    assert L.dsa_workspace_bytes(C.byref(_shape(B=2, T=3, topk=100, H=8, D=64, Hk=8, s_cap=700)),
                                 b.OP_INDEX_BWD) == 0         # D != 128: the sparse kernel


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_group_stats_need_host_copies_of_device_ranges(L):
    # a device range without its host copy: the counters cannot be formed, nothing is enqueued
    s = _shape()
    s.key_end = FAKE
    fu, k1 = _io(True)
    cache = b.TopkCache(FAKE, 0, 0, 0, 0, -1, 0)
    st = b.GroupStats()
    assert _group(L, s, [b.FULL], [fu], cache, stats=st) == 1
    assert "host copies" in b.last_error()
    assert cache.valid == 0 and st.n_launches == 0


# The next two tests need every kernel launch to fail, which only a host without a GPU
# gives (the library then reports DSA_ERR_HIP at the first launch and nothing runs).
# With a GPU visible the fake pointers would reach real kernels, so they are skipped.
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="relies on launches failing on a host without a GPU")


@no_gpu_only
@pytest.mark.parametrize("ranges", ["none", "host_copies"])
def test_group_forward_fills_every_counter_before_enqueue(L, ranges):
    T, S = 4, 16
    ks_h = np.array([[0, 2, 5, 1]], np.int32)
    ke_h = np.array([[3, 9, 16, 11]], np.int32)
    s = _shape(T=T, s_cap=S)
    if ranges == "host_copies":
        s.key_start, s.key_end = FAKE, FAKE
        s.key_start_host, s.key_end_host = ks_h.ctypes.data, ke_h.ctypes.data
    fu, k1 = _io(True)
    sh, k2 = _io(False)
    types = [b.FULL, b.SHARED, b.SHARED, b.FULL]
    st = b.GroupStats()
    cache = b.TopkCache(FAKE, 0, 0, 0, 0, -1, 0)
    assert _group(L, s, types, [fu, sh, sh, fu], cache, stats=st) == 6       # DSA_ERR_HIP: no device
    ref = b.group_stats_compute(_shape(T=T, s_cap=S), b.BF16, b.BF16, ["full", "shared", "shared", "full"],
                                ks_h if ranges == "host_copies" else None, ke_h if ranges == "host_copies" else None)
    assert (st.n_full, st.n_shared) == (2, 2)
    for key in ("indexer_flops", "indexer_bytes", "topk_bytes", "attn_flops", "attn_bytes"):
        assert getattr(st, key) == getattr(ref, key) and getattr(st, key) > 0, key
    # closed forms on the hand-sized case: sum n over the rows, sum min(n, topk) with topk = 8
    n = (ke_h - ks_h)[0] if ranges == "host_copies" else np.full(T, S)
    assert st.indexer_flops == 2 * 2 * 4 * 32 * n.sum()
    assert st.attn_flops == 4 * 2 * 8 * (2 * 64 + 16) * np.minimum(n, 8).sum()


@no_gpu_only
def test_group_forward_commits_the_cache_handle_only_after_a_whole_enqueue(L):
    fu, k1 = _io(True)
    sh, k2 = _io(False)
    # a fresh handle: the first launch (the indexer) fails -> still empty
    cache = b.TopkCache(FAKE, 0, 0, 0, 0, -1, 0)
    assert _group(L, _shape(), [b.FULL, b.SHARED], [fu, sh], cache, tag=9) == 6
    assert (cache.valid, cache.donor_layer, cache.tag) == (0, -1, 0)
    # a valid handle from an earlier call: a failure before any top-k leaves it as it was
    cache = b.TopkCache(FAKE, 1, 4, 8, 1, 3, 5)
    assert _group(L, _shape(), [b.FULL, b.SHARED], [fu, sh], cache, tag=9) == 6
    assert (cache.valid, cache.donor_layer, cache.tag, cache.B, cache.T, cache.topk) == (1, 3, 5, 1, 4, 8)
    # with an empty key capacity the indexer has nothing to do and the top-k launch is the
    # first to fail: the indices buffer may hold partial data, so the handle is invalidated
    cache = b.TopkCache(FAKE, 1, 4, 8, 1, 3, 5)
    assert _group(L, _shape(s_cap=0), [b.FULL, b.SHARED], [fu, sh], cache, tag=9) == 6
    assert cache.valid == 0 and cache.tag == 5


def test_noalloc_group_rejects_calls_beyond_its_scratch_before_anything(L):
    # the allocation-free group call holds DSA_NOALLOC_SCRATCH_BYTES of device scratch; a
    # larger need is refused on the host, before any device is touched
    big = _shape(B=1, T=4096, s_cap=8192, topk=2048, Hm=64, Dc=512, Dr=64)
    assert L.dsa_workspace_bytes(C.byref(big), b.OP_GROUP) > b.noalloc_scratch_bytes()
    fu, k1 = _io(True)
    arr = (b.LayerIO * 1)(fu)
    types = (C.c_int * 1)(b.FULL)
    cache = b.TopkCache(FAKE, 0, 0, 0, 0, -1, 0)
    assert L.dsa_group_forward_noalloc(C.byref(big), b.BF16, 1, types, arr, 0.1, C.byref(cache), 0, None, None,
                                       None) == 5
    assert "allocation-free" in b.last_error()
    assert cache.valid == 0
    assert b.noalloc_scratch_bytes() == 64 << 20
