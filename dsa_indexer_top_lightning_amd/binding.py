"""ctypes binding of libdsa.so (include/dsa.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module turns
torch tensors into pointers and sizes, passes the current HIP stream and raises
on a non-OK status.  It never computes results itself and has no fallback: if
the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dsa.h")

F32, BF16, FP8_E4M3 = 0, 1, 2
FULL, SHARED = 0, 1
OP_INDEXER, OP_TOPK, OP_SPARSE_MLA, OP_GROUP, OP_INDEXER_TOPK, OP_SPARSE_MLA_BWD, OP_INDEX_BWD = 0, 1, 2, 3, 4, 5, 6
STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_NO_DONOR",
          4: "DSA_ERR_STALE_CACHE", 5: "DSA_ERR_WORKSPACE_TOO_SMALL", 6: "DSA_ERR_HIP"}


class Shape(C.Structure):
    _fields_ = [("B", C.c_int32), ("T", C.c_int32), ("s_cap", C.c_int64),
                ("H", C.c_int32), ("D", C.c_int32), ("Hk", C.c_int32), ("topk", C.c_int32),
                ("Hm", C.c_int32), ("Dc", C.c_int32), ("Dr", C.c_int32),
                ("key_start", C.c_void_p), ("key_end", C.c_void_p),
                ("key_start_host", C.c_void_p), ("key_end_host", C.c_void_p)]


class TopkCache(C.Structure):
    _fields_ = [("indices", C.c_void_p), ("B", C.c_int32), ("T", C.c_int32), ("topk", C.c_int32),
                ("valid", C.c_int32), ("donor_layer", C.c_int32), ("tag", C.c_uint64)]


class IndexIO(C.Structure):
    _fields_ = [("idx_dtype", C.c_int), ("q", C.c_void_p), ("q_scale", C.c_void_p), ("k", C.c_void_p),
                ("k_scale", C.c_void_p), ("w", C.c_void_p)]


class LayerIO(C.Structure):
    _fields_ = [("index", C.POINTER(IndexIO)), ("q", C.c_void_p), ("kv", C.c_void_p), ("out", C.c_void_p),
                ("lse", C.c_void_p)]


class GroupStats(C.Structure):
    _fields_ = [("n_full", C.c_int32), ("n_shared", C.c_int32), ("n_launches", C.c_int32), ("n_fused", C.c_int32),
                ("indexer_flops", C.c_double), ("indexer_bytes", C.c_double), ("topk_bytes", C.c_double),
                ("attn_flops", C.c_double), ("attn_bytes", C.c_double)]


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None

_SIGS = {
    "dsa_indexer_scores": (C.c_int, [C.POINTER(Shape), C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]),
    "dsa_topk_select": (C.c_int, [C.POINTER(Shape), C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_size_t,
                                  C.c_void_p]),
    "dsa_indexer_topk": (C.c_int, [C.POINTER(Shape), C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]),
    "dsa_sparse_mla_attention": (C.c_int, [C.POINTER(Shape), C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_float, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                           C.c_void_p]),
    "dsa_group_forward": (C.c_int, [C.POINTER(Shape), C.c_int, C.c_int32, C.c_void_p, C.POINTER(LayerIO),
                                    C.c_float, C.POINTER(TopkCache), C.c_uint64, C.c_void_p, C.c_size_t,
                                    C.c_void_p, C.POINTER(GroupStats), C.c_void_p]),
    "dsa_group_forward_noalloc": (C.c_int, [C.POINTER(Shape), C.c_int, C.c_int32, C.c_void_p, C.POINTER(LayerIO),
                                            C.c_float, C.POINTER(TopkCache), C.c_uint64, C.c_void_p,
                                            C.POINTER(GroupStats), C.c_void_p]),
    "dsa_group_stats_compute": (C.c_int, [C.POINTER(Shape), C.c_int, C.c_int, C.c_int32, C.c_void_p, C.c_void_p,
                                          C.c_void_p, C.POINTER(GroupStats)]),
    "dsa_index_backward": (C.c_int, [C.POINTER(Shape), C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_size_t, C.c_void_p]),
    "dsa_sparse_mla_backward": (C.c_int, [C.POINTER(Shape), C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_float,
                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                          C.c_size_t, C.c_void_p]),
    "dsa_index_prep": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_float, C.c_int, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dsa_latent_append": (C.c_int, [C.c_int32, C.c_int32, C.c_int, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p,
                                    C.c_void_p]),
    "dsa_workspace_bytes": (C.c_size_t, [C.POINTER(Shape), C.c_int]),
    "dsa_status_string": (C.c_char_p, [C.c_int]),
    "dsa_last_error": (C.c_char_p, []),
    "dsa_abi_version": (C.c_int, []),
}


def header_functions() -> list[str]:
    """Names of the functions include/dsa.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(dsa_\w+)\s*\(", text, re.M)))


def lib():
    """The loaded library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().dsa_last_error().decode()


def _check(status: int):
    if status != 0:
        raise DsaError(status, last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _dev_ptr(t) -> int | None:
    if t is not None and t.device.type != "cuda":
        raise ValueError("tensors passed to the library must live on the GPU")
    return _ptr(t)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _host_i32(a):
    if a is None:
        return None
    import numpy as np
    return np.ascontiguousarray(a, dtype=np.int32)


def make_shape(B, T, s_cap, *, H=0, D=0, Hk=0, topk=0, Hm=0, Dc=0, Dr=0, key_start=None, key_end=None,
               key_start_host=None, key_end_host=None) -> Shape:
    """dsa_shape.  key_start / key_end are device int32 tensors [B,T] (or None); their host copies
    (numpy, optional) let dsa_group_forward fill the analytic counters."""
    ksh, keh = _host_i32(key_start_host), _host_i32(key_end_host)
    shape = Shape(B, T, s_cap, H, D, Hk, topk, Hm, Dc, Dr, _dev_ptr(key_start), _dev_ptr(key_end),
                  None if ksh is None else ksh.ctypes.data, None if keh is None else keh.ctypes.data)
    shape._keep = (key_start, key_end, ksh, keh)  # the struct holds raw pointers: keep their arrays alive
    return shape


def workspace_bytes(shape: Shape, op: int) -> int:
    return int(lib().dsa_workspace_bytes(C.byref(shape), op))


# ---------------------------------------------------------------- entry points

def indexer_scores(q, k, w, scores, *, q_scale=None, k_scale=None, key_start=None, key_end=None, stream=None):
    """dsa_indexer_scores.  q [B,T,H,D], k [B,S,Hk,D], w [B,T,H], scores [B,T,ld] fp32 (written in place)."""
    B, T, H, D = q.shape
    S, Hk = k.shape[1], k.shape[2]
    shape = make_shape(B, T, S, H=H, D=D, Hk=Hk, key_start=key_start, key_end=key_end)
    _check(lib().dsa_indexer_scores(C.byref(shape), dtype_code(q), _dev_ptr(q), _dev_ptr(q_scale), _dev_ptr(k),
                                    _dev_ptr(k_scale), _dev_ptr(w), _dev_ptr(scores), scores.shape[-1],
                                    _stream(stream)))
    return scores


def topk_select(scores, out, s_cap, *, key_start=None, key_end=None, workspace=None, stream=None):
    """dsa_topk_select.  scores [B,T,ld] fp32, out [B,T,topk] int32 (written in place)."""
    B, T, K = out.shape
    shape = make_shape(B, T, s_cap, topk=K, key_start=key_start, key_end=key_end)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_topk_select(C.byref(shape), _dev_ptr(scores), scores.shape[-1], _dev_ptr(out),
                                 _dev_ptr(workspace), ws_bytes, _stream(stream)))
    return out


def indexer_topk(q, k, w, out, *, q_scale=None, k_scale=None, key_start=None, key_end=None, sample_stride=0,
                 workspace=None, stream=None):
    """dsa_indexer_topk.  q [B,T,H,D], k [B,S,Hk,D], w [B,T,H], out [B,T,topk] int32 (written in place);
    workspace: uint8 tensor of at least workspace_bytes(shape, OP_INDEXER_TOPK) bytes."""
    B, T, H, D = q.shape
    S, Hk = k.shape[1], k.shape[2]
    shape = make_shape(B, T, S, H=H, D=D, Hk=Hk, topk=out.shape[-1], key_start=key_start, key_end=key_end)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_indexer_topk(C.byref(shape), dtype_code(q), _dev_ptr(q), _dev_ptr(q_scale), _dev_ptr(k),
                                  _dev_ptr(k_scale), _dev_ptr(w), _dev_ptr(out), int(sample_stride),
                                  _dev_ptr(workspace), ws_bytes, _stream(stream)))
    return out


def sparse_mla_attention(q, kv, topk_indices, sm_scale, out, lse=None, *, Dc, workspace=None, stream=None):
    """dsa_sparse_mla_attention.  q [B,T,Hm,Dc+Dr], kv [B,S,Dc+Dr], topk_indices [B,T,k], out [B,T,Hm,Dc]."""
    B, T, Hm, R = q.shape
    S = kv.shape[1]
    shape = make_shape(B, T, S, topk=topk_indices.shape[-1], Hm=Hm, Dc=Dc, Dr=R - Dc)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_sparse_mla_attention(C.byref(shape), dtype_code(q), _dev_ptr(q), _dev_ptr(kv),
                                          _dev_ptr(topk_indices), float(sm_scale), _dev_ptr(out), _dev_ptr(lse),
                                          _dev_ptr(workspace), ws_bytes, _stream(stream)))
    return out


def index_backward(q, k, w, topk_indices, dI, dq, dk, dw, *, q_scale=None, k_scale=None, workspace=None,
                   stream=None):
    """dsa_index_backward.  Index inputs as for indexer_scores, topk_indices and dI [B,T,topk];
    dq [B,T,H,D], dk [B,S,Hk,D] and dw [B,T,H] fp32 are written in place; workspace: uint8 tensor
    of at least workspace_bytes(shape, OP_INDEX_BWD) bytes (None when that is 0)."""
    B, T, H, D = q.shape
    S, Hk = k.shape[1], k.shape[2]
    shape = make_shape(B, T, S, H=H, D=D, Hk=Hk, topk=topk_indices.shape[-1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_index_backward(C.byref(shape), dtype_code(q), _dev_ptr(q), _dev_ptr(q_scale), _dev_ptr(k),
                                    _dev_ptr(k_scale), _dev_ptr(w), _dev_ptr(topk_indices), _dev_ptr(dI),
                                    _dev_ptr(dq), _dev_ptr(dk), _dev_ptr(dw), _dev_ptr(workspace), ws_bytes,
                                    _stream(stream)))
    return dq, dk, dw


def sparse_mla_backward(q, kv, topk_indices, sm_scale, out, lse, dout, dq, dkv, *, Dc, workspace=None, stream=None):
    """dsa_sparse_mla_backward.  Forward inputs and results (out, lse), dout [B,T,Hm,Dc];
    dq [B,T,Hm,Dc+Dr] and dkv [B,S,Dc+Dr] fp32 are written in place; workspace: uint8 tensor
    of at least workspace_bytes(shape, OP_SPARSE_MLA_BWD) bytes (None when that is 0)."""
    B, T, Hm, R = q.shape
    S = kv.shape[1]
    shape = make_shape(B, T, S, topk=topk_indices.shape[-1], Hm=Hm, Dc=Dc, Dr=R - Dc)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_sparse_mla_backward(C.byref(shape), dtype_code(q), _dev_ptr(q), _dev_ptr(kv),
                                         _dev_ptr(topk_indices), float(sm_scale), _dev_ptr(out), _dev_ptr(lse),
                                         _dev_ptr(dout), _dev_ptr(dq), _dev_ptr(dkv), _dev_ptr(workspace), ws_bytes,
                                         _stream(stream)))
    return dq, dkv


def index_prep(x, pos, out, out_scale=None, *, rows=None, rope_theta=8.0e6, stream=None):
    """dsa_index_prep.  x [n, heads, D] fp32, pos [n] int32, out [n_rows, heads, D] (bf16 bits as
    uint16/bfloat16, or e4m3fn codes as uint8/float8_e4m3fn), out_scale [n_rows, heads] fp32 (fp8)."""
    n, heads, D = x.shape
    if out.dtype in (torch.uint8, torch.float8_e4m3fn):
        dt = FP8_E4M3
    elif out.dtype in (torch.uint16, torch.int16, torch.bfloat16):
        dt = BF16
    else:
        raise ValueError(f"unsupported out dtype {out.dtype}")
    _check(lib().dsa_index_prep(n, heads, D, float(rope_theta), dt, _dev_ptr(x), _dev_ptr(pos), _dev_ptr(rows),
                                out.shape[0], _dev_ptr(out), _dev_ptr(out_scale), _stream(stream)))
    return out


def latent_append(latent_new, rows, latent_cache, *, stream=None):
    """dsa_latent_append.  latent_new [n, R] and latent_cache [n_rows, R], float32 or bf16."""
    n, R = latent_new.shape
    _check(lib().dsa_latent_append(n, R, dtype_code(latent_new), _dev_ptr(latent_new), _dev_ptr(rows),
                                   latent_cache.shape[0], _dev_ptr(latent_cache), _stream(stream)))
    return latent_cache


class IndexCache:
    """Caller-owned cached top-k indices (dsa_topk_cache) with its device buffer."""

    def __init__(self, B, T, topk, device="cuda"):
        self.indices = torch.full((B, T, topk), -1, dtype=torch.int32, device=device)
        self.c = TopkCache(self.indices.data_ptr(), 0, 0, 0, 0, -1, 0)

    @property
    def valid(self):
        return bool(self.c.valid)


def group_forward(shape: Shape, mla_dtype: int, indexer_types, layers, sm_scale, cache: IndexCache, tag: int,
                  workspace, *, events=None, stream=None, _noalloc=False):
    """dsa_group_forward.  ``layers`` is a list of dicts with keys q, kv, out, lse and, on full
    layers, index = dict(q, k, w, q_scale, k_scale).  Returns GroupStats, or None when the shape
    has device key ranges without host copies (the counters cannot be formed then)."""
    n = len(indexer_types)
    types = (C.c_int * n)(*[FULL if t in ("full", FULL) else SHARED for t in indexer_types])
    idx_ios = []
    arr = (LayerIO * n)()
    for l, L in enumerate(layers):
        io = None
        if L.get("index") is not None:
            I = L["index"]
            io = IndexIO(dtype_code(I["q"]), _dev_ptr(I["q"]), _dev_ptr(I.get("q_scale")), _dev_ptr(I["k"]),
                         _dev_ptr(I.get("k_scale")), _dev_ptr(I["w"]))
            idx_ios.append(io)
        arr[l] = LayerIO(C.pointer(io) if io is not None else None, _dev_ptr(L["q"]), _dev_ptr(L["kv"]),
                         _dev_ptr(L["out"]), _dev_ptr(L.get("lse")))
    ev = None
    if events is not None:
        ev = (C.c_void_p * len(events))(*events)
    want = (not shape.key_start or shape.key_start_host) and (not shape.key_end or shape.key_end_host)
    stats = GroupStats() if want else None
    st = C.byref(stats) if want else None
    if _noalloc:
        _check(lib().dsa_group_forward_noalloc(C.byref(shape), mla_dtype, n, types, arr, float(sm_scale),
                                               C.byref(cache.c), tag, ev, st, _stream(stream)))
        return stats
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_group_forward(C.byref(shape), mla_dtype, n, types, arr, float(sm_scale), C.byref(cache.c),
                                   tag, _dev_ptr(workspace), ws_bytes, ev, st, _stream(stream)))
    return stats


def noalloc_scratch_bytes() -> int:
    """DSA_NOALLOC_SCRATCH_BYTES as the header defines it."""
    with open(HEADER) as f:
        m = re.search(r"#define\s+DSA_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", f.read())
    return int(m.group(1)) << int(m.group(2))


def group_forward_noalloc(shape: Shape, mla_dtype: int, indexer_types, layers, sm_scale, cache: IndexCache,
                          tag: int, *, events=None, stream=None):
    """dsa_group_forward_noalloc: dsa_group_forward with the library's own device scratch instead of a
    workspace (nothing is allocated).  Arguments and return value as for group_forward."""
    return group_forward(shape, mla_dtype, indexer_types, layers, sm_scale, cache, tag, None, events=events,
                         stream=stream, _noalloc=True)


def group_stats_compute(shape: Shape, idx_dtype: int, mla_dtype: int, indexer_types, key_start_host=None,
                        key_end_host=None) -> GroupStats:
    """dsa_group_stats_compute (pure host).  Key ranges as host int32 arrays (numpy) or None."""
    import numpy as np
    n = len(indexer_types)
    types = (C.c_int * n)(*[FULL if t in ("full", FULL) else SHARED for t in indexer_types])
    ks = None if key_start_host is None else np.ascontiguousarray(key_start_host, dtype=np.int32)
    ke = None if key_end_host is None else np.ascontiguousarray(key_end_host, dtype=np.int32)
    out = GroupStats()
    _check(lib().dsa_group_stats_compute(C.byref(shape), idx_dtype, mla_dtype, n, types,
                                         None if ks is None else ks.ctypes.data,
                                         None if ke is None else ke.ctypes.data, C.byref(out)))
    return out
