"""Throughput of one IndexShare layer group on one MI355X.

A step is one dsa_group_forward over the workload's whole layer list (indexer
scores -> top-k -> sparse MLA on full layers, sparse MLA with the cached indices
on shared layers) for one batch of synthetic queries whose inputs are already
resident in HBM.  Prints one JSON line:
  value          query tokens/s per 4-layer group = B*T / (step time) * n_layers / 4, on the
                 4096-query fp8 chunk over a 131,072-token prefix by default
  roofline       the kernel with the largest share of the step: algorithmic FLOPs (or
                 bytes) per launch / mean launch time (HIP events recorded by the library
                 around each launch on the timed stream) vs the MFMA peak of its input
                 type (or HBM)
  kernels        the same for every kernel family
  cpu_baseline   the CPU oracle on a time-bounded sample of query rows of the same workload
  workloads      the same measurements for the 4096-token prefill and the two decodes
                 (the decodes also as HIP-graph replays of one group call)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-sub]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query tokens/s per 4-layer F/S group (indexer+top-k+sparse MLA); MFMA% & HBM GB/s"
# the headline: the largest single-GPU workload by work per group (4096 queries over a 131,072-token
# prefix, fp8 index keys); the others follow as sub-results
HEADLINE = "chunk128k_fp8"
SUB_WORKLOADS = ["prefill4k_bf16", "decode32k_b64_bf16", "decode1m_b4_fp8"]
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
# HBM bytes per launch of the roofline kernel from two rocprofv3 --pmc runs (FETCH_SIZE, then
# WRITE_SIZE) of `bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-sub --workload <name>`, each
# scaled by the same counter's reading on a plain copy of known size (`bench.py --copy-calibration`);
# keyed (workload, kernel), with the profile summary it comes from, and removed whenever that kernel
# changes (then reported as null).
MEASURED_TRAFFIC = {
    ("chunk128k_fp8", "mla_mfma"): {
        "bytes": 3917845.3 * 1024 * 2.0 + 263168.0 * 1024 * 1.0,
        "source": "profiles/mla_mfma_chunk128k_fp8_hbm_counters.md"},
    ("prefill4k_bf16", "mla_mfma"): {
        "bytes": 314290.2 * 1024 * 2.0 + 263168.0 * 1024 * 1.0,
        "source": "profiles/mla_mfma_prefill4k_bf16_hbm_counters.md"},
    ("decode1m_b4_fp8", "indexer_stream"): {
        "bytes": 8651439.6 * 1024 * 2.0 + 16384.0 * 1024 * 1.0,
        "source": "profiles/indexer_stream_decode1m_b4_fp8_hbm_counters.md"},
    ("decode32k_b64_bf16", "indexer_stream"): {
        "bytes": 8393959.4 * 1024 * 2.0 + 8192.0 * 1024 * 1.0,
        "source": "profiles/indexer_stream_decode32k_b64_bf16_hbm_counters.md"},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="time budget of the CPU oracle baseline (rows evenly spaced over the workload, "
                         "taken in a fixed order until the budget is spent)")
    ap.add_argument("--no-sub", action="store_true",
                    help="time only --workload (by default the other workloads follow as sub-results)")
    ap.add_argument("--graph", action="store_true",
                    help="also time HIP-graph replays of one group call for --workload (the sub-results "
                         "of decode workloads always carry them)")
    ap.add_argument("--backward", action="store_true",
                    help="time layer 0's backward instead of the forward group: the sparse MLA backward (its "
                         "forward's indices, output and lse, a seeded output gradient) and the index-score "
                         "backward at the selected positions (a seeded score gradient)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run the calibration library's copy kernel over BYTES (3 times) and exit: the "
                         "reference kernel whose FETCH_SIZE / WRITE_SIZE counters scale the HBM traffic figures")
    ap.add_argument("--ab-indexer-topk", action="store_true",
                    help="only time layer 0's indexer -> top-k both ways on --workload and exit: "
                         "dsa_indexer_scores + dsa_topk_select, and dsa_indexer_topk (default sample stride), "
                         "with a check that both give the same indices")
    ap.add_argument("--calibrate", action="store_true",
                    help="only measure achievable peaks with the calibration library's own kernels and exit: a "
                         "4 GiB copy, the sparse attention's row gather over the 128K chunk's and the 4K "
                         "prefill's key ranges, and bf16 / fp8 matrix-core loops")
    return ap.parse_args()


def calib_lib():
    import ctypes as C
    L = C.CDLL(os.path.join(ROOT, "dsa_indexer_top_lightning_amd", "libdsa_calib.so"))
    L.calib_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
    L.calib_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
    L.calib_gather.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    L.calib_mfma.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    return L


def _ok(rc):
    if rc != 0:
        raise RuntimeError(f"calibration kernel launch failed (HIP error {rc})")


def copy_calibration(nbytes):
    import torch
    L = calib_lib()
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    for _ in range(3):
        _ok(L.calib_copy(src.data_ptr(), dst.data_ptr(), nbytes // 16, st))
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "copy16", "copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 3}))


def ab_indexer_topk(w, steps, warmup):
    """Layer 0's indexer -> top-k of workload w, unfused and fused, HIP-event timed (mean of `steps`)."""
    import torch

    from dsa_indexer_top_lightning_amd import binding as B
    from dsa_indexer_top_lightning_amd import synth
    L = synth.build_layer_inputs(w, 0, True, with_mla=False)
    dt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[w.idx_dtype]
    q = torch.from_numpy(L["idx_q"].view(np.int16) if w.idx_dtype == "bf16" else L["idx_q"]).cuda().view(dt)
    k = torch.from_numpy(L["idx_k"].view(np.int16) if w.idx_dtype == "bf16" else L["idx_k"]).cuda().view(dt)
    wt = torch.from_numpy(L["w"]).cuda()
    qs = torch.from_numpy(L["idx_q_scale"]).cuda() if "idx_q_scale" in L else None
    ks = torch.from_numpy(L["idx_k_scale"]).cuda() if "idx_k_scale" in L else None
    del L
    ke = torch.from_numpy(w.key_end()).cuda()
    shape = B.make_shape(w.B, w.T, w.S, H=w.H, D=w.D, Hk=w.Hk, topk=w.topk, key_end=ke)
    ws = torch.empty((B.workspace_bytes(shape, B.OP_INDEXER_TOPK),), dtype=torch.uint8, device="cuda")
    scores = ws[:w.B * w.T * w.S * 4].view(torch.float32).view(w.B, w.T, w.S)
    tws = torch.empty((max(1, B.workspace_bytes(shape, B.OP_TOPK)),), dtype=torch.uint8, device="cuda")
    a = torch.empty((w.B, w.T, w.topk), dtype=torch.int32, device="cuda")
    f = torch.empty_like(a)
    ex = dict(q_scale=qs, k_scale=ks, key_end=ke)

    def unfused():
        B.indexer_scores(q, k, wt, scores, **ex)
        B.topk_select(scores, a, w.S, key_end=ke, workspace=tws)

    def fused():
        B.indexer_topk(q, k, wt, f, workspace=ws, **ex)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    t_u, t_f = timed(unfused), timed(fused)
    same = bool(torch.equal(a, f))
    print(json.dumps({"workload": w.name, "unfused_ms": t_u, "fused_ms": t_f, "indices_identical": same,
                      "steps": steps, "warmup": warmup}))


def calibrate():
    """Achievable peaks from the calibration library's kernels (HIP events on the launch stream)."""
    import torch
    L = calib_lib()
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream

    def timed(f, n):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    out = {}
    nbytes = 4 << 30
    src = torch.arange(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: _ok(L.calib_copy(src.data_ptr(), dst.data_ptr(), nbytes // 16, st)), 5)
    assert torch.equal(dst, src), "copy kernel result differs from its source"
    out["copy"] = {"bytes_moved": 2 * nbytes, "ms": ms, "GBps": 2 * nbytes / (ms * 1e-3) / 1e9}
    del dst
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    ms = timed(lambda: _ok(L.calib_read(src.data_ptr(), nbytes // 16, sink.data_ptr(), st)), 5)
    out["read"] = {"bytes_read": nbytes, "ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9}
    del src, sink
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    nq, k, row_bytes = 4096, 2048, 1152
    for name, S in (("chunk128k_rows", 131072), ("prefill4k_rows", 4096)):
        rows = torch.randint(0, 256, (S * row_bytes,), dtype=torch.uint8, device="cuda", generator=g)
        idx = torch.empty((nq, k), dtype=torch.int32, device="cuda")
        for q0 in range(0, nq, 256):   # k distinct random rows per query, ascending
            r = torch.rand((256, S), device="cuda", generator=g).argsort(dim=1)[:, :k]
            idx[q0:q0 + 256] = r.sort(dim=1).values.to(torch.int32)
        sink = torch.zeros(nq, dtype=torch.int32, device="cuda")
        ms = timed(lambda: _ok(L.calib_gather(rows.data_ptr(), idx.data_ptr(), nq, k, row_bytes, sink.data_ptr(),
                                              st)), 10)
        out[f"gather_{name}"] = {"rows": S, "queries": nq, "rows_per_query": k, "row_bytes": row_bytes, "ms": ms,
                                 "TBps": nq * k * row_bytes / (ms * 1e-3) / 1e12}
        del rows, idx
    blocks, iters = 256 * 8, 4000
    res = torch.empty(blocks * 256, device="cuda")
    for fp8, name, flop in ((0, "mfma_bf16_32x32x16", 32 * 32 * 16 * 2), (1, "mfma_fp8_32x32x64", 32 * 32 * 64 * 2)):
        ms = timed(lambda: _ok(L.calib_mfma(fp8, blocks, iters, res.data_ptr(), st)), 5)
        total = blocks * 4 * iters * 4 * flop
        out[name] = {"ms": ms, "TFLOPs": total / (ms * 1e-3) / 1e12}
    print(json.dumps(out))


def upload(w, inputs, torch):
    def dev(a, dt):
        if dt == "f32":
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda().view(torch.float8_e4m3fn)

    out = []
    odt = torch.float32 if w.mla_dtype == "f32" else torch.bfloat16
    for L in inputs:
        d = {"q": dev(L["mla_q"], w.mla_dtype), "kv": dev(L["kv"], w.mla_dtype),
             "out": torch.empty((w.B, w.T, w.Hm, w.Dc), device="cuda", dtype=odt),
             "lse": torch.empty((w.B, w.T, w.Hm), device="cuda")}
        if "idx_q" in L:
            d["index"] = {"q": dev(L["idx_q"], w.idx_dtype), "k": dev(L["idx_k"], w.idx_dtype),
                          "w": dev(L["w"], "f32")}
            if w.idx_dtype == "fp8":
                d["index"]["q_scale"] = dev(L["idx_q_scale"], "f32")
                d["index"]["k_scale"] = dev(L["idx_k_scale"], "f32")
        out.append(d)
    return out


def host_info():
    """CPU model, logical CPUs and the CPUs this process may run on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "affinity": aff, "blas_threads": blas_threads()}


def blas_threads():
    """Threads the oracle's NumPy BLAS runs on."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:
        return 1


def sample_order(n):
    """Row indices 0..n-1 in an order whose every prefix is spread over the whole range
    (bit-reversal order of the next power of two), so a time-bounded sample stays even."""
    m = 1 << max(0, (n - 1).bit_length())
    bits = max(1, m.bit_length() - 1)
    order = [int(format(i, f"0{bits}b")[::-1], 2) for i in range(m)] if m > 1 else [0]
    return [i for i in order if i < n]


def cpu_baseline(w, inputs, seconds, max_rows=None):
    """The oracle, as it stands, on query rows spread over the workload (all layers), taken until
    `seconds` of work are spent (at least two rows)."""
    import oracle as O
    blas = blas_threads()
    types = ["full" if c == "F" else "shared" for c in w.layers]
    ke, ks = w.key_end(), w.key_start()
    picks = [(b, t) for b in range(w.B) for t in range(w.T)]
    order = [picks[i] for i in sample_order(len(picks))]
    if max_rows:
        order = order[:max_rows]
    dec = [{"kv": {}, "k": {}} for _ in inputs]
    done = 0
    phase = {"decode": 0.0, "score": 0.0, "sort": 0.0, "attention": 0.0}
    t0 = time.perf_counter()
    for (b, t) in order:
        idx = None
        for l, L in enumerate(inputs):
            p0 = time.perf_counter()
            if types[l] == "full" and b not in dec[l]["k"]:
                dec[l]["k"][b] = O.decode(L["idx_k"][b], w.idx_dtype,
                                          L["idx_k_scale"][b] if "idx_k_scale" in L else None)
            if b not in dec[l]["kv"]:
                dec[l]["kv"][b] = O.decode(L["kv"][b], w.mla_dtype)
            p1 = time.perf_counter()
            phase["decode"] += p1 - p0
            if types[l] == "full":
                qs = L["idx_q_scale"][b, t] if "idx_q_scale" in L else None
                q = O.decode(L["idx_q"][b, t], w.idx_dtype, qs)
                row = O.index_scores_row(q, dec[l]["k"][b], L["w"][b, t].astype(np.float64),
                                         int(ks[b, t]), int(ke[b, t]))
                p2 = time.perf_counter()
                idx, _ = O.topk_row(row, int(ks[b, t]), int(ke[b, t]), w.topk)
                p3 = time.perf_counter()
                phase["score"] += p2 - p1
                phase["sort"] += p3 - p2
                p1 = p3
            O.sparse_mla_row(O.decode(L["mla_q"][b, t], w.mla_dtype), dec[l]["kv"][b], idx, w.sm_scale, w.Dc)
            phase["attention"] += time.perf_counter() - p1
        done += 1
        if done >= 2 and time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt * w.n_layers / 4.0, "unit": "query tokens/s", "cores": int(blas),
            "kind": "oracle",
            "sample": f"{done} of the {w.B}x{w.T} query rows of {w.name} (spread over the rows in bit-reversed "
                      f"order, taken until {seconds:.0f} s were spent), all {w.n_layers} layers, float64 NumPy, "
                      f"{dt:.1f} s including decoding of the inputs they read",
            "phase_s": {k: round(v, 2) for k, v in phase.items()}, "host": host_info()}


def run_forward(w, dev, steps, warmup, graph, torch, B):
    """Time `steps` group calls of workload w (inputs resident in HBM) after `warmup` untimed ones.
    Per-kernel times come from HIP events the library records around each launch on the timed
    stream.  Returns the measurement dict of the workload."""
    ke_host, ks_host = w.key_end(), w.key_start()
    ke = torch.from_numpy(ke_host).cuda()
    ks = torch.from_numpy(ks_host).cuda() if ks_host.any() else None
    types = ["full" if c == "F" else "shared" for c in w.layers]
    shape = B.make_shape(w.B, w.T, w.S, H=w.H, D=w.D, Hk=w.Hk, topk=w.topk, Hm=w.Hm, Dc=w.Dc, Dr=w.Dr,
                         key_start=ks, key_end=ke, key_start_host=ks_host if ks is not None else None,
                         key_end_host=ke_host)
    ws = torch.empty(max(B.workspace_bytes(shape, B.OP_GROUP), 1), dtype=torch.uint8, device="cuda")
    cache = B.IndexCache(w.B, w.T, w.topk)
    mdt = B.F32 if w.mla_dtype == "f32" else B.BF16
    stream = torch.cuda.current_stream()
    n = len(types)

    def new_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(6 * n)]
        for e in evs:
            e.record(stream)           # creates the HIP event; the library re-records it
        return evs

    stats = None
    for _ in range(warmup):
        stats = B.group_forward(shape, mdt, types, dev, w.sm_scale, cache, 1, ws, stream=stream)
    events = [new_events() for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(steps):
        B.group_forward(shape, mdt, types, dev, w.sm_scale, cache, 1, ws, stream=stream,
                        events=[e.cuda_event for e in events[s]])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    if stats is None:
        idt = {"f32": B.F32, "bf16": B.BF16, "fp8": B.FP8_E4M3}[w.idx_dtype]
        stats = B.group_stats_compute(shape, idt, mdt, types, ks_host, ke_host)

    def mean_ms(slot, layers):
        v = [events[s][6 * l + slot].elapsed_time(events[s][6 * l + slot + 1]) for s in range(steps) for l in layers]
        return float(np.mean(v)) if v else None

    full = [l for l in range(n) if types[l] == "full"]
    nf = max(len(full), 1)
    t_idx, t_topk, t_attn = mean_ms(0, full), mean_ms(2, full), mean_ms(4, range(n))
    idx_flops = stats.indexer_flops / nf
    idx_bytes = stats.indexer_bytes / nf
    topk_bytes = stats.topk_bytes / nf
    attn_flops, attn_bytes = stats.attn_flops / n, stats.attn_bytes / n
    prefill = w.T > 1
    idx_peak = PEAK_FP8_TFLOPS if w.idx_dtype == "fp8" else PEAK_BF16_TFLOPS
    fused = stats.n_fused > 0   # full layers run as the fused indexer -> top-k: one span, no score matrix
    if fused:
        t_topk = None
    kernels = {
        "indexer": {"ms": t_idx, "tflops": idx_flops / (t_idx * 1e-3) / 1e12 if t_idx else None,
                    "gbs": idx_bytes / (t_idx * 1e-3) / 1e9 if t_idx else None,
                    "includes_topk": fused},
        "topk": {"ms": t_topk, "gbs": topk_bytes / (t_topk * 1e-3) / 1e9 if t_topk else None},
        "sparse_mla": {"ms": t_attn, "tflops": attn_flops / (t_attn * 1e-3) / 1e12,
                       # every selected row's bytes per query: mostly served by the caches on a prefill
                       "gather_gbs_algorithmic": attn_bytes / (t_attn * 1e-3) / 1e9},
    }
    # roofline of the kernel family with the largest share of the step: prefill kernels are
    # dense matrix-core work (bound: the MFMA peak of their input type), decode kernels and
    # top-k stream memory (bound: HBM)
    share = {"indexer": (t_idx or 0.0) * len(full), "topk": (t_topk or 0.0) * len(full), "sparse_mla": t_attn * n}
    dom = max(share, key=share.get)
    if dom == "indexer" and prefill:
        kname = ("indexer_fp8_groups+fused_select" if fused else "indexer_fp8_groups") if w.idx_dtype == "fp8" \
            else "indexer_tile<BF16>"
        roof = {"bound": "mfma", "achieved": kernels["indexer"]["tflops"], "peak": idx_peak, "unit": "TFLOP/s",
                "kernel": kname, "algorithmic_per_launch": idx_flops, "launch_ms": t_idx}
        if w.idx_dtype == "fp8":
            roof["frac_of_bf16_peak"] = roof["achieved"] / PEAK_BF16_TFLOPS
    elif dom == "indexer":
        roof = {"bound": "hbm", "achieved": kernels["indexer"]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "kernel": "indexer_stream", "algorithmic_per_launch": idx_bytes, "launch_ms": t_idx}
    elif dom == "topk":
        roof = {"bound": "hbm", "achieved": kernels["topk"]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "kernel": "topk", "algorithmic_per_launch": topk_bytes, "launch_ms": t_topk}
    elif prefill:
        roof = {"bound": "mfma", "achieved": kernels["sparse_mla"]["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "kernel": "mla_mfma", "algorithmic_per_launch": attn_flops, "launch_ms": t_attn}
    else:
        ach = attn_bytes / (t_attn * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "kernel": "mla_mfma+mla_combine", "algorithmic_per_launch": attn_bytes, "launch_ms": t_attn}
    roof["frac"] = roof["achieved"] / roof["peak"]
    tr = MEASURED_TRAFFIC.get((w.name, roof["kernel"]))
    roof["traffic"] = tr["bytes"] if tr else None
    if tr:
        roof["traffic_source"] = tr["source"]
    step_dev = [events[s][0].elapsed_time(events[s][6 * n - 1]) for s in range(steps)]
    tokens = w.B * w.T
    res = {"value": tokens / (elapsed / steps) * n / 4.0, "ms_per_step": elapsed / steps * 1e3,
           "roofline": roof, "kernels": kernels,
           "step_device_ms": {f"p{q}": float(np.percentile(step_dev, q)) for q in (10, 50, 90)},
           "graph": None, "_cache": cache, "_stream": stream}
    if graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                B.group_forward(shape, mdt, types, dev, w.sm_scale, cache, 1, ws, stream=side)
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        gel = time.perf_counter() - t0
        res["graph"] = {"ms_per_step": gel / steps * 1e3, "value": tokens / (gel / steps) * n / 4.0,
                        "replays": steps}
        del g
    return res


def config_of(w):
    return {"workload": w.name, "batch": w.B, "queries_per_item": w.T, "prefix": w.S, "layers": w.layers,
            "index_heads": w.H, "index_dim": w.D, "index_key_heads": w.Hk, "index_dtype": w.idx_dtype,
            "topk": w.topk, "mla_heads": w.Hm, "latent": f"{w.Dc}+{w.Dr}", "parallelism": "single GPU"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.calibrate:
        calibrate()
        return
    if args.ab_indexer_topk:
        from dsa_indexer_top_lightning_amd import synth
        ab_indexer_topk(synth.WORKLOADS[args.workload], args.steps, args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path runs on a single "
              f"MI355X; sharding is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch

    from dsa_indexer_top_lightning_amd import binding as B
    from dsa_indexer_top_lightning_amd import synth

    w = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    inputs = synth.build_inputs(w)
    dev = upload(w, inputs, torch)
    print(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    if args.backward:
        m = run_forward(w, dev, 1, 1, False, torch, B)
        print(json.dumps(backward(args, w, inputs, dev, m["_cache"], torch, B, m["_stream"])))
        return
    m = run_forward(w, dev, args.steps, args.warmup, args.graph, torch, B)
    print(f"[bench] {w.name}: {m['ms_per_step']:.3f} ms per group call", file=sys.stderr, flush=True)
    res = {
        "metric": METRIC, "value": m["value"], "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.mla_dtype == "bf16" else "f32", "data": "synthetic",
        "config": config_of(w), "roofline": m["roofline"], "kernels": m["kernels"],
        "step_device_ms": m["step_device_ms"], "graph": m["graph"],
    }
    del dev
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a row sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    del inputs
    if not args.no_sub:
        res["workloads"] = {}
        for name in SUB_WORKLOADS:
            if name == w.name:
                continue
            sw = synth.WORKLOADS[name]
            print(f"[bench] sub-result {name}: generating inputs", file=sys.stderr, flush=True)
            t0 = time.perf_counter()
            sdev = upload(sw, synth.build_inputs(sw), torch)
            print(f"[bench] sub-result {name}: inputs ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
                  flush=True)
            sm = run_forward(sw, sdev, max(3, args.steps // 2), args.warmup, sw.T == 1, torch, B)
            res["workloads"][name] = {"config": config_of(sw), "steps": max(3, args.steps // 2),
                                      **{k: v for k, v in sm.items() if not k.startswith("_")}}
            print(f"[bench] sub-result {name}: {sm['ms_per_step']:.3f} ms per group call", file=sys.stderr,
                  flush=True)
            del sdev, sm
            torch.cuda.empty_cache()
    print(json.dumps(res))


# vector ALU fp32 peak without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP (FMA) x 2.4 GHz
PEAK_VALU_F32_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12


def backward(args, w, inputs, dev, cache, torch, B, stream):
    """Layer 0's backward on the forward group's indices and layer-0 results: the sparse MLA
    backward and the index-score backward at the selected positions, back to back."""
    L = dev[0]
    R = w.Dc + w.Dr
    g = torch.Generator(device="cuda").manual_seed(w.seed + 1000)
    dout = torch.randn(w.B, w.T, w.Hm, w.Dc, device="cuda", generator=g).to(L["out"].dtype)
    dI = torch.randn(w.B, w.T, w.topk, device="cuda", generator=g)
    dq = torch.empty(w.B, w.T, w.Hm, R, device="cuda")
    dkv = torch.empty(w.B, w.S, R, device="cuda")
    I = L["index"]
    dqi = torch.empty(w.B, w.T, w.H, w.D, device="cuda")
    dki = torch.empty(w.B, w.S, w.Hk, w.D, device="cuda")
    dwi = torch.empty(w.B, w.T, w.H, device="cuda")
    idx = cache.indices
    bshape = B.make_shape(w.B, w.T, w.S, topk=w.topk, Hm=w.Hm, Dc=w.Dc, Dr=w.Dr)
    nbws = B.workspace_bytes(bshape, B.OP_SPARSE_MLA_BWD)
    bws = torch.empty((nbws,), dtype=torch.uint8, device="cuda") if nbws else None
    ishape = B.make_shape(w.B, w.T, w.S, H=w.H, D=w.D, Hk=w.Hk, topk=w.topk)
    niws = B.workspace_bytes(ishape, B.OP_INDEX_BWD)
    iws = torch.empty((niws,), dtype=torch.uint8, device="cuda") if niws else None

    def call(ev=None):
        if ev:
            ev[0].record(stream)
        B.sparse_mla_backward(L["q"], L["kv"], idx, w.sm_scale, L["out"], L["lse"], dout, dq, dkv, Dc=w.Dc,
                              workspace=bws, stream=stream)
        if ev:
            ev[1].record(stream)
        B.index_backward(I["q"], I["k"], I["w"], idx, dI, dqi, dki, dwi, q_scale=I.get("q_scale"),
                         k_scale=I.get("k_scale"), workspace=iws, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        call()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.steps):
        call(evs[st])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_mla = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    t_idx = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    pairs = float((idx >= 0).sum().item())
    flops = pairs * w.Hm * 2.0 * (3 * R + 2 * w.Dc)
    iflops = pairs * w.H * 2.0 * 3 * w.D
    ach = flops / (t_mla * 1e-3) / 1e12
    iach = iflops / (t_idx * 1e-3) / 1e12
    dom_mla = t_mla >= t_idx
    # the matrix-core paths (a workspace is asked for exactly when they run) against the bf16 MFMA
    # peak, the vector kernels against the fp32 vector-ALU figure
    mla_mfma, idx_mfma = nbws > 0, niws > 0
    dom_mfma = mla_mfma if dom_mla else idx_mfma
    dom_peak = PEAK_BF16_TFLOPS if dom_mfma else PEAK_VALU_F32_TFLOPS
    res = {
        "metric": "query tokens/s through one layer's backward (sparse MLA dq, dkv; index score dq, dk, dw)",
        "value": w.B * w.T / (elapsed / args.steps), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.mla_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward, layer 0", "batch": w.B, "queries_per_item": w.T,
                   "prefix": w.S, "topk": w.topk, "index_heads": w.H, "index_dim": w.D, "index_key_heads": w.Hk,
                   "index_dtype": w.idx_dtype, "mla_heads": w.Hm, "latent": f"{w.Dc}+{w.Dr}",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma" if dom_mfma else "alu", "achieved": ach if dom_mla else iach, "peak": dom_peak,
                     "unit": "TFLOP/s", "frac": (ach if dom_mla else iach) / dom_peak, "traffic": None,
                     "kernel": "sparse MLA backward" if dom_mla else "index-score backward",
                     "algorithmic_per_launch": flops if dom_mla else iflops},
        "kernels": {"sparse_mla_bwd": {"ms": t_mla, "tflops": ach, "path": "matrix cores" if mla_mfma else "vector ALU"},
                    "index_bwd": {"ms": t_idx, "tflops": iach,
                                  "path": "matrix cores, dense selection" if idx_mfma else "vector ALU"}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle as O
        print("[bench] timing the CPU oracle backward on a row sample", file=sys.stderr, flush=True)
        idx_h = idx.cpu().numpy()
        dout_h = dout.to(torch.float64).cpu().numpy()
        q_h = O.decode(inputs[0]["mla_q"], w.mla_dtype)
        picks = [(b, t) for b in range(w.B) for t in range(w.T)]
        n = min(len(picks), 256)
        sel = [picks[i] for i in np.linspace(0, len(picks) - 1, n).astype(int)]
        dI_h = dI.to(torch.float64).cpu().numpy()
        I0 = inputs[0]
        kv_h, k_h = {}, {}
        t0 = time.perf_counter()
        for (b, t) in sel:
            if b not in kv_h:
                kv_h[b] = O.decode(inputs[0]["kv"][b], w.mla_dtype)
                k_h[b] = O.decode(I0["idx_k"][b], w.idx_dtype, I0["idx_k_scale"][b] if "idx_k_scale" in I0 else None)
            O.sparse_mla_backward_row(q_h[b, t], kv_h[b], idx_h[b, t], w.sm_scale, w.Dc, dout_h[b, t])
            qi = O.decode(I0["idx_q"][b, t], w.idx_dtype, I0["idx_q_scale"][b, t] if "idx_q_scale" in I0 else None)
            # the oracle on the row's selected keys only (same arithmetic, no full-size dk)
            row = idx_h[b, t]
            keys, pos = np.unique(row[row >= 0], return_inverse=True)
            ridx = np.full_like(row, -1)
            ridx[row >= 0] = pos
            O.index_scores_backward_selected(qi[None, None], k_h[b][keys][None],
                                             I0["w"][b, t][None, None].astype(np.float64), ridx[None, None],
                                             dI_h[b, t][None, None])
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": n / dt, "unit": "query tokens/s", "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{n} query rows evenly spaced over the {w.B}x{w.T} rows of {w.name}, "
                                         f"layer 0 backward (both), float64 NumPy, {dt:.1f} s (input decoding included)"}
    return res


if __name__ == "__main__":
    main()
