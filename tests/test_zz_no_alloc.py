"""dsa_group_forward_noalloc against dsa_group_forward: the allocation-free entry point runs
the same kernels on the library's own device scratch, so its indices and outputs must equal
those of the workspace call bit for bit.  Two calls in a row, the second on a smaller input
(the scratch then holds the first call's data), and the size limit."""
import numpy as np
import pytest
import torch

from dsa_indexer_top_lightning_amd import binding as b
from dsa_indexer_top_lightning_amd import synth
from helpers import f32_dev, i32_dev, to_dev

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="t", B=1, T=64, S=64, pos0=0, layers="FSSS", H=32, D=128, Hk=32, topk=2048, Hm=64, Dc=512,
                Dr=64, idx_dtype="bf16", mla_dtype="bf16", seed=31)
    base.update(kw)
    return synth.Workload(**base)


def _upload(w):
    dev = []
    for L in synth.build_inputs(w):
        d = {"q": to_dev(L["mla_q"], w.mla_dtype), "kv": to_dev(L["kv"], w.mla_dtype),
             "out": torch.full((w.B, w.T, w.Hm, w.Dc), float("nan"), device="cuda", dtype=torch.bfloat16),
             "lse": torch.full((w.B, w.T, w.Hm), float("nan"), device="cuda")}
        if "idx_q" in L:
            d["index"] = {"q": to_dev(L["idx_q"], w.idx_dtype), "k": to_dev(L["idx_k"], w.idx_dtype),
                          "w": f32_dev(L["w"])}
            if w.idx_dtype == "fp8":
                d["index"]["q_scale"] = f32_dev(L["idx_q_scale"])
                d["index"]["k_scale"] = f32_dev(L["idx_k_scale"])
        dev.append(d)
    return dev


def _both(w):
    dev = _upload(w)
    types = ["full" if c == "F" else "shared" for c in w.layers]
    ke = w.key_end()
    shape = b.make_shape(w.B, w.T, w.S, H=w.H, D=w.D, Hk=w.Hk, topk=w.topk, Hm=w.Hm, Dc=w.Dc, Dr=w.Dr,
                         key_end=i32_dev(ke), key_end_host=ke)
    need = b.workspace_bytes(shape, b.OP_GROUP)
    assert 0 < need <= b.noalloc_scratch_bytes()
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    c1 = b.IndexCache(w.B, w.T, w.topk)
    s1 = b.group_forward(shape, b.BF16, types, dev, w.sm_scale, c1, 5, ws)
    ref = [(d["out"].clone(), d["lse"].clone()) for d in dev]
    for d in dev:
        d["out"].fill_(float("nan"))
        d["lse"].fill_(float("nan"))
    c2 = b.IndexCache(w.B, w.T, w.topk)
    s2 = b.group_forward_noalloc(shape, b.BF16, types, dev, w.sm_scale, c2, 5)
    torch.cuda.synchronize()
    assert torch.equal(c2.indices, c1.indices)
    assert (c2.c.valid, c2.c.tag, c2.c.donor_layer) == (1, 5, c1.c.donor_layer)
    for l, d in enumerate(dev):
        assert torch.equal(d["out"], ref[l][0]), f"layer {l}: out"
        assert torch.equal(d["lse"], ref[l][1]), f"layer {l}: lse"
    for key in ("n_full", "n_shared", "n_launches", "indexer_flops", "attn_flops", "attn_bytes"):
        assert getattr(s1, key) == getattr(s2, key), key
    return need


def test_noalloc_group_matches_workspace_call_twice_second_smaller():
    # a decode batch (chunked top-k and split attention both use the scratch), then a smaller
    # prefill: the second call runs over scratch that still holds the first call's data
    big = _both(_wl(B=6, T=1, S=20000, pos0=19999, layers="FSSF"))
    small = _both(_wl(B=1, T=300, S=300, pos0=0, topk=256, layers="FS"))
    assert small < big


def test_noalloc_rejects_a_call_beyond_its_scratch():
    w = _wl(B=1, T=4096, S=8192, pos0=4096, layers="F")
    shape = b.make_shape(w.B, w.T, w.S, H=w.H, D=w.D, Hk=w.Hk, topk=w.topk, Hm=w.Hm, Dc=w.Dc, Dr=w.Dr)
    assert b.workspace_bytes(shape, b.OP_GROUP) > b.noalloc_scratch_bytes()
    cache = b.IndexCache(1, 4096, 2048)
    layer = {"q": torch.empty(0, device="cuda"), "kv": torch.empty(0, device="cuda"),
             "out": torch.empty(0, device="cuda"),
             "index": {"q": torch.empty(0, device="cuda"), "k": torch.empty(0, device="cuda"),
                       "w": torch.empty(0, device="cuda")}}
    with pytest.raises(b.DsaError) as e:
        b.group_forward_noalloc(shape, b.BF16, ["full"], [layer], w.sm_scale, cache, 1)
    assert e.value.status == 5 and "allocation-free" in str(e.value)
    assert not cache.valid
