"""GPU parity of the sparse-MLA decode over an fp8 latent cache (the decode
call site of the DeepSeek-V4 XPU sparse-MLA page) against oracle/fp8.py:
dequantized cache, top-k masked softmax, null-logit sink folded after the
merge of the list pieces, LSE over the selected keys only."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import fp8
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def run(case):
    d = G.sam().decode_case_on_device(case)
    G.sam().attn_sink_mla_decode_fp8(d["q"], d["kv"], d["kv_scale"], d["topk_idx"], d["sinks"], d["sink_mode"],
                                     d["scale"], d["out"], d["lse"], d["workspace"])
    torch.cuda.synchronize()
    return d


def check(case, label, rows=None):
    d = run(case)
    out = d["out"].float().cpu().numpy().astype(np.float64)
    lse = d["lse"].cpu().numpy().astype(np.float64)
    ref_o, ref_l = fp8.decode_ref(case, rows=rows)
    if rows is not None:
        out, lse = out[rows], lse[:, rows]
    rel, dl = G.compare(out, lse, ref_o, ref_l)
    G.say(f"[decode] {label}: max rel L2 {rel:.3e}, lse max abs {dl:.3e}")
    assert rel <= G.BF16_REL_L2 and dl <= G.BF16_LSE_ABS, (rel, dl)
    return d


@pytest.mark.parametrize("T,Hq,topk,counts,kw", [
    (1, 64, 2048, (2048,), {}),
    (5, 64, 300, (0, 1, 17, 300), {"shuffled": True}),
    (17, 128, 256, (1, 4, 16, 128, 256), {"shuffled": True, "out_of_range": True}),
    (64, 64, 2048, (1, 4, 16, 128, 512, 2048), {}),
    (300, 64, 512, (0, 33, 512), {"sink_mode": "none"}),
])
def test_decode_small(T, Hq, topk, counts, kw):
    case = W.mla_decode_fp8_case(T, 5000, Hq, topk, counts=counts, seed=T + Hq, **kw)
    check(case, f"T={T} Hq={Hq} topk={topk} {kw}")


@pytest.mark.parametrize("seed", [0, 1])
def test_decode_full_size(seed):
    """The decode workload the benchmark times (128 rows x 64 heads, 65536-row
    fp8 cache, full 2048-entry lists), every row against the oracle."""
    check(W.make_workload("mla_decode_fp8", seed=seed), f"mla_decode_fp8 seed {seed}")


def test_decode_full_size_buckets():
    case = W.make_workload("mla_decode_fp8", seed=2, counts=(1, 4, 16, 128, 512, 2048), shuffled=True)
    check(case, "mla_decode_fp8 buckets, shuffled padding")


def test_decode_neg_inf_sink_is_bitwise_noop():
    case = W.mla_decode_fp8_case(40, 3000, 64, 512, counts=(1, 9, 512), seed=9)
    a = run(case)
    case_inf = dict(case, sinks=np.full_like(case["sinks"], -np.inf))
    b = run(case_inf)
    none = run(dict(case, sink_mode="none", sinks=None))
    assert torch.equal(b["out"], none["out"]) and torch.equal(b["lse"], none["lse"])
    assert torch.equal(a["lse"], none["lse"])          # the LSE never includes the sink
    assert not torch.equal(a["out"], none["out"])


def test_decode_cache_rows_past_2_31():
    """The fp8 cache is a strided view with a row stride just over 2 MB, so
    every entry from row 1024 on starts past byte 2**31 of the allocation (an
    fp8 element is a byte): the gathers are correct only with 64-bit row
    offsets.  The lists address only those rows (distinct per row)."""
    case = W.mla_decode_fp8_case(24, 3000, 64, 256, counts=(1, 17, 256), shuffled=True, seed=8)
    idx = case["topk_idx"]
    g = np.random.default_rng(8)
    for i in range(idx.shape[0]):
        slots = np.flatnonzero(idx[i] >= 0)
        idx[i, slots] = g.choice(np.arange(1024, 3000), size=len(slots), replace=False)
    stride = (1 << 21) + 4096                          # bytes per cache row
    assert 1024 * stride > 2 ** 31
    d = G.sam().decode_case_on_device(case)
    big = torch.zeros(3000 * stride, dtype=torch.uint8, device="cuda:0")
    kv = big.as_strided((3000, 1, 576), (stride, 576, 1))
    kv.copy_(torch.from_numpy(case["kv_fp8"]).cuda())
    G.sam().attn_sink_mla_decode_fp8(d["q"], kv.view(torch.float8_e4m3fn), d["kv_scale"], d["topk_idx"],
                                     d["sinks"], d["sink_mode"], d["scale"], d["out"], d["lse"], d["workspace"])
    torch.cuda.synchronize()
    out = d["out"].float().cpu().numpy().astype(np.float64)
    lse = d["lse"].cpu().numpy().astype(np.float64)
    ref_o, ref_l = fp8.decode_ref(case)
    rel, dl = G.compare(out, lse, ref_o, ref_l)
    G.say(f"[decode >2^31 row offsets] rel {rel:.3e} lse {dl:.3e}")
    assert rel <= G.BF16_REL_L2 and dl <= G.BF16_LSE_ABS
    del big, kv
    torch.cuda.empty_cache()
