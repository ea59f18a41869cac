"""The allocation-free fp8 decode entry point (attn_sink_mla_decode_fp8_noalloc)
against the workspace entry point it shares its kernels with: two calls in a
row through the C ABI, the second on a smaller input (so it runs on scratch
that still holds the first call's partials), each bit-identical to the
workspace call on the same inputs, hence within the parity bar of the oracle
comparison in test_gpu_decode.py; and a call past the scratch limit refused on
the host before anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _both(case):
    import torch
    sam = G.sam()
    d = sam.decode_case_on_device(case, "cuda:0")
    sam.attn_sink_mla_decode_fp8(d["q"], d["kv"], d["kv_scale"], d["topk_idx"], d["sinks"], d["sink_mode"],
                                 d["scale"], d["out"], d["lse"], d["workspace"])
    out2 = torch.full_like(d["out"], float("nan"))
    lse2 = torch.full_like(d["lse"], float("nan"))
    sam.attn_sink_mla_decode_fp8_noalloc(d["q"], d["kv"], d["kv_scale"], d["topk_idx"], d["sinks"], d["sink_mode"],
                                         d["scale"], out2, lse2)
    torch.cuda.synchronize()
    return d["out"], d["lse"], out2, lse2


def test_noalloc_matches_workspace_entry_point_twice():
    import torch
    calls = [
        # the decode workload: 128 rows x 64 heads, full 2048-entry lists (4 pieces, 67.2 MB of partials)
        W.make_workload("mla_decode_fp8", seed=3),
        # then a smaller call: 5 rows, 128 heads, mixed list lengths with padding anywhere
        W.mla_decode_fp8_case(5, 3000, 128, 256, counts=(0, 1, 17, 256), shuffled=True, out_of_range=True,
                              seed=4),
    ]
    for n, case in enumerate(calls):
        G.say(f"[noalloc] call {n}: T={case['q'].shape[0]} Hq={case['q'].shape[1]} topk={case['topk_idx'].shape[1]}")
        o1, l1, o2, l2 = _both(case)
        assert torch.equal(o1, o2), "out differs from the workspace entry point"
        assert torch.equal(l1.isneginf(), l2.isneginf())
        fin = ~l1.isneginf()
        assert torch.equal(l1[fin], l2[fin]), "lse differs from the workspace entry point"
        rel, dl = G.compare(o2.float().cpu().numpy().astype(np.float64), l2.cpu().numpy().astype(np.float64),
                            o1.float().cpu().numpy().astype(np.float64), l1.cpu().numpy().astype(np.float64))
        assert rel <= G.BF16_REL_L2 and dl <= G.BF16_LSE_ABS


def test_noalloc_refuses_calls_past_the_scratch_limit():
    import torch
    sam = G.sam()
    T, Hq, topk, Tk = 1024, 64, 2048, 4096
    need = sam.attn_sink_mla_decode_fp8_workspace(T, Hq, topk)
    assert need > sam.DECODE_SCRATCH_BYTES
    q = torch.zeros((T, Hq, 576), dtype=torch.bfloat16, device="cuda:0")
    kv = torch.zeros((Tk, 1, 576), dtype=torch.uint8, device="cuda:0").view(torch.float8_e4m3fn)
    idx = torch.full((T, topk), -1, dtype=torch.int32, device="cuda:0")
    out = torch.empty((T, Hq, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda:0")
    with pytest.raises(sam.AttnSinkError) as e:
        sam.attn_sink_mla_decode_fp8_noalloc(q, kv, torch.ones(Tk, device="cuda:0"), idx, None, "none", 0.04,
                                             out, lse)
    assert e.value.status == -8  # ATTN_ERR_RANGE
