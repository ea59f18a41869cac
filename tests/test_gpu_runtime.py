"""Runtime properties the C ABI promises, on the GPU: every kernel can be
captured in a HIP graph and replayed (several replays, with eager work and
synchronisations between them, each bit-identical to the eager call); calls
on two streams at once give the results of the same calls one after the
other (no hidden shared state); repeated calls are bitwise deterministic."""
from __future__ import annotations

import pytest
import torch

import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def small_cases():
    return {
        "window_bf16": W.window_case([300, 17, 200], 16, 4, 80, 64, sink_mode="key0_bias", seed=31),
        "window_f32": W.tiny_window(seed=2),
        "topk_mla": W.topk_case(64, 4000, 64, 576, 512, 512, counts=(0, 3, 100, 512), shuffled=True, seed=32),
        "blocksel": W.blocksel_case([400, 230], 32, 8, 128, n_random=6, sink_mode="null_logit", seed=33),
    }


def fwd_call(d, out, lse):
    return lambda: G.sam().fwd(**d, out=out, lse=lse)


@pytest.mark.parametrize("name", list(small_cases()))
def test_graph_replays_match_eager(name):
    case = small_cases()[name]
    sam = G.sam()
    d = sam.case_on_device(case, DEV)
    ref_o, ref_l = sam.fwd(**d)
    out, lse = torch.empty_like(ref_o), torch.empty_like(ref_l)
    fwd_call(d, out, lse)()  # warm up on the capture's buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd_call(d, out, lse)()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), (name, rep)
        sam.fwd(**d, out=torch.empty_like(ref_o), lse=torch.empty_like(ref_l))  # eager work in between
        torch.cuda.synchronize()


def test_graph_replays_of_decode_and_merge():
    sam = G.sam()
    case = W.mla_decode_fp8_case(24, 3000, 64, 256, counts=(1, 40, 256), seed=34)
    d = sam.decode_case_on_device(case, DEV)
    args = (d["q"], d["kv"], d["kv_scale"], d["topk_idx"], d["sinks"], d["sink_mode"], d["scale"])
    sam.attn_sink_mla_decode_fp8(*args, d["out"], d["lse"], d["workspace"])
    torch.cuda.synchronize()
    ref_o, ref_l = d["out"].clone(), d["lse"].clone()
    mo, ml = torch.empty_like(ref_o), torch.empty_like(ref_l)
    sam.attn_sink_merge([(ref_o, ref_l)], d["sinks"], "null_logit", mo, ml)
    torch.cuda.synchronize()
    ref_mo, ref_ml = mo.clone(), ml.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sam.attn_sink_mla_decode_fp8(*args, d["out"], d["lse"], d["workspace"])
        sam.attn_sink_merge([(d["out"], d["lse"])], d["sinks"], "null_logit", mo, ml)
    for rep in range(3):
        for t in (d["out"], d["lse"], mo, ml):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["out"], ref_o) and torch.equal(d["lse"], ref_l), rep
        assert torch.equal(mo, ref_mo) and torch.equal(ml, ref_ml), rep


def test_two_streams_concurrently_equal_sequential():
    sam = G.sam()
    cases = small_cases()
    a = sam.case_on_device(cases["topk_mla"], DEV)
    b = sam.case_on_device(cases["blocksel"], DEV)
    ra, rb = sam.fwd(**a), sam.fwd(**b)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    outs = []
    for _ in range(4):
        oa, la = torch.empty_like(ra[0]), torch.empty_like(ra[1])
        ob, lb = torch.empty_like(rb[0]), torch.empty_like(rb[1])
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            sam.fwd(**a, out=oa, lse=la)
        with torch.cuda.stream(s2):
            sam.fwd(**b, out=ob, lse=lb)
        outs.append((oa, la, ob, lb))
    torch.cuda.synchronize()
    for oa, la, ob, lb in outs:
        assert torch.equal(oa, ra[0]) and torch.equal(la, ra[1])
        assert torch.equal(ob, rb[0]) and torch.equal(lb, rb[1])


@pytest.mark.parametrize("name", list(small_cases()))
def test_repeated_calls_are_bitwise_deterministic(name):
    sam = G.sam()
    d = sam.case_on_device(small_cases()[name], DEV)
    first = sam.fwd(**d)
    for _ in range(3):
        again = sam.fwd(**d)
        torch.cuda.synchronize()
        assert torch.equal(again[0], first[0]) and torch.equal(again[1], first[1])
