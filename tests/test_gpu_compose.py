"""GPU parity of the entry points that act on (out, lse) pairs.

* attn_sink_key0_correct -- the unfused key-0 sink of the MiMo window-attention
  page (closed form on the first W + 1 rows of each sequence, after a no-sink
  window attention).  Its plain definition is the oracle's key0_bias result.
* attn_sink_merge -- partial results over disjoint key sets merged by their
  LSEs, the null-logit sink folded in once after the merge (DeepSeek-V4 page,
  Implementation paragraph).  Its plain definition is the oracle's result over
  the union of the key sets.

Each kernel is checked in isolation (fed the oracle's own partial results,
rounded to the kernel's input types) and behind attn_sink_fwd (the whole
composed path on the GPU), plus the bitwise no-op cases the algebra fixes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def tdt(case):
    return torch.bfloat16 if case["dtype"] == "bf16" else torch.float32


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV, dtype)


def host(out, lse):
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(out, lse, ref_o, ref_l, case, label):
    rel, dl = G.compare(out, lse, ref_o, ref_l)
    tr, tl = G.tolerances(case)
    G.say(f"[compose] {label}: max rel L2 {rel:.3e} (<= {tr}), lse max abs {dl:.3e} (<= {tl})")
    assert rel <= tr and dl <= tl, (rel, dl)


def first_rows_mask(cu, W, T):
    """True for rows i with i - start(i) <= W (the rows that see their key 0)."""
    m = np.zeros(T, dtype=bool)
    for s in range(len(cu) - 1):
        m[cu[s]:min(cu[s + 1], cu[s] + W + 1)] = True
    return m


# ------------------------------------------------------- key-0 correction
def correct(case, d, out, lse):
    G.sam().attn_sink_key0_correct(d["q"], d["k"], d["v"], d["cu_seqlens"], case["window"], d["sinks"],
                                   case["scale"], out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_key0_correct_on_oracle_partials(dtype):
    """Fed the oracle's no-sink result, the correction reaches the oracle's
    key0_bias result on the affected rows and leaves every other row's bytes
    untouched.  Sequences shorter and longer than W + 1, GQA 16/4."""
    case = W.window_case([300, 40, 172, 65, 66], 16, 4, 80, 64, dtype=dtype, sink_mode="key0_bias",
                         sink_range=(-2.0, 2.0), seed=5)
    none_o, none_l = G.oracle_run(case, sink_mode="none", sinks=None)
    ref_o, ref_l = G.oracle_run(case)
    d = G.sam().case_on_device(case, DEV)
    out, lse = to_dev(none_o, tdt(case)), to_dev(none_l, torch.float32)
    out0, lse0 = out.clone(), lse.clone()
    correct(case, d, out, lse)
    o, l = host(out, lse)
    check(o, l, ref_o, ref_l, case, f"key0 correction on oracle partials ({dtype})")
    far = ~first_rows_mask(case["cu_seqlens"], case["window"], case["q"].shape[0])
    far_t = torch.from_numpy(far).to(DEV)
    assert torch.equal(out[far_t], out0[far_t]) and torch.equal(lse[:, far_t], lse0[:, far_t])


@pytest.mark.parametrize("name,seed,over", [
    ("window_4k", 0, {}), ("window_4k", 1, {"sink_range": (-2.0, 2.0)}), ("window_4k", 2, {"gqa": True}),
    ("window_16k", 0, {}), ("tiny_window_f32", 0, {})])
def test_unfused_pipeline_matches_oracle(name, seed, over):
    """No-sink window attention followed by the correction (the MiMo page's
    unfused design, both on the GPU) against the oracle's key0_bias result
    on every row; the fused key0_bias kernel is checked on the same inputs."""
    case = W.make_workload(name, seed=seed, **over)
    ref_o, ref_l = G.oracle_run(case)
    d = G.sam().case_on_device(case, DEV)
    base = dict(d, sink_mode="none", sinks=None)
    out, lse = G.sam().fwd(**base)
    correct(case, d, out, lse)
    o, l = host(out, lse)
    check(o, l, ref_o, ref_l, case, f"unfused {name} seed {seed} {over}")
    fo, fl = G.gpu_run(case)
    check(fo, fl, ref_o, ref_l, case, f"fused {name} seed {seed} {over}")


def test_key0_correct_zero_sink_is_bitwise_noop():
    """s = 0 gives c = p0 (e^0 - 1) = 0 exactly: out and lse keep their bits."""
    case = W.window_case([500, 12], 16, 16, 64, 64, sink_mode="key0_bias", seed=7)
    d = G.sam().case_on_device(case, DEV)
    d["sinks"].zero_()
    out, lse = G.sam().fwd(**dict(d, sink_mode="none", sinks=None))
    out0, lse0 = out.clone(), lse.clone()
    correct(case, d, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, out0) and torch.equal(lse, lse0)


# ------------------------------------------------------------------ merge
def merge(parts, sinks, sink_mode, like_out, like_lse):
    out, lse = torch.empty_like(like_out), torch.empty_like(like_lse)
    G.sam().attn_sink_merge(parts, sinks, sink_mode, out, lse)
    return out, lse


def topk_halves(case, nparts=2):
    idx = case["topk_idx"]
    cuts = np.linspace(0, idx.shape[1], nparts + 1).astype(int)
    return [np.ascontiguousarray(idx[:, a:b]) for a, b in zip(cuts[:-1], cuts[1:])]


def blocksel_residue_split(case, nparts):
    """Key block b goes to part b % nparts."""
    tab = case["block_sel"]
    nb = np.arange(tab.shape[3])
    return [np.ascontiguousarray(tab * (nb % nparts == r)[None, None, None, :].astype(np.uint8))
            for r in range(nparts)]


def split_kw(case, piece):
    return {"topk_idx": piece} if case["mask_kind"] == "topk" else {"block_sel": piece}


def splits(case, nparts):
    return topk_halves(case, nparts) if case["mask_kind"] == "topk" else blocksel_residue_split(case, nparts)


CASES = {
    "mla_small": lambda: W.topk_case(96, 3000, 64, 576, 512, 256, counts=(0, 1, 5, 31, 100, 256), shuffled=True,
                                     seed=21),
    "topk_f32": lambda: W.topk_case(40, 500, 8, 64, 32, 48, counts=(0, 1, 7, 48), shuffled=True, mla=False, Hkv=2,
                                    std=1.0, dtype="f32", seed=22),
    "blocksel": lambda: W.blocksel_case([700, 120, 461], 32, 8, 128, n_random=5, Hidx=8, sink_mode="null_logit",
                                        sink_range=(-2.0, 2.0), seed=23),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("nparts", [2, 3])
def test_merge_on_oracle_partials(name, nparts):
    """The oracle's no-sink results over a split of every row's key set
    (top-k column ranges; key blocks by residue), rounded to the kernel's
    input types and merged on the GPU with the null-logit sink, reach the
    oracle's result over the whole key set."""
    case = CASES[name]()
    ref_o, ref_l = G.oracle_run(case)
    parts = []
    for piece in splits(case, nparts):
        po, pl = G.oracle_run(case, sink_mode="none", sinks=None, **split_kw(case, piece))
        parts.append((to_dev(po, tdt(case)), to_dev(pl, torch.float32)))
    sinks = to_dev(case["sinks"], torch.float32)
    out, lse = merge(parts, sinks, "null_logit", parts[0][0], parts[0][1])
    o, l = host(out, lse)
    check(o, l, ref_o, ref_l, case, f"merge of {nparts} oracle partials ({name})")


@pytest.mark.parametrize("name", list(CASES))
def test_split_fwd_then_merge(name):
    """The composed GPU path: attn_sink_fwd without sink on each part of the
    split, attn_sink_merge with the sink, against the oracle on the union."""
    case = CASES[name]()
    ref_o, ref_l = G.oracle_run(case)
    d = G.sam().case_on_device(case, DEV)
    parts = []
    for piece in splits(case, 2):
        key = "topk_idx" if case["mask_kind"] == "topk" else "block_sel"
        dd = dict(d, sink_mode="none", sinks=None)
        dd[key] = torch.from_numpy(piece).to(DEV, dd[key].dtype)
        parts.append(G.sam().fwd(**dd))
    out, lse = merge(parts, d["sinks"], "null_logit", parts[0][0], parts[0][1])
    o, l = host(out, lse)
    check(o, l, ref_o, ref_l, case, f"split fwd + merge ({name})")


def test_split_fwd_then_merge_mla_full_size():
    """The sparse-MLA workload at full size, its 2048-entry lists cut into two
    column halves, each half through the no-sink kernel, then merged with the
    null-logit sink; oracle on rows from every valid-count bucket."""
    case = W.make_workload("mla_topk", seed=1)
    d = G.sam().case_on_device(case, DEV)
    parts = []
    for piece in topk_halves(case):
        parts.append(G.sam().fwd(**dict(d, sink_mode="none", sinks=None,
                                        topk_idx=torch.from_numpy(piece).to(DEV))))
    out, lse = merge(parts, d["sinks"], "null_logit", parts[0][0], parts[0][1])
    o, l = host(out, lse)
    n = (case["topk_idx"] >= 0).sum(1)
    g = np.random.default_rng(3)
    rows = np.array(sorted(sum((g.choice(np.flatnonzero(n == c), size=12, replace=False).tolist()
                                for c in np.unique(n)), [])), dtype=np.int64)
    ref_o, ref_l = G.oracle_run(case, rows=rows)
    check(o[rows], l[:, rows], ref_o, ref_l, case, "mla_topk split in two + merge")


def test_merge_identities_bitwise():
    """Exact cases of the merge algebra: one part with no sink returns that
    part; an empty part (lse = -inf) carries no weight; a sink of -inf equals
    no sink."""
    case = CASES["mla_small"]()
    d = G.sam().case_on_device(case, DEV)
    a_o, a_l = G.sam().fwd(**dict(d, sink_mode="none", sinks=None))
    o1, l1 = merge([(a_o, a_l)], None, "none", a_o, a_l)
    empty_o, empty_l = torch.zeros_like(a_o), torch.full_like(a_l, float("-inf"))
    o2, l2 = merge([(a_o, a_l), (empty_o, empty_l)], None, "none", a_o, a_l)
    ninf = torch.full_like(d["sinks"], float("-inf"))
    o3, l3 = merge([(a_o, a_l), (empty_o, empty_l)], ninf, "null_logit", a_o, a_l)
    torch.cuda.synchronize()
    for o, l in ((o1, l1), (o2, l2), (o3, l3)):
        assert torch.equal(o, a_o) and torch.equal(l, a_l)
