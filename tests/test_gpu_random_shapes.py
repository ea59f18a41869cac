"""GPU parity over seeded random shapes: for each mask kind, cases whose
sequence lengths, head groupings, head dims, window widths, list lengths,
padding patterns, selection densities and sink modes are drawn from a fixed
seed, each checked against the oracle on every row.  The draws stay inside
what the kernels accept (the shapes the C ABI documents), so every case is a
valid call; the point is combinations no hand-written case covers."""
from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

N_CASES = 12


def window_draw(seed):
    g = np.random.default_rng(1000 + seed)
    nseq = int(g.integers(1, 6))
    lens = [int(x) for x in g.integers(0, 400, size=nseq)]
    if sum(lens) == 0:
        lens[0] = 1
    Hq, Hkv = [(4, 4), (8, 2), (6, 3), (16, 1), (2, 1)][int(g.integers(0, 5))]
    D = int(g.choice([64, 80, 96, 128]))
    Wd = int(g.choice([0, 1, 7, 31, 64, 100, 250, 1 << 20]))
    sink = str(g.choice(["none", "key0_bias", "null_logit"]))
    scale = float(g.choice([1.0 / np.sqrt(D), 0.3, -0.2]))
    return W.window_case(lens, Hq, Hkv, D, Wd, dtype="bf16", sink_mode=sink, sink_range=(-2, 2), scale=scale,
                         seed=2000 + seed), f"lens={lens} H={Hq}/{Hkv} D={D} W={Wd} {sink} scale={scale:.3f}"


def topk_draw(seed):
    g = np.random.default_rng(3000 + seed)
    T = int(g.integers(1, 40))
    Tk = int(g.integers(32, 9000))
    topk = int(g.choice([1, 31, 32, 33, 200, 1024, 2047, 3000]))
    counts = tuple(sorted(set(int(c) for c in g.integers(0, topk + 1, size=4))))
    Hq = int(g.choice([64, 128]))
    sink = str(g.choice(["none", "null_logit"]))
    kw = dict(shuffled=bool(g.integers(0, 2)), out_of_range=bool(g.integers(0, 2)))
    return W.topk_case(T, Tk, Hq, 576, 512, topk, counts=counts, sink_mode=sink, seed=4000 + seed, **kw), \
        f"T={T} Tk={Tk} topk={topk} counts={counts} Hq={Hq} {sink} {kw}"


def blocksel_draw(seed):
    g = np.random.default_rng(5000 + seed)
    ndoc = int(g.integers(1, 5))
    lens = [int(x) for x in g.integers(1, 700, size=ndoc)]
    Hkv = int(g.choice([1, 2, 4]))
    Hidx = int(g.choice([h for h in (1, 2, 4) if Hkv % h == 0]))
    nr = int(g.choice([0, 1, 3, 15, 40]))
    sink = str(g.choice(["none", "key0_bias", "null_logit"]))
    return W.blocksel_case(lens, 4 * Hkv, Hkv, 128, n_random=nr, Hidx=Hidx, sink_mode=sink, sink_range=(-2, 2),
                           seed=6000 + seed), f"lens={lens} Hkv={Hkv} Hidx={Hidx} nr={nr} {sink}"


@pytest.mark.parametrize("seed", range(N_CASES))
def test_window_random_shapes(seed):
    case, label = window_draw(seed)
    G.assert_parity(case, label=f"window random {seed}: {label}")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_topk_random_shapes(seed):
    case, label = topk_draw(seed)
    G.assert_parity(case, label=f"topk random {seed}: {label}")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_blocksel_random_shapes(seed):
    case, label = blocksel_draw(seed)
    G.assert_parity(case, label=f"blocksel random {seed}: {label}")


def decode_draw(seed):
    g = np.random.default_rng(7000 + seed)
    T = int(g.integers(1, 64))
    Tk = int(g.integers(64, 20000))
    topk = int(g.choice([1, 32, 100, 512, 2048, 4096]))
    counts = tuple(sorted(set(int(c) for c in g.integers(0, topk + 1, size=3))))
    Hq = int(g.choice([64, 128]))
    sink = str(g.choice(["none", "null_logit"]))
    kw = dict(shuffled=bool(g.integers(0, 2)), out_of_range=bool(g.integers(0, 2)))
    return W.mla_decode_fp8_case(T, Tk, Hq, topk, counts=counts, sink_mode=sink, seed=8000 + seed, **kw), \
        f"T={T} Tk={Tk} topk={topk} counts={counts} Hq={Hq} {sink} {kw}"


@pytest.mark.parametrize("seed", range(N_CASES // 2))
def test_decode_fp8_random_shapes(seed):
    import torch
    from oracle import fp8
    case, label = decode_draw(seed)
    d = G.sam().decode_case_on_device(case)
    G.sam().attn_sink_mla_decode_fp8(d["q"], d["kv"], d["kv_scale"], d["topk_idx"], d["sinks"], d["sink_mode"],
                                     d["scale"], d["out"], d["lse"], d["workspace"])
    torch.cuda.synchronize()
    out = d["out"].float().cpu().numpy().astype(np.float64)
    lse = d["lse"].cpu().numpy().astype(np.float64)
    ref_o, ref_l = fp8.decode_ref(case)
    rel, dl = G.compare(out, lse, ref_o, ref_l)
    G.say(f"[decode random {seed}] {label}: max rel L2 {rel:.3e}, lse max abs {dl:.3e}")
    assert rel <= G.BF16_REL_L2 and dl <= G.BF16_LSE_ABS, (rel, dl)


@pytest.mark.parametrize("seed", range(N_CASES // 2))
def test_topk_split_merge_random(seed):
    """A random top-k case, its lists cut at random columns into 2..8 parts,
    each part through the no-sink kernel, merged with the case's sink."""
    import torch
    case, label = topk_draw(100 + seed)
    g = np.random.default_rng(9000 + seed)
    idx = case["topk_idx"]
    nparts = int(g.integers(2, 9))
    cuts = np.sort(g.choice(np.arange(1, idx.shape[1]), size=min(nparts - 1, idx.shape[1] - 1), replace=False)) \
        if idx.shape[1] > 1 else np.array([], dtype=int)
    edges = [0] + [int(c) for c in cuts] + [idx.shape[1]]
    d = G.sam().case_on_device(case, "cuda:0")
    parts = []
    for a, b in zip(edges[:-1], edges[1:]):
        piece = torch.from_numpy(np.ascontiguousarray(idx[:, a:b])).to("cuda:0")
        parts.append(G.sam().fwd(**dict(d, sink_mode="none", sinks=None, topk_idx=piece)))
    out, lse = torch.empty_like(parts[0][0]), torch.empty_like(parts[0][1])
    G.sam().attn_sink_merge(parts, d["sinks"], case["sink_mode"], out, lse)
    torch.cuda.synchronize()
    o, l = out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    ref_o, ref_l = G.oracle_run(case)
    rel, dl = G.compare(o, l, ref_o, ref_l)
    G.say(f"[merge random {seed}] {len(edges) - 1} parts, {label}: max rel L2 {rel:.3e}, lse max abs {dl:.3e}")
    assert rel <= G.BF16_REL_L2 and dl <= G.BF16_LSE_ABS, (rel, dl)
