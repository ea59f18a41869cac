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
