"""The seeded input generators produce the structure each workload promises (no GPU)."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch_rne():
    x = W.rng(0).standard_normal(100_003).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(W.round_bf16(x), ref)
    assert np.array_equal(W.bf16_bits(ref), torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_seeded_and_bf16_representable():
    a = W.window_case([40, 30], 4, 2, 80, 8, seed=3)
    b = W.window_case([40, 30], 4, 2, 80, 8, seed=3)
    c = W.window_case([40, 30], 4, 2, 80, 8, seed=4)
    for key in ("q", "k", "v", "sinks"):
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["q"], c["q"])
    assert np.array_equal(W.round_bf16(a["q"]), a["q"])
    assert a["sinks"].min() >= -0.1 and a["sinks"].max() <= 0.6


def test_long_window_lengths():
    for seed in range(3):
        lens = W.c3_seqlens(seed)
        assert len(lens) == 8 and sum(lens) == 16384
        assert sum(1 for n in lens if n < 64) >= 1 and min(lens) >= 1


def test_blocksparse_documents_and_table():
    for seed in range(3):
        lens = W.c5_doc_lens(seed)
        cu = np.cumsum(lens)
        assert len(lens) == 4 and cu[-1] == 32768 and np.all(cu[:-1] % 64 != 0)
    lens = [1000, 3000, 2100]
    case = W.blocksel_case(lens, 4, 2, 16, block_size=64, n_random=15, seed=1)
    tab = case["block_sel"]
    T = sum(lens)
    starts = np.repeat(case["cu_seqlens"][:-1], lens)
    for h in range(2):
        for i in range(0, T, 7):
            sel = np.flatnonzero(tab[0, h, i])
            diag = i // 64
            c = diag - starts[i] // 64
            assert diag in sel
            assert len(sel) == 1 + min(15, c)
            assert sel.min() >= starts[i] // 64 and sel.max() == diag


def test_topk_lists():
    case = W.topk_case(300, 5000, 4, 32, 16, 64, counts=(1, 4, 16, 64), seed=2)
    idx = case["topk_idx"]
    n = (idx >= 0).sum(1)
    assert set(n.tolist()) <= {1, 4, 16, 64}
    for r in idx:
        valid = r[r >= 0]
        assert len(set(valid.tolist())) == len(valid) and valid.max() < 5000
        assert np.all(r[len(valid):] == -1)
    sh = W.topk_case(50, 500, 2, 32, 16, 20, counts=(3, 7), shuffled=True, seed=2)
    assert any(np.any(r[:(r >= 0).sum()] < 0) for r in sh["topk_idx"])
    assert np.shares_memory(case["k"], case["v"]) and case["v"].shape[2] == 16
