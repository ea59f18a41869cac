"""The benchmark's accounting, on the CPU.  Every reported TFLOP/s and roofline
fraction rests on two numbers: the useful (row, head, key) pairs
2 (Dqk + Dv) |S(i,h)| counts, and the algorithmic bytes of one launch.  Here
the pair counts equal membership counted from masks built with explicit
loops, and the full-size figures equal closed forms of the workloads' shapes
(MiMo window: L (2W + 1) - W (W + 1) pairs per sequence of length L > W)."""
from __future__ import annotations

import numpy as np
import pytest

import bench
import workloads as W
from tests import pins as P


def brute_pairs(case) -> np.ndarray:
    T, Hq = case["q"].shape[:2]
    tot = np.zeros(T, dtype=np.int64)
    for h in range(Hq):
        tot += P.loop_mask(case, h).sum(1)
    return tot


SMALL = {
    "window": lambda: W.window_case([70, 3, 130, 1], 4, 2, 64, 9, dtype="bf16", sink_mode="key0_bias", seed=1),
    "window_wide": lambda: W.window_case([50, 40], 2, 2, 64, 1000, dtype="bf16", sink_mode="none", seed=2),
    "topk": lambda: W.topk_case(40, 300, 4, 64, 64, 50, counts=(0, 1, 7, 50), shuffled=True, mla=False, Hkv=2,
                                std=1.0, dtype="bf16", sink_mode="null_logit", seed=3, out_of_range=True),
    "blocksel": lambda: W.blocksel_case([150, 99, 140], 8, 2, 128, n_random=3, Hidx=2, sink_mode="none", seed=4),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_pairs_per_row_match_loop_masks(name):
    case = SMALL[name]()
    assert np.array_equal(bench.pairs_per_row(case), brute_pairs(case))


def test_window_4k_pairs_and_bytes_closed_form():
    case = W.make_workload("window_4k", seed=0)
    L, Wd, Hq, D = 2048, 64, 16, 80
    assert bench.pairs_per_row(case).sum() == Hq * 2 * (L * (2 * Wd + 1) - Wd * (Wd + 1))   # 520,064 per head
    q_o = 2 * 4096 * Hq * D * 2          # q read, out written (bf16)
    k_v = 2 * 4096 * Hq * D * 2          # every key row once (Hkv = Hq)
    lse = Hq * 4096 * 4
    meta = 3 * 4 + Hq * 4                # cu_seqlens, sinks
    assert bench.algorithmic_bytes(case) == q_o + k_v + lse + meta == 42_205_260


def test_window_16k_pairs_closed_form():
    case = W.make_workload("window_16k", seed=0)
    lens = np.diff(case["cu_seqlens"])
    per_head = sum(int(n) * int(n) if n <= 64 else int(n) * 129 - 64 * 65 for n in lens)
    assert bench.pairs_per_row(case).sum() == 16 * per_head


def test_mla_topk_pairs_are_valid_entries_times_heads():
    case = W.make_workload("mla_topk", seed=0)
    idx = case["topk_idx"]
    assert bench.pairs_per_row(case).sum() == 64 * int(((idx >= 0) & (idx < 65536)).sum())


def test_blocksparse_32k_pairs_on_sampled_rows():
    case = W.make_workload("blocksparse_32k", seed=0)
    got = bench.pairs_per_row(case)
    g = np.random.default_rng(0)
    for i in g.choice(case["q"].shape[0], size=40, replace=False):
        want = sum(P.closed_form_count(case, int(i), h) for h in range(32))
        assert got[i] == want, int(i)


def test_bench_refuses_more_than_one_gpu(capsys):
    """One GPU only: --gpus above 1 exits with status 2 and says why."""
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_extra_compiler_options_name_existing_sources():
    """Per-source compiler options apply only to files that exist, so a
    renamed kernel source cannot silently lose its options."""
    import os
    import __graft_entry__ as g
    for name, flags in g.EXTRA_FLAGS.items():
        assert os.path.exists(os.path.join(g.CSRC, name)), name
        assert flags and all(isinstance(f, str) for f in flags)


def test_traffic_record_is_keyed_to_source_and_options(monkeypatch):
    """The committed PMC traffic of a kernel is used only for the source and
    the compiler options it was measured on."""
    import __graft_entry__ as g
    base = bench.kernel_hash("blocksel")
    monkeypatch.setitem(g.EXTRA_FLAGS, "blocksel_fwd.hip", ["-O2"])
    assert bench.kernel_hash("blocksel") != base
    monkeypatch.delitem(g.EXTRA_FLAGS, "blocksel_fwd.hip")
    assert bench.kernel_hash("blocksel") != base
