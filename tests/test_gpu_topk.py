"""GPU parity of the top-k mask over a shared latent KV (bf16 sparse-MLA
instance, and the f32 instance) against the CPU oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest

import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BUCKETS = (1, 4, 16, 128, 512, 2048)


def bucket_rows(case, per_bucket=24, seed=0):
    n = (case["topk_idx"] >= 0).sum(1)
    g = np.random.default_rng(seed)
    rows = []
    for c in np.unique(n):
        cand = np.flatnonzero(n == c)
        rows += g.choice(cand, size=min(per_bucket, len(cand)), replace=False).tolist()
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mla_topk_full_size(seed):
    """The sparse-MLA workload at full size (4096 rows x 64 heads, 65536-entry
    latent KV, top-k 2048), in the launch configuration the benchmark times;
    seed 0 on every row, seeds 1 and 2 on rows sampled from every valid-count
    bucket; errors reported per bucket."""
    case = W.make_workload("mla_topk", seed=seed)
    rows = np.arange(case["q"].shape[0]) if seed == 0 else bucket_rows(case, seed=seed)
    out, lse = G.gpu_run(case)
    ref_o, ref_l = G.oracle_run(case, rows=rows)
    n = (case["topk_idx"][rows] >= 0).sum(1)
    worst = 0.0
    for c in np.unique(n):
        sel = n == c
        rel, dl = G.compare(out[rows][sel], lse[:, rows][:, sel], ref_o[sel], ref_l[:, sel])
        G.say(f"[mla seed{seed}] valid keys {c:5d} ({int(sel.sum())} rows): max rel L2 {rel:.3e}, "
              f"tensor rel L2 {G.tensor_rel_l2(out[rows][sel], ref_o[sel]):.3e}, lse max abs {dl:.3e}")
        assert rel <= G.BF16_REL_L2 and dl <= G.BF16_LSE_ABS
        worst = max(worst, rel)
    assert set(np.unique(n).tolist()) == set(BUCKETS)


def small_mla(seed=0, T=96, Tk=3000, Hq=64, topk=256, **kw):
    return W.topk_case(T, Tk, Hq, 576, 512, topk, counts=kw.pop("counts", (0, 1, 5, 31, 32, 33, 100, 256)),
                       seed=seed, **kw)


@pytest.mark.parametrize("variant", ["front", "shuffled", "out_of_range", "no_sink", "hq128"])
def test_mla_small_variants(variant):
    kw = {"front": {}, "shuffled": {"shuffled": True}, "out_of_range": {"shuffled": True, "out_of_range": True},
          "no_sink": {"sink_mode": "none"}, "hq128": {"Hq": 128}}[variant]
    seed = {"front": 10, "shuffled": 11, "out_of_range": 12, "no_sink": 13, "hq128": 14}[variant]
    case = small_mla(seed=seed, **kw)
    G.assert_parity(case, label=f"mla small {variant}")


def test_mla_long_list_multiple_chunks():
    """topk larger than one compaction pass (2048 entries), -1 interleaved."""
    case = W.topk_case(20, 9000, 64, 576, 512, 5000, counts=(0, 7, 2047, 2048, 2049, 5000), shuffled=True, seed=3)
    G.assert_parity(case, label="mla topk=5000")


def test_mla_noop_and_differs_on_short_rows():
    import torch
    case = small_mla(seed=4)
    o0, l0 = G.gpu_run(case, sink_mode="none", sinks=None)
    ninf = torch.full((64,), -math.inf, dtype=torch.float32, device="cuda:0")
    o1, l1 = G.gpu_run(case, sink_mode="null_logit", sinks=ninf)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    o2, l2 = G.gpu_run(case)
    n = (case["topk_idx"] >= 0).sum(1)
    short = (n >= 1) & (n <= 5)
    assert np.array_equal(l2, l0)  # the LSE covers the selected keys only
    d = np.abs(o2[short] - o0[short]).max(axis=2)
    assert np.all(d > 0)


def test_mla_count_and_membership_probes():
    import torch  # noqa: F401
    case = small_mla(seed=5, T=40, Tk=700, topk=64, counts=(0, 1, 2, 17, 64), shuffled=True, out_of_range=True)
    q0 = np.zeros_like(case["q"])
    _, lse = G.gpu_run(dict(case, q=q0), sink_mode="none", sinks=None)
    idx = case["topk_idx"]
    n = ((idx >= 0) & (idx < 700)).sum(1)
    for i in range(40):
        if n[i] == 0:
            assert np.all(np.isneginf(lse[:, i]))
        else:
            assert np.all(np.rint(np.exp(lse[:, i])) == n[i]), i
    probes = sorted(set(idx[(idx >= 0) & (idx < 700)].ravel().tolist()[:40]) | {0, 1, 699})
    for j in probes:
        kv = np.zeros_like(case["k"])
        kv[j, 0, 0] = 1.0
        out, _ = G.gpu_run(dict(case, q=q0, k=kv, v=kv[:, :, :512]), sink_mode="none", sinks=None)
        got = out[:, :, 0] != 0
        want = np.any(idx == j, axis=1)
        assert np.array_equal(got, np.repeat(want[:, None], 64, axis=1)), j


def test_topk_f32_instance():
    case = W.topk_case(30, 200, 8, 64, 48, 40, counts=(0, 1, 3, 40), shuffled=True, mla=False, Hkv=2,
                       std=1.0, dtype="f32", sink_mode="null_logit", seed=6, out_of_range=True)
    G.assert_parity(case, label="f32 topk GQA")
    mla32 = W.topk_case(12, 300, 64, 576, 512, 50, counts=(1, 9, 50), dtype="f32", seed=7)
    G.assert_parity(mla32, label="f32 topk MLA")


def test_mla_latent_rows_past_2_31():
    """The shared latent KV is a strided view with a 4 MB row stride, so every
    entry from row 1024 on starts 2**31 elements (4 GiB) or more into the
    allocation; the gathers are correct only with 64-bit row offsets.  The top-k lists favour
    those high rows (DeepSeek-V4 sparse-MLA page: indices address one shared
    latent cache)."""
    import torch
    case = W.topk_case(24, 3000, 64, 576, 512, 256, counts=(1, 17, 256), shuffled=True, seed=8)
    idx = case["topk_idx"]
    g = np.random.default_rng(8)
    for i in range(idx.shape[0]):                     # distinct rows >= 1024 in the same slots
        slots = np.flatnonzero(idx[i] >= 0)
        idx[i, slots] = g.choice(np.arange(1024, 3000), size=len(slots), replace=False)
    stride = 1 << 21                                  # elements: 4 MB per latent row
    assert 1024 * stride >= 2 ** 31
    big = torch.zeros(3000 * stride, dtype=torch.bfloat16, device="cuda:0")
    kv = big.as_strided((3000, 1, 576), (stride, 576, 1))
    kv.copy_(torch.from_numpy(case["k"]).to(torch.bfloat16))
    out, lse = G.gpu_run(case, k=kv, v=kv[:, :, :512])
    ref_o, ref_l = G.oracle_run(case)
    rel, dl = G.compare(out, lse, ref_o, ref_l)
    G.say(f"[mla >2^31 row offsets] rel {rel:.3e} lse {dl:.3e}")
    assert rel <= G.BF16_REL_L2 and dl <= G.BF16_LSE_ABS
    del big, kv
    torch.cuda.empty_cache()
