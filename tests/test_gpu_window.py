"""GPU parity of the window mask (bf16 MFMA instance and the f32 instance)
against the CPU oracle, plus bitwise self-checks and mask probes."""
from __future__ import annotations

import math

import numpy as np
import pytest

import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_window_f32(seed):
    G.assert_parity(W.make_workload("tiny_window_f32", seed=seed), label=f"tiny_window_f32 seed{seed}")


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("variant", ["base", "wide_sinks", "gqa"])
def test_window_4k(seed, variant):
    kw = {"base": {}, "wide_sinks": {"sink_range": (-2.0, 2.0)}, "gqa": {"gqa": True}}[variant]
    case = W.make_workload("window_4k", seed=seed, **kw)
    G.assert_parity(case, label=f"window_4k {variant} seed{seed}")


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("sink", ["key0_bias", "none"])
def test_window_16k(seed, sink):
    """16384-token window workload: seed 0 on every row, seeds 1 and 2 on
    sampled rows (segment ends included)."""
    case = W.make_workload("window_16k", seed=seed, sink_mode=sink)
    rows = None if seed == 0 else G.sample_rows(case, 3000, seed=seed)
    G.assert_parity(case, rows=rows, label=f"window_16k {sink} seed{seed}")


EDGE = [
    # (seqlens, Hq, Hkv, D, W, sink)
    ([37], 4, 4, 64, 0, "key0_bias"),                 # W = 0: every row sees only itself
    ([50, 3, 80], 2, 1, 64, 1 << 20, "key0_bias"),    # W >= T: full bidirectional per sequence
    ([1, 1, 1, 5], 4, 2, 80, 3, "null_logit"),        # single-token sequences
    ([0, 70, 0, 61, 0], 8, 2, 96, 8, "key0_bias"),    # empty segments in cu_seqlens
    ([130, 65, 64, 63, 200], 16, 4, 128, 64, "null_logit"),  # tiles straddling sequences
    ([333], 1, 1, 80, 17, "none"),                    # one head, ragged tail tile
    ([64, 64], 16, 16, 80, 64, "key0_bias"),          # exactly one tile per sequence
    ([2047, 3, 70], 8, 1, 64, 100, "null_logit"),     # MQA, W larger than a tile
    ([50, 3, 200], 4, 2, 80, 2 ** 31 - 1, "key0_bias"),  # W = INT32_MAX: unbounded window, no int32 wrap
]


@pytest.mark.parametrize("idx", range(len(EDGE)))
def test_window_edges(idx):
    lens, Hq, Hkv, D, Wd, sink = EDGE[idx]
    case = W.window_case(lens, Hq, Hkv, D, Wd, dtype="bf16", sink_mode=sink, sink_range=(-2, 2), seed=idx)
    G.assert_parity(case, label=f"edge{idx} lens={lens} Hq={Hq} Hkv={Hkv} D={D} W={Wd} {sink}")


@pytest.mark.parametrize("D", [64, 80, 128])
def test_window_f32_instance_matches_oracle(D):
    case = W.window_case([40, 100, 7], 4, 2, D, 9, dtype="f32", sink_mode="null_logit",
                         sink_range=(-2, 2), seed=D)
    G.assert_parity(case, label=f"f32 window D={D}")


def test_noop_sinks_bitwise():
    """key0_bias with s = 0 and null_logit with s = -inf equal the no-sink
    result bit for bit on the GPU."""
    import torch
    case = W.make_workload("window_4k", seed=0)
    base_o, base_l = G.gpu_run(case, sink_mode="none", sinks=None)
    z = torch.zeros(16, dtype=torch.float32, device="cuda:0")
    o, l = G.gpu_run(case, sink_mode="key0_bias", sinks=z)
    assert np.array_equal(o, base_o) and np.array_equal(l, base_l)
    ninf = torch.full((16,), -math.inf, dtype=torch.float32, device="cuda:0")
    o, l = G.gpu_run(case, sink_mode="null_logit", sinks=ninf)
    assert np.array_equal(o, base_o) and np.array_equal(l, base_l)


def test_only_first_w_plus_1_rows_change():
    case = W.make_workload("window_16k", seed=1)
    o0, l0 = G.gpu_run(case, sink_mode="none", sinks=None)
    o1, l1 = G.gpu_run(case)
    cu, Wd = case["cu_seqlens"], case["window"]
    seg_start = np.repeat(cu[:-1], np.diff(cu))
    affected = (np.arange(len(seg_start)) - seg_start) <= Wd
    assert np.array_equal(o1[~affected], o0[~affected])
    assert np.array_equal(l1[:, ~affected], l0[:, ~affected])
    assert np.all(np.any(l1[:, affected] != l0[:, affected], axis=0))


def test_count_probe_exact():
    """Q = 0: every selected logit is 0, so lse = ln |S(i,h)| and exp(lse)
    recovers the window size of every row exactly."""
    case = W.window_case([130, 1, 7, 300, 64], 4, 2, 80, 37, dtype="bf16", sink_mode="none", seed=4)
    q0 = np.zeros_like(case["q"])
    c0 = dict(case, q=q0)
    _, lse = G.gpu_run(c0)
    cu, Wd = case["cu_seqlens"], case["window"]
    for s in range(len(cu) - 1):
        for i in range(cu[s], cu[s + 1]):
            n = min(i + Wd, cu[s + 1] - 1) - max(i - Wd, cu[s]) + 1
            assert np.all(np.rint(np.exp(lse[:, i])) == n), (i, np.exp(lse[:, i]), n)


def test_membership_probe():
    """Q = 0 and a one-hot V (row j* = 1, all other rows 0): out[i, h, 0] != 0
    exactly when key j* is in the window of row i.  Swept over sequence
    boundaries and window edges."""
    import torch
    lens, Wd = [70, 5, 90], 6
    case = W.window_case(lens, 2, 1, 64, Wd, dtype="bf16", sink_mode="none", seed=9)
    cu = case["cu_seqlens"]
    T = int(cu[-1])
    q0 = np.zeros_like(case["q"])
    probes = set()
    for s in range(len(cu) - 1):
        for base in (cu[s], cu[s + 1] - 1):
            for d in range(-Wd - 2, Wd + 3):
                if 0 <= base + d < T:
                    probes.add(int(base + d))
    probes |= {35, 36, 100, 140}
    seg = np.repeat(np.arange(len(lens)), lens)
    for j in sorted(probes):
        v = np.zeros_like(case["v"])
        v[j] = 1.0
        out, _ = G.gpu_run(dict(case, q=q0, v=v))
        got = out[:, :, 0] != 0
        i = np.arange(T)
        want = (seg == seg[j]) & (np.abs(i - j) <= Wd)
        assert np.array_equal(got, np.repeat(want[:, None], 2, axis=1)), j


def test_window_kv_rows_past_2_31():
    """K and V are strided views with a 16 MB token stride, so every key row
    from token 128 on starts past byte 2**31 of its allocation: the band loads
    are correct only with 64-bit row offsets."""
    import torch
    case = W.window_case([120, 180], 4, 2, 80, 16, dtype="bf16", sink_mode="key0_bias", sink_range=(-2, 2),
                         seed=21)
    T, Hkv, D = case["k"].shape
    stride = (1 << 23) + 64                            # elements per token row
    assert 128 * stride * 2 > 2 ** 31

    def strided(a):
        big = torch.zeros(T * stride, dtype=torch.bfloat16, device="cuda:0")
        view = big.as_strided((T, Hkv, D), (stride, D, 1))
        view.copy_(torch.from_numpy(a).to(torch.bfloat16))
        return big, view

    kb, k = strided(case["k"])
    vb, v = strided(case["v"])
    out, lse = G.gpu_run(case, k=k, v=v)
    ref_o, ref_l = G.oracle_run(case)
    rel, dl = G.compare(out, lse, ref_o, ref_l)
    G.say(f"[window >2^31 row offsets] rel {rel:.3e} lse {dl:.3e}")
    assert rel <= G.BF16_REL_L2 and dl <= G.BF16_LSE_ABS
    del kb, vb, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_unbounded_int32_max(dtype):
    """An 'unbounded' window W = 2^31 - 1 on both instances equals full
    attention within each sequence (the library clamps W to T; row +- W never
    wraps in int32)."""
    case = W.window_case([50, 3, 200, 1], 4, 2, 64, 2 ** 31 - 1, dtype=dtype, sink_mode="null_logit",
                         sink_range=(-2, 2), seed=11)
    G.assert_parity(case, label=f"window W=INT32_MAX {dtype}")
