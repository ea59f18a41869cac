"""GPU parity with large logits (scale far above 1/sqrt(D)): the running max
of the online softmax then moves many times along a row, so every lazy
rescale of the accumulators and of the row sum is exercised, and the softmax
is nearly one-hot.  The oracle (fp64, the plain definition) needs no max
tracking at all, so a rescale applied twice, skipped or applied to the wrong
state shows up as a parity failure."""
from __future__ import annotations

import pytest

import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("scale", [1.0, 4.0])
@pytest.mark.parametrize("sink", ["key0_bias", "null_logit"])
def test_window_large_logits(scale, sink):
    case = W.window_case([700, 50, 333], 8, 2, 80, 64, dtype="bf16", sink_mode=sink, sink_range=(-2, 2),
                         scale=scale, seed=41)
    G.assert_parity(case, label=f"window scale={scale} {sink}")


@pytest.mark.parametrize("scale", [1.0, 3.0])
def test_mla_large_logits(scale):
    case = W.topk_case(48, 5000, 64, 576, 512, 2048, counts=(1, 16, 512, 2048), shuffled=True, scale=scale, seed=42)
    G.assert_parity(case, label=f"mla scale={scale}")


@pytest.mark.parametrize("scale", [1.0, 3.0])
def test_blocksel_large_logits(scale):
    case = W.blocksel_case([900, 400], 8, 2, 128, n_random=8, Hidx=2, sink_mode="null_logit", scale=scale, seed=43)
    G.assert_parity(case, label=f"blocksel scale={scale}")
