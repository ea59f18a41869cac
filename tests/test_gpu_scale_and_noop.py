"""GPU checks of the scale handling and of the no-op sinks across the bf16
kernels.

The kernels keep the dot products raw and apply the softmax scale inside the
exponent, which needs a positive factor: a negative scale is moved into Q's
sign and a zero scale is replaced by the least normal float.  Both must still
match the oracle, which applies the scale as written.  The no-op sinks
(key0_bias with s = 0, null_logit with s = -inf) must give the no-sink result
bit for bit on every mask kind (MiMo window-attention page: the bias only
touches key 0; DeepSeek-V4 sparse-MLA page: a -inf sink drops out of the
fold)."""
from __future__ import annotations

import math

import numpy as np
import pytest

import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [64, 80, 96, 128])
@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_window_scale_sign_and_zero(D, scale):
    case = W.window_case([300, 41, 200], 4, 2, D, 64, dtype="bf16", sink_mode="key0_bias",
                         sink_range=(-2, 2), seed=D, scale=scale)
    G.assert_parity(case, label=f"window D={D} scale={scale}")


@pytest.mark.parametrize("scale", [-1.0 / 24.0, 0.0])
def test_mla_scale_sign_and_zero(scale):
    case = W.topk_case(96, 3000, 64, 576, 512, 256, counts=(1, 16, 100, 256), seed=5, scale=scale)
    G.assert_parity(case, label=f"mla scale={scale}")


@pytest.mark.parametrize("scale", [-0.0884, 0.0])
def test_blocksel_scale_sign_and_zero(scale):
    case = W.blocksel_case([300, 190], 8, 2, 128, n_random=3, sink_mode="key0_bias", seed=21, scale=scale)
    G.assert_parity(case, label=f"blocksel scale={scale}")


def _noop_bitwise(case, Hq):
    import torch
    base_o, base_l = G.gpu_run(case, sink_mode="none", sinks=None)
    z = torch.zeros(Hq, dtype=torch.float32, device="cuda:0")
    o, l = G.gpu_run(case, sink_mode="key0_bias", sinks=z)
    assert np.array_equal(o, base_o) and np.array_equal(l, base_l)
    ninf = torch.full((Hq,), -math.inf, dtype=torch.float32, device="cuda:0")
    o, l = G.gpu_run(case, sink_mode="null_logit", sinks=ninf)
    assert np.array_equal(o, base_o) and np.array_equal(l, base_l)


def test_blocksel_noop_sinks_bitwise():
    case = W.blocksel_case([700, 390, 300], 16, 4, 128, n_random=5, sink_mode="key0_bias", seed=22)
    _noop_bitwise(case, 16)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_window_noop_sinks_bitwise_other_dims(D):
    case = W.window_case([500, 31, 600], 8, 2, D, 64, dtype="bf16", sink_mode="key0_bias", seed=D + 1)
    _noop_bitwise(case, 8)
