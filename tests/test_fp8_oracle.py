"""Pins for the fp8 decode oracle (oracle/fp8.py): the e4m3 decoder against
values the OCP 8-bit format's definition fixes by hand and against torch's
independent float8_e4m3fn type on all 256 codes, and the dequantized decode
against the bf16 top-k oracle where the two must agree exactly."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import workloads as W
from oracle import fp8


def test_e4m3_hand_values():
    cases = {0x00: 0.0, 0x80: -0.0, 0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0xFE: -448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x30: 0.5, 0x77: 240.0}
    for code, want in cases.items():
        got = float(fp8.e4m3_to_float([code])[0])
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (hex(code), got, want)
    assert np.isnan(fp8.e4m3_to_float([0x7F, 0xFF])).all()
    finite = fp8.e4m3_to_float(np.arange(256))
    assert np.nanmax(np.abs(finite)) == 448.0 and np.isnan(finite).sum() == 2


def test_e4m3_against_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = fp8.e4m3_to_float(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(mine[~np.isnan(mine)]), np.signbit(ref[~np.isnan(ref)]))


def test_decode_matches_topk_oracle_on_dequantized_cache():
    """The fp8 decode is the top-k attention over the dequantized cache: with
    the cache's values handed to the bf16-path oracle directly, the two agree
    bit for bit; a wrong scale (per row, not applied) does not."""
    case = W.mla_decode_fp8_case(6, 300, 64, 64, counts=(1, 7, 64), shuffled=True, seed=3)
    o1, l1 = fp8.decode_ref(case)
    k = fp8.dequantize(case["kv_fp8"], case["kv_scale"]).astype(np.float32)
    o2, l2 = oracle.attn_ref(case["q"], k, k[:, :, :512], mask_kind="topk", scale=case["scale"],
                             topk_idx=case["topk_idx"], sinks=case["sinks"], sink_mode="null_logit")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    kb = fp8.e4m3_to_float(case["kv_fp8"]).astype(np.float32)   # scale forgotten
    o3, _ = oracle.attn_ref(case["q"], kb, kb[:, :, :512], mask_kind="topk", scale=case["scale"],
                            topk_idx=case["topk_idx"], sinks=case["sinks"], sink_mode="null_logit")
    assert not np.allclose(o1, o3, rtol=1e-3, atol=1e-6)
