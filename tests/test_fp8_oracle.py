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


def _golden_dequant():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "fp8_dequant.json")
    return json.load(open(path))["cases"]


def _check_fixtures(dequantize_fn) -> bool:
    """True iff dequantize_fn reproduces every hand-worked (byte, row scale)
    value, sign of zero included."""
    for c in _golden_dequant():
        b = np.array([[[int(c["byte"], 16)]]], dtype=np.uint8)
        got = float(dequantize_fn(b, np.array([c["scale"]], dtype=np.float32))[0, 0, 0])
        if got != c["value"] or math.copysign(1, got) != math.copysign(1, c["value"]):
            return False
    return True


def test_dequantize_hand_worked_fixtures():
    """Per-row scaling pinned to values worked by hand (tests/golden/fp8_dequant.json):
    value = e4m3(byte) * scale[row].  Plausible wrong conventions fail it."""
    assert _check_fixtures(fp8.dequantize)
    divide = lambda b, s: fp8.e4m3_to_float(b) / np.asarray(s, dtype=np.float64)[:, None, None]
    assert not _check_fixtures(divide), "dividing by the row scale must fail the fixtures"
    forget = lambda b, s: fp8.e4m3_to_float(b) + 0.0 * np.asarray(s, dtype=np.float64)[:, None, None]
    assert not _check_fixtures(forget), "ignoring the row scale must fail the fixtures"


def test_dequantize_within_half_ulp_of_source_rows():
    """The generator rounds fp32 rows x to e4m3 after dividing by the row scale
    (round to nearest even); dequantizing must land within half an e4m3 unit in
    the last place of x / scale, times the scale, of x.  A divide-by-scale or a
    transposed scale (wrong row) lands far outside it."""
    case = W.mla_decode_fp8_case(2, 512, 64, 16, counts=(16,), seed=5)
    x = case["kv_source"].astype(np.float64)                    # [Tk, 576]
    sc = case["kv_scale"].astype(np.float64)[:, None]
    y = np.abs(x / sc)
    assert y.max() <= 448.0
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))             # exponent; subnormal range has e = -6
    half_ulp = 0.5 * np.exp2(e - 3) * sc                          # 3 mantissa bits
    err = np.abs(fp8.dequantize(case["kv_fp8"], case["kv_scale"])[:, 0, :] - x)
    assert np.all(err <= half_ulp * (1 + 1e-12)), float((err / half_ulp).max())
    wrong = fp8.e4m3_to_float(case["kv_fp8"])[:, 0, :] / sc
    assert not np.all(np.abs(wrong - x) <= half_ulp)
    shifted = fp8.e4m3_to_float(case["kv_fp8"])[:, 0, :] * np.roll(sc, 1, axis=0)
    assert not np.all(np.abs(shifted - x) <= half_ulp)
