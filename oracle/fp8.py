"""CPU oracle for the sparse-MLA decode over an fp8 latent cache: TEST
INFRASTRUCTURE.  Only ``tests/`` and the CPU-baseline leg of ``bench.py`` may
use it; it shares no code with the HIP library.

* :func:`e4m3_to_float` -- the OCP 8-bit e4m3 encoding decoded from its
  definition: sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 is subnormal (m / 8 * 2^-6); S.1111.111 is NaN (there is
  no infinity), so the largest finite magnitude is 1.75 * 2^8 = 448.
* :func:`decode_ref` -- the decode's plain definition: every cache row
  dequantized as e4m3(byte) * kv_scale[row] (exact in fp64), then the top-k
  masked softmax with the null-logit sink of :func:`oracle.attn_ref`
  (DeepSeek-V4 sparse-MLA page: the sink joins the denominator only, the LSE
  covers the selected keys), V = the first 512 of the 576 values.
"""
from __future__ import annotations

import numpy as np


def e4m3_to_float(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def dequantize(kv_fp8, kv_scale) -> np.ndarray:
    """[Tk, 1, 576] bytes and [Tk] scales -> fp64 values."""
    return e4m3_to_float(kv_fp8) * np.asarray(kv_scale, dtype=np.float64)[:, None, None]


def decode_ref(case: dict, rows=None):
    from . import attn_ref
    k = dequantize(case["kv_fp8"], case["kv_scale"])
    # every dequantized value is exact in fp32 (at most 12 significant bits)
    k32 = k.astype(np.float32)
    assert np.array_equal(k32.astype(np.float64), k), "dequantized cache not exact in fp32"
    return attn_ref(case["q"], k32, k32[:, :, :512], mask_kind="topk", scale=case["scale"],
                    topk_idx=case["topk_idx"], sinks=case["sinks"], sink_mode=case["sink_mode"], rows=rows)
