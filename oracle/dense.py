"""Dense fp64 twin of the sink-aware masked attention oracle (NumPy).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library or with ``oracle/ref.c``.

Where ``ref.c`` enumerates each row's valid keys, this twin builds the whole
``[R, Tk]`` logit matrix per head and turns every part of the method into an
explicit matrix: a boolean mask over all keys, an additive bias column for each
segment's first key (``key0_bias``), and an appended "null" key with logit
``sinks[h]`` and an all-zero value row (``null_logit``).  A textbook softmax
over that augmented row then gives the output; the LSE is taken over the
selected keys only.  Sources:

* ``key0_bias`` -- "[Bugfix][MiMo] Apply vision attention sinks in the window
  attention path", closed-form correction paragraph: a per-head bias on key 0
  of every sequence, applied after scaling (the closed form multiplies key 0's
  weight by exp(s)).
* window -- same page: symmetric window inside each cu_seqlens sequence; the
  bound is inclusive (rows 0 .. W of a sequence, W + 1 of them, reach key 0).
* ``null_logit`` -- "Apply DeepSeek-V4 attn_sink in the XPU sparse-MLA Triton
  kernel", Implementation paragraph: the sink joins the softmax denominator,
  the returned LSE covers the selected keys only; top-k lists use -1 padding.
* block selection -- "cp_sparse_attn" API page: selected key blocks
  (kv_idx // block_size) combined with token causality and same-document masks;
  fully masked rows give a zero output (``_local_sparse_forward``); their LSE
  is -inf, the log of an empty sum.

The small helpers below are the seams the oracle's own tests use to plant
mistakes and check that the pins catch them.  Only for small inputs (O(R * Tk)
memory per head) and for sampled rows.
"""
from __future__ import annotations

import numpy as np

MASK_KINDS = ("window", "topk", "blocksel")
SINK_MODES = ("none", "key0_bias", "null_logit")


def segment_ids(cu_seqlens, n: int) -> np.ndarray:
    """Segment index of each of the n packed tokens (-1 if outside every segment)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seg = np.full(n, -1, dtype=np.int64)
    for s in range(len(cu) - 1):
        seg[cu[s]:cu[s + 1]] = s
    return seg


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Grouped-query mapping: consecutive groups of Hq/Hkv query heads share a kv head."""
    return h // (Hq // Hkv)


def window_keep(i: np.ndarray, j: np.ndarray, W: int) -> np.ndarray:
    return np.abs(i - j) <= W


def key_mask(mask_kind: str, rows: np.ndarray, h: int, Tk: int, Hq: int, *,
             cu_seqlens=None, window=None, topk_idx=None, block_sel=None,
             block_size=None) -> np.ndarray:
    """Boolean [len(rows), Tk] matrix: entry (r, j) is True iff key j is in S(rows[r], h)."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(Tk, dtype=np.int64)
    if mask_kind == "window":
        seg = segment_ids(cu_seqlens, Tk)
        same = (seg[rows][:, None] == seg[None, :]) & (seg[rows][:, None] >= 0)
        return same & window_keep(rows[:, None], j[None, :], int(window))
    if mask_kind == "topk":
        idx = np.asarray(topk_idx, dtype=np.int64)[rows]
        m = np.zeros((len(rows), Tk), dtype=bool)
        for r in range(len(rows)):
            sel = idx[r][(idx[r] >= 0) & (idx[r] < Tk)]
            m[r, sel] = True
        return m
    if mask_kind == "blocksel":
        bs = np.asarray(block_sel)
        hidx = kv_head(h, Hq, bs.shape[1])
        seg = segment_ids(cu_seqlens, Tk)
        blk = bs[0, hidx][rows][:, j // int(block_size)] != 0
        causal = j[None, :] <= rows[:, None]
        same = (seg[rows][:, None] == seg[None, :]) & (seg[rows][:, None] >= 0)
        return blk & causal & same
    raise ValueError(f"unknown mask kind {mask_kind!r}")


def key0_columns(cu_seqlens, Tk: int) -> np.ndarray:
    """Boolean [Tk]: True at the first key of every cu_seqlens segment."""
    first = np.zeros(Tk, dtype=bool)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for s in range(len(cu) - 1):
        if cu[s] < cu[s + 1]:
            first[cu[s]] = True
    return first


def key0_bias_value(sink: float, scale: float) -> float:
    """The sink is added to the already-scaled logit, unscaled."""
    return float(sink)


def selected_lse(sel_logits: np.ndarray, sink_logit) -> float:
    """Natural-log LSE over the selected keys only; the null sink never enters it."""
    ms = sel_logits.max()
    return float(ms + np.log(np.exp(sel_logits - ms).sum()))


def attn_dense(q, k, v, *, mask_kind: str, scale: float, cu_seqlens=None,
               window=None, topk_idx=None, block_sel=None, block_size=None,
               sinks=None, sink_mode: str = "none", rows=None):
    """Return (out[len(rows), Hq, Dv], lse[Hq, len(rows)]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, _ = q.shape
    Tk, Hkv, _ = k.shape
    Dv = v.shape[2]
    if sink_mode not in SINK_MODES:
        raise ValueError(sink_mode)
    if sink_mode == "key0_bias" and mask_kind == "topk":
        raise ValueError("key0_bias needs cu_seqlens segments; a top-k list has none")
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), Hq, Dv))
    lse = np.full((Hq, len(rows)), -np.inf)
    first = key0_columns(cu_seqlens, Tk) if sink_mode == "key0_bias" else None
    for h in range(Hq):
        kv = kv_head(h, Hq, Hkv)
        mask = key_mask(mask_kind, rows, h, Tk, Hq, cu_seqlens=cu_seqlens, window=window,
                        topk_idx=topk_idx, block_sel=block_sel, block_size=block_size)
        logits = scale * (q[rows, h, :] @ k[:, kv, :].T)                  # [R, Tk]
        if sink_mode == "key0_bias":
            bias = key0_bias_value(float(sinks[h]), scale)
            logits = logits + np.where(first, bias, 0.0)[None, :]
        logits = np.where(mask, logits, -np.inf)
        vals = v[:, kv, :]                                                 # [Tk, Dv]
        sink_logit = None
        if sink_mode == "null_logit":
            sink_logit = float(sinks[h])
            null = np.full((len(rows), 1), sink_logit)
            aug = np.concatenate([logits, null], axis=1)                   # [R, Tk+1]
            vals = np.concatenate([vals, np.zeros((1, Dv))], axis=0)       # [Tk+1, Dv]
        else:
            aug = logits
        for r in range(len(rows)):
            if not mask[r].any():
                continue                                                   # out 0, lse -inf
            lse[h, r] = selected_lse(logits[r][mask[r]], sink_logit)
            a = aug[r]
            am = a[np.isfinite(a)].max()
            w = np.exp(a - am)                                             # exp(-inf) = 0
            out[r, h, :] = (w / w.sum()) @ vals
    return out, lse
