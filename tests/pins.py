"""Pins for the CPU oracle: checks against facts the source pages and plain
mathematics fix, written so that each takes the oracle implementation as an
argument.  ``test_oracle_pins.py`` runs them against both oracle
implementations, and against deliberately broken copies of the dense one to
show that every planted mistake fails at least one pin.

Sources for what is pinned:
* "[Bugfix][MiMo] Apply vision attention sinks in the window attention path":
  the key-0 closed form p0 = exp(logit0 - lse), out' = (out + p0 (e^s - 1) v0)
  / (1 + p0 (e^s - 1)); the rows that reach key 0 are a sequence's first W + 1
  (so only they change); a null-logit sink is a different operation.
* "Apply DeepSeek-V4 attn_sink in the XPU sparse-MLA Triton kernel": the sink
  joins the softmax denominator only, the LSE covers the selected keys only,
  a sink of -inf is a no-op, and short rows must differ from the no-sink result.
* "cp_sparse_attn" API page: document ids are cumsum(positions == 0) - 1;
  block-selection table offsets must not wrap at 2**31 elements.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import workloads as W


def oracle_kwargs(case: dict, **over) -> dict:
    kw = dict(mask_kind=case["mask_kind"], scale=case["scale"], cu_seqlens=case["cu_seqlens"],
              window=case["window"], topk_idx=case["topk_idx"], block_sel=case["block_sel"],
              block_size=case["block_size"], sinks=case["sinks"], sink_mode=case["sink_mode"])
    kw.update(over)
    return kw


def run(fn, case: dict, q=None, k=None, v=None, **over):
    return fn(case["q"] if q is None else q, case["k"] if k is None else k,
              case["v"] if v is None else v, **oracle_kwargs(case, **over))


# ---------------------------------------------------------------- tiny cases
def tiny_cases(seed: int = 0) -> list[dict]:
    """Small seeded cases covering every mask kind, GQA, ragged segments,
    degenerate windows, -1 anywhere in top-k lists, out-of-range indices,
    empty rows, and blocks that straddle documents."""
    cs = []
    for W_, lens in ((0, [7, 3]), (1, [9, 1, 6]), (3, [5, 23, 12]), (1 << 20, [11, 17])):
        cs.append(W.window_case(lens, 4, 2, 16, W_, dtype="f32", sink_mode="key0_bias",
                                sink_range=(-2, 2), seed=seed, name=f"win{W_}"))
    cs.append(W.window_case([6, 25], 2, 2, 8, 4, dtype="f32", sink_mode="null_logit",
                            sink_range=(-2, 2), seed=seed + 1, Dv=12, name="win_null"))
    cs.append(W.topk_case(12, 40, 4, 16, 16, 9, counts=(0, 1, 3, 9), shuffled=True, mla=False, Hkv=2,
                          std=1.0, dtype="f32", sink_mode="null_logit", seed=seed, out_of_range=True,
                          name="topk_gqa"))
    cs.append(W.topk_case(10, 33, 4, 24, 16, 6, counts=(1, 2, 6), shuffled=False, mla=True,
                          std=1.0, dtype="f32", sink_mode="null_logit", seed=seed + 2, name="topk_mla"))
    cs.append(W.blocksel_case([13, 30, 21], 4, 2, 16, block_size=4, n_random=3, Hidx=2, dtype="f32",
                              sink_mode="null_logit", seed=seed, name="bsel4"))
    cs.append(W.blocksel_case([9, 19], 4, 4, 8, block_size=8, n_random=1, Hidx=2, dtype="f32",
                              sink_mode="key0_bias", seed=seed + 3, name="bsel8"))
    return cs


# ------------------------------------------------- independent constructions
def loop_mask(case: dict, h: int) -> np.ndarray:
    """Membership built with explicit loops (a different construction from
    both oracle implementations): [T, Tk] bool for query head h."""
    q, k = case["q"], case["k"]
    T, Hq, _ = q.shape
    Tk = k.shape[0]
    m = np.zeros((T, Tk), dtype=bool)
    kind = case["mask_kind"]
    if kind == "window":
        cu, Wd = case["cu_seqlens"], case["window"]
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            for i in range(a, b):
                m[i, max(a, i - Wd):min(b, i + Wd + 1)] = True
    elif kind == "topk":
        for i in range(T):
            for j in case["topk_idx"][i]:
                if 0 <= j < Tk:
                    m[i, j] = True
    else:
        cu, bs, tab = case["cu_seqlens"], case["block_size"], case["block_sel"]
        hidx = h * tab.shape[1] // Hq
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            for i in range(a, b):
                for blk in np.flatnonzero(tab[0, hidx, i]):
                    lo, hi = max(a, blk * bs), min(i + 1, (blk + 1) * bs)
                    if lo < hi:
                        m[i, lo:hi] = True
    return m


def closed_form_count(case: dict, i: int, h: int) -> int:
    """|S(i,h)| from closed forms per mask kind."""
    kind = case["mask_kind"]
    if kind == "window":
        cu, Wd = case["cu_seqlens"], case["window"]
        s = int(np.searchsorted(cu, i, side="right") - 1)
        return min(i + Wd, int(cu[s + 1]) - 1) - max(i - Wd, int(cu[s])) + 1
    if kind == "topk":
        row = case["topk_idx"][i]
        return int(((row >= 0) & (row < case["k"].shape[0])).sum())
    cu, bs, tab = case["cu_seqlens"], case["block_size"], case["block_sel"]
    Hq = case["q"].shape[1]
    hidx = h * tab.shape[1] // Hq
    s = int(np.searchsorted(cu, i, side="right") - 1)
    a = int(cu[s])
    n = 0
    for blk in np.flatnonzero(tab[0, hidx, i]):
        n += max(0, min(i + 1, (blk + 1) * bs) - max(a, blk * bs))
    return n


def first_key(case: dict, i: int) -> int:
    cu = case["cu_seqlens"]
    return int(cu[int(np.searchsorted(cu, i, side="right") - 1)])


# ---------------------------------------------------------------------- pins
def pin_sdpa(fn, case: dict, exact: bool = True, atol=1e-10):
    """Library reduction: torch's scaled_dot_product_attention in float64, with
    enable_gqa for the head grouping, a float mask (0 / -inf, plus the key-0
    bias) and, for null_logit, one appended key whose logit is the sink and
    whose value is zero.  LSE from torch.logsumexp over the same logits."""
    q = torch.from_numpy(np.asarray(case["q"], dtype=np.float64))
    k = torch.from_numpy(np.asarray(case["k"], dtype=np.float64))
    v = torch.from_numpy(np.ascontiguousarray(case["v"], dtype=np.float64))
    T, Hq, D = q.shape
    Tk, Hkv, Dv = v.shape
    mode, sinks, scale = case["sink_mode"], case["sinks"], case["scale"]
    masks = np.stack([loop_mask(case, h) for h in range(Hq)])               # [Hq, T, Tk]
    fm = torch.where(torch.from_numpy(masks), 0.0, -math.inf).to(torch.float64)
    if mode == "key0_bias":
        cu = case["cu_seqlens"]
        for s in range(len(cu) - 1):
            if cu[s] < cu[s + 1]:
                fm[:, :, int(cu[s])] += torch.from_numpy(np.asarray(sinks, dtype=np.float64))[:, None]
    kk, vv, mm = k, v, fm
    if mode == "null_logit":
        kk = torch.cat([k, torch.zeros(1, Hkv, D, dtype=torch.float64)], 0)
        vv = torch.cat([v, torch.zeros(1, Hkv, Dv, dtype=torch.float64)], 0)
        col = torch.from_numpy(np.asarray(sinks, dtype=np.float64))[:, None, None].expand(Hq, T, 1)
        mm = torch.cat([fm, col], 2)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2)[None], kk.permute(1, 0, 2)[None], vv.permute(1, 0, 2)[None],
        attn_mask=mm[None], scale=scale, enable_gqa=True)[0].permute(1, 0, 2).numpy()
    logits = scale * torch.einsum("thd,shd->hts", q, torch.repeat_interleave(k, Hq // Hkv, dim=1)) + fm
    lse_ref = torch.logsumexp(logits, dim=-1).numpy()                       # [Hq, T]
    out, lse = run(fn, case)
    nonempty = masks.any(axis=2).T                                          # [T, Hq]
    assert np.allclose(out[nonempty], o[nonempty], atol=atol, rtol=0), np.abs(out[nonempty] - o[nonempty]).max()
    assert np.all(out[~nonempty] == 0.0)
    assert np.allclose(lse.T[nonempty], lse_ref.T[nonempty], atol=atol, rtol=0)
    assert np.all(np.isneginf(lse.T[~nonempty]))


def pin_count_probe(fn, case: dict, exact: bool = True):
    """Q = 0 makes every selected logit equal, so lse = ln |S(i,h)| (no sink /
    null sink); with key0_bias and key 0 selected, lse = ln(|S| - 1 + e^s)."""
    q0 = np.zeros_like(case["q"])
    out, lse = run(fn, case, q=q0)
    T, Hq, _ = case["q"].shape
    for i in range(T):
        for h in range(Hq):
            n = closed_form_count(case, i, h)
            if n == 0:
                assert np.isneginf(lse[h, i]) and np.all(out[i, h] == 0.0)
                continue
            expect = math.log(n)
            if case["sink_mode"] == "key0_bias":
                j0 = first_key(case, i)
                if loop_mask(case, h)[i, j0]:
                    expect = math.log(n - 1 + math.exp(float(case["sinks"][h])))
            assert abs(lse[h, i] - expect) < 1e-12, (i, h, lse[h, i], expect)


def pin_key0_closed_form(fn, case: dict):
    """oracle(key0_bias, s) equals the MiMo page's closed-form correction of
    oracle(none), with the LSE shifted by log1p(p0 (e^s - 1))."""
    assert case["mask_kind"] != "topk"
    out0, lse0 = run(fn, case, sink_mode="none", sinks=None)
    out1, lse1 = run(fn, case, sink_mode="key0_bias")
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (case["q"], case["k"], case["v"]))
    T, Hq, _ = q.shape
    g = Hq // k.shape[1]
    for h in range(Hq):
        m = loop_mask(case, h)
        s = float(case["sinks"][h])
        for i in range(T):
            j0 = first_key(case, i)
            if not m[i, j0]:
                assert np.array_equal(out1[i, h], out0[i, h]) and lse1[h, i] == lse0[h, i]
                continue
            l0 = case["scale"] * float(q[i, h] @ k[j0, h // g])
            p0 = math.exp(l0 - lse0[h, i])
            c = p0 * (math.exp(s) - 1.0)
            expect = (out0[i, h] + c * v[j0, h // g]) / (1.0 + c)
            assert np.allclose(out1[i, h], expect, atol=1e-12, rtol=0)
            assert abs(lse1[h, i] - (lse0[h, i] + math.log1p(c))) < 1e-12


def pin_first_w_plus_1_rows(fn, case: dict):
    """Window mask: only the first W+1 queries of each sequence change under
    key0_bias; every other row is bitwise identical to the no-sink result."""
    assert case["mask_kind"] == "window"
    out0, lse0 = run(fn, case, sink_mode="none", sinks=None)
    out1, lse1 = run(fn, case, sink_mode="key0_bias")
    cu, Wd = case["cu_seqlens"], case["window"]
    for i in range(case["q"].shape[0]):
        affected = i - first_key(case, i) <= Wd
        same = np.array_equal(out1[i], out0[i]) and np.array_equal(lse1[:, i], lse0[:, i])
        if not affected:
            assert same, i
        elif np.all(np.asarray(case["sinks"]) != 0):
            assert not np.array_equal(lse1[:, i], lse0[:, i]), i


def pin_noop_sinks(fn, case: dict, exact: bool = True):
    """key0_bias with s = 0 and null_logit with s = -inf both reproduce the
    no-sink result -- bit for bit when the implementation sums in a fixed
    order (the C enumerator); the dense twin's null key lengthens its BLAS
    dot products, which may reorder their rounding, so it gets 1e-15."""
    def same(a, b):
        if exact:
            return np.array_equal(a, b)
        fa, fb = np.isfinite(a), np.isfinite(b)
        return np.array_equal(fa, fb) and np.array_equal(a[~fa], b[~fb]) and np.allclose(a[fa], b[fb], atol=1e-15, rtol=0)
    out0, lse0 = run(fn, case, sink_mode="none", sinks=None)
    Hq = case["q"].shape[1]
    if case["mask_kind"] != "topk":
        o, l = run(fn, case, sink_mode="key0_bias", sinks=np.zeros(Hq, np.float32))
        assert np.array_equal(o, out0) and np.array_equal(l, lse0)
    o, l = run(fn, case, sink_mode="null_logit", sinks=np.full(Hq, -np.inf, np.float32))
    assert same(o, out0) and same(l, lse0)


def pin_null_closed_form(fn, case: dict, exact: bool = True):
    """null_logit: out = out_none / (1 + exp(s - lse_none)); LSE unchanged."""
    sinks = case["sinks"] if case["sinks"] is not None else np.linspace(-2, 2, case["q"].shape[1])
    out0, lse0 = run(fn, case, sink_mode="none", sinks=None)
    out1, lse1 = run(fn, case, sink_mode="null_logit", sinks=np.asarray(sinks, np.float32))
    for h in range(case["q"].shape[1]):
        s = float(np.float32(sinks[h]))
        fin = np.isfinite(lse0[h])
        f = 1.0 / (1.0 + np.exp(s - lse0[h, fin]))
        assert np.allclose(out1[fin, h], out0[fin, h] * f[:, None], atol=1e-12, rtol=0)
        assert np.array_equal(lse1[h], lse0[h]) if exact else np.allclose(lse1[h][fin], lse0[h][fin], atol=1e-15, rtol=0)
        assert np.all(out1[~fin, h] == 0.0)


def pin_single_key(fn, seed: int = 0):
    """One valid key j: out = v_j / (1 + e^(s - l)) and lse = l, l = scale q.k_j."""
    case = W.topk_case(9, 30, 4, 16, 12, 5, counts=(1,), shuffled=True, mla=False, Hkv=4, std=1.0,
                       dtype="f32", sink_mode="null_logit", sink_range=(-2.2, 2.5), seed=seed)
    out, lse = run(fn, case)
    q, k, v = (np.asarray(a, np.float64) for a in (case["q"], case["k"], case["v"]))
    for i in range(9):
        j = int(case["topk_idx"][i][case["topk_idx"][i] >= 0][0])
        for h in range(4):
            l = case["scale"] * float(q[i, h] @ k[j, h])
            s = float(case["sinks"][h])
            assert np.allclose(out[i, h], v[j, h] / (1.0 + math.exp(s - l)), atol=1e-12, rtol=0)
            assert abs(lse[h, i] - l) < 1e-12


def pin_constant_values(fn, case: dict, exact: bool = True):
    """V = c everywhere: out = c (none / key0_bias) and c * sigmoid(lse - s) (null_logit)."""
    c = np.float32(0.75)
    vc = np.full_like(np.ascontiguousarray(case["v"]), c)
    out, lse = run(fn, case, v=vc)
    for h in range(case["q"].shape[1]):
        fin = np.isfinite(lse[h])
        if case["sink_mode"] == "null_logit":
            s = float(case["sinks"][h])
            expect = float(c) / (1.0 + np.exp(s - lse[h, fin]))
            assert np.allclose(out[fin, h], expect[:, None], atol=1e-12, rtol=0)
        else:
            assert np.allclose(out[fin, h], float(c), atol=1e-12, rtol=0)


def pin_topk_permutation(fn, case: dict, seed: int = 0):
    """Reordering a top-k row (padding included) leaves the result unchanged."""
    g = np.random.default_rng(seed)
    idx = case["topk_idx"].copy()
    for i in range(idx.shape[0]):
        g.shuffle(idx[i])
    a = run(fn, case)
    b = run(fn, case, topk_idx=idx)
    assert np.allclose(a[0], b[0], atol=1e-12, rtol=0) and np.allclose(a[1], b[1], atol=1e-12, rtol=0)


def pin_conventions_differ(fn, case: dict):
    """key0_bias and null_logit are different operations for s != 0 (MiMo
    page), and rows with few keys differ from the no-sink result (sparse-MLA
    page)."""
    out0, _ = run(fn, case, sink_mode="none", sinks=None)
    outn, _ = run(fn, case, sink_mode="null_logit")
    assert np.abs(outn - out0).max() > 1e-3
    if case["mask_kind"] != "topk":
        outk, _ = run(fn, case, sink_mode="key0_bias")
        assert np.abs(outk - outn).max() > 1e-3


ALL_CASE_PINS = (pin_sdpa, pin_count_probe, pin_noop_sinks, pin_null_closed_form, pin_constant_values)
