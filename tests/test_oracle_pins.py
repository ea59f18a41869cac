"""The CPU oracle against what the pages and plain mathematics fix (no GPU)."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import dense
from tests import pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
IMPLS = {"enum_c": oracle.attn_ref, "dense_np": oracle.attn_dense}
EXACT = {"enum_c": True, "dense_np": False}
CASES = P.tiny_cases(0) + P.tiny_cases(5)


def _ids(cs):
    return [f"{c['name']}-{i}" for i, c in enumerate(cs)]


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("case", CASES, ids=_ids(CASES))
def test_case_pins(impl, case):
    for pin in P.ALL_CASE_PINS:
        pin(IMPLS[impl], case, exact=EXACT[impl])


@pytest.mark.parametrize("impl", list(IMPLS))
def test_key0_closed_form(impl):
    for case in CASES:
        if case["mask_kind"] != "topk" and case["sink_mode"] == "key0_bias":
            P.pin_key0_closed_form(IMPLS[impl], case)


@pytest.mark.parametrize("impl", list(IMPLS))
def test_first_w_plus_1_rows(impl):
    for case in CASES:
        if case["mask_kind"] == "window" and case["sink_mode"] == "key0_bias":
            P.pin_first_w_plus_1_rows(IMPLS[impl], case)


@pytest.mark.parametrize("impl", list(IMPLS))
def test_single_key_and_permutation(impl):
    P.pin_single_key(IMPLS[impl])
    for case in CASES:
        if case["mask_kind"] == "topk":
            P.pin_topk_permutation(IMPLS[impl], case)


@pytest.mark.parametrize("impl", list(IMPLS))
def test_conventions_differ(impl):
    for case in CASES:
        if case["sinks"] is not None:
            P.pin_conventions_differ(IMPLS[impl], case)


def test_twins_agree_on_all_tiny_cases():
    for case in CASES:
        a = P.run(oracle.attn_ref, case)
        b = P.run(oracle.attn_dense, case)
        assert np.allclose(a[0], b[0], atol=1e-12, rtol=0)
        assert np.array_equal(np.isneginf(a[1]), np.isneginf(b[1]))
        fin = np.isfinite(a[1])
        assert np.allclose(a[1][fin], b[1][fin], atol=1e-12, rtol=0)


def test_twins_agree_on_tiny_window_workload():
    case = W.make_workload("tiny_window_f32", seed=1)
    a = P.run(oracle.attn_ref, case)
    b = P.run(oracle.attn_dense, case)
    assert np.allclose(a[0], b[0], atol=1e-12, rtol=0) and np.allclose(a[1], b[1], atol=1e-12, rtol=0)
    P.pin_key0_closed_form(oracle.attn_ref, case)
    P.pin_first_w_plus_1_rows(oracle.attn_ref, case)


def test_row_subset_matches_full():
    case = CASES[2]
    full = P.run(oracle.attn_ref, case)
    rows = np.array([5, 0, 17, 39, 6])
    sub = P.run(oracle.attn_ref, case, rows=rows)
    assert np.array_equal(sub[0], full[0][rows]) and np.array_equal(sub[1], full[1][:, rows])


# ----------------------------------------------------------- golden fixtures
def test_golden_affected_rows():
    fx = json.load(open(os.path.join(GOLDEN, "key0_affected_rows.json")))
    for c in fx["cases"]:
        case = W.window_case(c["seqlens"], 2, 1, 8, c["window"], dtype="f32", sink_mode="key0_bias",
                             sink_range=(0.5, 1.5), seed=3)
        for fn in IMPLS.values():
            o0, l0 = P.run(fn, case, sink_mode="none", sinks=None)
            o1, l1 = P.run(fn, case)
            changed = [i for i in range(len(o0)) if not np.array_equal(l0[:, i], l1[:, i])]
            assert changed == c["affected_rows"]


def test_golden_document_ids():
    fx = json.load(open(os.path.join(GOLDEN, "document_ids.json")))
    for c in fx["cases"]:
        pos = np.asarray(c["positions"])
        starts = np.flatnonzero(pos == 0).tolist() + [len(pos)]
        seg = dense.segment_ids(np.asarray(starts), len(pos))
        assert seg.tolist() == c["doc_ids"]
        assert (np.cumsum(pos == 0) - 1).tolist() == c["doc_ids"]


def test_golden_blocksel_offset_does_not_wrap():
    fx = json.load(open(os.path.join(GOLDEN, "blocksel_offset_limit.json")))
    H, S, bs = fx["num_index_heads"], fx["seq_len"], fx["block_size"]
    NB = S // bs
    assert NB == fx["num_blocks"] and H * S * NB == fx["elements_at_limit"] == 2 ** 31
    last = oracle.blocksel_flat_offset(0, H - 1, S - 1, NB - 1, H, S, NB)
    assert last == 2 ** 31 - 1
    # one more block of queries: offsets now pass 2**31 and must stay exact (no wrap)
    S2 = S + bs
    NB2 = S2 // bs
    off = oracle.blocksel_flat_offset(0, H - 1, S2 - 1, NB2 - 1, H, S2, NB2)
    assert off == H * S2 * NB2 - 1 > 2 ** 31
    assert off == ((0 * H + (H - 1)) * S2 + (S2 - 1)) * NB2 + (NB2 - 1)


# --------------------------------------------------- the pins have teeth
def _mutants():
    """Plausible mistakes, each planted in the dense oracle through its seams."""
    def window_exclusive(i, j, Wd):
        return np.abs(i - j) < Wd

    def kv_modulo(h, Hq, Hkv):
        return h % Hkv

    def key0_last(cu, Tk):
        m = np.zeros(Tk, dtype=bool)
        for s in range(len(cu) - 1):
            if cu[s] < cu[s + 1]:
                m[int(cu[s + 1]) - 1] = True
        return m

    def bias_scaled(s, scale):
        return s * scale

    def lse_with_sink(sel, sink):
        allv = sel if sink is None else np.concatenate([sel, [sink]])
        ms = allv.max()
        return float(ms + np.log(np.exp(allv - ms).sum()))

    orig_mask = dense.key_mask

    def topk_minus1_valid(kind, rows, h, Tk, Hq, **kw):
        if kind != "topk":
            return orig_mask(kind, rows, h, Tk, Hq, **kw)
        idx = np.asarray(kw["topk_idx"], dtype=np.int64)[np.asarray(rows)]
        m = np.zeros((len(rows), Tk), dtype=bool)
        for r in range(len(rows)):
            sel = idx[r][(idx[r] >= -Tk) & (idx[r] < Tk)]   # forgets the lower bound: -1 wraps to the last key
            m[r, sel] = True
        return m

    def blocksel_no_causal(kind, rows, h, Tk, Hq, **kw):
        m = orig_mask(kind, rows, h, Tk, Hq, **kw)
        if kind != "blocksel":
            return m
        rows = np.asarray(rows)
        j = np.arange(Tk)
        tab = np.asarray(kw["block_sel"])
        blk = tab[0, h // (Hq // tab.shape[1])][rows][:, j // kw["block_size"]] != 0
        seg = dense.segment_ids(kw["cu_seqlens"], Tk)
        return blk & (seg[rows][:, None] == seg[None, :])

    return {
        "window_exclusive": ("window_keep", window_exclusive),
        "gqa_modulo": ("kv_head", kv_modulo),
        "key0_on_last_key": ("key0_columns", key0_last),
        "sink_scaled": ("key0_bias_value", bias_scaled),
        "lse_includes_null_sink": ("selected_lse", lse_with_sink),
        "topk_minus1_valid": ("key_mask", topk_minus1_valid),
        "blocksel_no_causal": ("key_mask", blocksel_no_causal),
    }


def _all_pins(fn):
    for case in CASES:
        for pin in P.ALL_CASE_PINS:
            pin(fn, case, exact=False)
        if case["mask_kind"] != "topk" and case["sink_mode"] == "key0_bias":
            P.pin_key0_closed_form(fn, case)
        if case["mask_kind"] == "window" and case["sink_mode"] == "key0_bias":
            P.pin_first_w_plus_1_rows(fn, case)


@pytest.mark.parametrize("name", list(_mutants()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fake = _mutants()[name]
    monkeypatch.setattr(dense, attr, fake)
    with pytest.raises(AssertionError):
        _all_pins(dense.attn_dense)


def test_swapped_operands_are_caught():
    """Transposed logits (q and k swapped in self-attention) and values taken
    from k both fail the library-reduction pin."""
    mha = [c for c in CASES if c["q"].shape == c["k"].shape]
    same_d = [c for c in CASES if c["k"].shape == np.shape(c["v"])]
    assert mha and same_d
    swap_qk = lambda q, k, v, **kw: oracle.attn_dense(k, q, v, **kw)
    v_from_k = lambda q, k, v, **kw: oracle.attn_dense(q, k, k, **kw)
    with pytest.raises(AssertionError):
        P.pin_sdpa(swap_qk, mha[0])
    with pytest.raises(AssertionError):
        P.pin_sdpa(v_from_k, same_d[0])
