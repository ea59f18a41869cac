"""Pins for the context-parallel reorder oracle (oracle/cp.py) against what
the NeMo AutoModel 'cp_sparse_attn' API page states: hand-worked slot maps
(tests/golden/cp_slots.json), the load balance the pairing {r, 2cp-1-r} is
for, the round trip of order_by_positions / restore_by_positions, the
rejection of positions that are not a permutation, and cp_document_ids'
cumsum(positions == 0) - 1 (tests/golden/document_ids.json)."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

from oracle import cp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_slots():
    fx = json.load(open(os.path.join(GOLDEN, "cp_slots.json")))
    for c in fx["cases"]:
        for r, want in enumerate(c["ranks"]):
            assert cp.load_balanced_slots(c["cp_size"], c["t_local"], rank=r).tolist() == want
        assert cp.load_balanced_slots(c["cp_size"], c["t_local"]).tolist() == c["all"]


def balanced_and_paired(slots_of, cp_size, t_local):
    """Every rank holds two whole chunks, r and 2cp-1-r, and the same total of
    causal work (sum of global indices), and together the ranks cover 0..T-1."""
    c = t_local // 2
    T = cp_size * t_local
    allslots = np.concatenate([slots_of(r) for r in range(cp_size)])
    if not np.array_equal(np.sort(allslots), np.arange(T)):
        return False
    sums = {int(slots_of(r).sum()) for r in range(cp_size)}
    if len(sums) != 1:
        return False
    for r in range(cp_size):
        s = slots_of(r)
        if not (np.array_equal(s[:c], np.arange(r * c, (r + 1) * c))
                and np.array_equal(s[c:], np.arange((2 * cp_size - 1 - r) * c, (2 * cp_size - r) * c))):
            return False
    return True


@pytest.mark.parametrize("cp_size,t_local", [(1, 2), (2, 8), (3, 6), (8, 4096), (5, 0), (16, 32)])
def test_slots_invariants(cp_size, t_local):
    assert balanced_and_paired(lambda r: cp.load_balanced_slots(cp_size, t_local, rank=r), cp_size, t_local)
    allslots = cp.load_balanced_slots(cp_size, t_local)
    assert np.array_equal(allslots, np.concatenate([cp.load_balanced_slots(cp_size, t_local, r)
                                                    for r in range(cp_size)]))


def test_slots_pins_have_teeth():
    """Plausible wrong pairings (r with cp + r; r with 2cp - 2 - r) fail."""
    def pair_shift(cp_size, t_local, r):
        c = t_local // 2
        return np.concatenate([np.arange(r * c, (r + 1) * c), np.arange((cp_size + r) * c, (cp_size + r + 1) * c)])

    def pair_off_by_one(cp_size, t_local, r):
        c = t_local // 2
        o = (2 * cp_size - 2 - r) % (2 * cp_size)
        return np.concatenate([np.arange(r * c, (r + 1) * c), np.arange(o * c, (o + 1) * c)])
    for bad in (pair_shift, pair_off_by_one):
        assert not balanced_and_paired(lambda r: bad(4, 8, r), 4, 8)
    fx = json.load(open(os.path.join(GOLDEN, "cp_slots.json")))
    c = fx["cases"][0]
    assert pair_shift(c["cp_size"], c["t_local"], 0).tolist() != c["ranks"][0]


def test_order_and_restore_round_trip():
    g = np.random.default_rng(0)
    cp_size, t_local = 4, 10
    T = cp_size * t_local
    x = g.standard_normal((T, 3, 5))                      # global token order
    pos_all = cp.load_balanced_slots(cp_size, t_local)
    gathered = x[pos_all]                                 # what an all-gather of the shards holds
    glob, order = cp.order_by_positions(gathered, pos_all)
    assert np.array_equal(glob, x)
    assert np.array_equal(pos_all[order], np.arange(T))
    for r in range(cp_size):
        mine = cp.load_balanced_slots(cp_size, t_local, r)
        assert np.array_equal(cp.restore_by_positions(glob, mine), gathered[r * t_local:(r + 1) * t_local])
    # seq_dim other than 0
    y = np.moveaxis(gathered, 0, 1)
    gy, _ = cp.order_by_positions(y, pos_all, seq_dim=1)
    assert np.array_equal(np.moveaxis(gy, 1, 0), x)


@pytest.mark.parametrize("bad", [[0, 1, 1, 3], [0, 1, 2, 4], [1, 2, 3], [-1, 0, 1, 2]])
def test_order_rejects_non_permutations(bad):
    with pytest.raises(ValueError):
        cp.order_by_positions(np.zeros((4, 2)), np.asarray(bad))


def test_document_ids_and_segments():
    fx = json.load(open(os.path.join(GOLDEN, "document_ids.json")))
    for c in fx["cases"]:
        pos = np.asarray(c["positions"])
        assert cp.document_ids(pos).tolist() == c["doc_ids"]
        cu = cp.segment_starts(pos)
        seg = np.searchsorted(cu, np.arange(len(pos)), side="right") - 1
        assert seg.tolist() == c["doc_ids"]  # position 0 first: segments are the documents
    # a leading run without a position-0 token: ids start at -1, segments at 0
    pos = np.array([3, 4, 0, 1, 0])
    assert cp.document_ids(pos).tolist() == [-1, -1, 0, 0, 1]
    assert cp.segment_starts(pos).tolist() == [0, 2, 4, 5]
    assert cp.segment_starts(np.array([], dtype=np.int64)).tolist() == [0]
