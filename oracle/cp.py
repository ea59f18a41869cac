"""CPU oracle for the context-parallel reorder primitives: TEST INFRASTRUCTURE.

Only ``tests/`` and the CPU-baseline leg of ``bench.py`` may use this module;
the HIP library never does, and the two share no code.

Plain NumPy, written from the NeMo AutoModel ``cp_sparse_attn`` API page:

* :func:`load_balanced_slots` -- ``cp_load_balanced_global_slots``: causal
  context parallelism cuts the sequence into ``2 * cp_size`` equal chunks and
  gives rank ``r`` chunks ``r`` and ``2 * cp_size - 1 - r``, in that order;
  with ``rank=None`` the slots of every rank, rank-major (the all-gathered
  concatenation).
* :func:`order_by_positions` -- gathered rows into global token order, with
  the sort order; rejects positions that are not a permutation of 0..S-1.
* :func:`restore_by_positions` -- rows of a global-ordered tensor at given
  positions, in that order.
* :func:`document_ids` -- ``cp_document_ids``: cumsum(positions == 0) - 1.
* :func:`segment_starts` -- the same documents as a ``cu_seqlens`` boundary
  list (token 0 always opens a segment), the form the attention kernels take.
"""
from __future__ import annotations

import numpy as np


def load_balanced_slots(cp_size: int, t_local: int, rank: int | None = None) -> np.ndarray:
    if cp_size < 1 or t_local < 0 or t_local % 2:
        raise ValueError("cp_size >= 1 and an even t_local are required")
    chunk = t_local // 2

    def one(r):
        first = np.arange(r * chunk, (r + 1) * chunk)
        second = np.arange((2 * cp_size - 1 - r) * chunk, (2 * cp_size - r) * chunk)
        return np.concatenate([first, second])
    if rank is not None:
        return one(rank).astype(np.int64)
    return np.concatenate([one(r) for r in range(cp_size)]).astype(np.int64)


def order_by_positions(gathered: np.ndarray, positions: np.ndarray, seq_dim: int = 0):
    positions = np.asarray(positions)
    S = gathered.shape[seq_dim]
    if positions.ndim != 1 or len(positions) != S or not np.array_equal(np.sort(positions), np.arange(S)):
        raise ValueError("gathered positions must be a permutation of 0..S-1")
    order = np.argsort(positions, kind="stable")
    return np.take(gathered, order, axis=seq_dim), order


def restore_by_positions(global_tensor: np.ndarray, target_positions: np.ndarray, seq_dim: int = 0):
    return np.take(global_tensor, np.asarray(target_positions), axis=seq_dim)


def document_ids(positions: np.ndarray) -> np.ndarray:
    return np.cumsum(np.asarray(positions) == 0) - 1


def segment_starts(positions: np.ndarray) -> np.ndarray:
    """cu_seqlens: 0, every later index whose position is 0, then T."""
    pos = np.asarray(positions)
    T = len(pos)
    starts = [0] + [i for i in range(1, T) if pos[i] == 0] if T else []
    return np.asarray(starts + [T], dtype=np.int64)
