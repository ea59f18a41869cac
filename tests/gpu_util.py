"""Shared helpers for the GPU parity tests: run a generated case through the
C ABI on cuda:0 and compare it with the CPU oracle on the same inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from tests import pins as P

BF16_REL_L2 = 5e-3     # max over (row, head) of |o - o_ref|_2 / |o_ref|_2
BF16_LSE_ABS = 1e-4    # max |lse - lse_ref|
F32_REL_L2 = 1e-5
F32_LSE_ABS = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sam():
    import sink_aware_masked_amd
    return sink_aware_masked_amd


def gpu_run(case: dict, device="cuda:0", **over):
    """(out, lse) as float64 NumPy arrays from the HIP path."""
    import torch
    out, lse = sam().run_case(case, device=device, **over)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_run(case: dict, rows=None, **over):
    return P.run(oracle.attn_ref, case, rows=rows, **over)


def tensor_rel_l2(out, ref_out) -> float:
    """One relative L2 over the whole output tensor (the pages' error
    statistic, reported beside the per-row maximum that gates)."""
    den = float(np.linalg.norm(ref_out))
    return float(np.linalg.norm(out - ref_out)) / den if den > 0 else 0.0


def compare(out, lse, ref_out, ref_lse):
    """Returns (max rel L2 over non-empty (row, head), max |dLSE| over finite).
    Asserts that rows the oracle calls empty are exactly 0 / -inf."""
    ref_n = np.linalg.norm(ref_out, axis=2)                     # [R, Hq]
    empty = np.isneginf(ref_lse.T)                              # [R, Hq]
    assert np.all(out[empty] == 0.0), "empty rows must be exactly zero"
    assert np.all(np.isneginf(lse.T[empty])), "empty rows must have lse = -inf"
    assert np.all(np.isfinite(lse.T[~empty])), "non-empty rows need a finite lse"
    nz = (~empty) & (ref_n > 0)
    rel = np.linalg.norm(out - ref_out, axis=2)[nz] / ref_n[nz]
    dl = np.abs(lse.T[~empty] - ref_lse.T[~empty])
    return (float(rel.max()) if rel.size else 0.0), (float(dl.max()) if dl.size else 0.0)


def tolerances(case):
    return (BF16_REL_L2, BF16_LSE_ABS) if case["dtype"] == "bf16" else (F32_REL_L2, F32_LSE_ABS)


def assert_parity(case: dict, rows=None, label="", **over):
    """Run case on the GPU and the oracle on `rows` (all rows if None)."""
    say(f"[parity] {label or case['name']} rows={'all' if rows is None else len(rows)}")
    out, lse = gpu_run(case, **over)
    ref_out, ref_lse = oracle_run(case, rows=rows, **over)
    if rows is not None:
        out, lse = out[rows], lse[:, rows]
    rel, dl = compare(out, lse, ref_out, ref_lse)
    tr, tl = tolerances(case)
    say(f"[parity] {label or case['name']}: max rel L2 {rel:.3e} (<= {tr}), tensor rel L2 "
        f"{tensor_rel_l2(out, ref_out):.3e}, lse max abs {dl:.3e} (<= {tl})")
    assert rel <= tr and dl <= tl, (rel, dl)
    return out, lse


def sample_rows(case: dict, n: int, seed: int = 0, extra=()):
    """Sorted unique rows: n seeded random rows plus the ends of every segment
    and `extra`."""
    T = case["q"].shape[0]
    g = np.random.default_rng(seed)
    rows = set(g.choice(T, size=min(n, T), replace=False).tolist()) | set(int(x) for x in extra)
    cu = case.get("cu_seqlens")
    if cu is not None:
        for s in range(len(cu) - 1):
            for r in (cu[s], cu[s] + 1, cu[s + 1] - 1, cu[s + 1] - 2):
                if cu[s] <= r < cu[s + 1]:
                    rows.add(int(r))
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int64)
