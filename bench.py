#!/usr/bin/env python3
"""Benchmark of the sink-aware masked attention forward on one MI355X.

One step = one attn_sink_fwd call (the whole hot path: varlen scheduling, key
enumeration, K/V staging, logits, online softmax, output accumulation and the
sink epilogue -- one kernel launch) over one batch of seeded synthetic input
that is already resident in HBM.

Default workload (no flags): the MiniMax-M3-style block-sparse layer of the
NeMo AutoModel "cp_sparse_attn" page (_flex_sparse_attention: selected block
and token-causal and same document) -- 32768 tokens in 4 packed documents,
32 query / 8 kv heads, head dim 128, 64-token key blocks, each query its own
diagonal block plus 15 random earlier blocks of its document, bf16, null_logit
sinks from U(-2, 2) -- the largest workload that fits one GPU; the same layer
without a sink is timed too and reported as a ratio (sink_vs_none).
Other workloads: --workload window_4k | window_16k | mla_topk | mla_decode_fp8.
--compare-unfused (window workloads) also times the page's unfused design (no-sink
kernel + closed-form key-0 correction); --measure-merge (mla_topk) times the
top-k lists split in two halves, each through the no-sink kernel, merged by LSE
with the sink folded in after the merge; --measure-cp (blocksparse_32k) times the
context-parallel reorder of K/V from an 8-rank load-balanced layout.
--workload mla_decode_fp8 times the sparse-MLA decode over an fp8 latent cache.

Prints ONE JSON line:
  value      useful TFLOP/s of the whole job = 2 (Dqk + Dv) sum |S(i,h)| / wall time
  roofline   the kernel against its binding roof, from HIP events on the
             launch stream around the timed launches (algorithmic bytes or
             useful flops per launch / average launch duration); also the
             median, p10 and p90 of per-launch durations (HIP events around
             each of `steps` further launches)
  cpu_baseline  the CPU oracle (C, fp64, OpenMP) on a bounded row sample of
             the same workload, in the same unit
Cold cache: the step rotates over enough input sets to exceed the 256 MB
Infinity Cache when one set is smaller than that.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/call + useful TFLOP/s (frac of MFMA bf16 peak) for sink-aware masked attn fwd"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
PEAK_MFMA_BF16_TFS = 2500.0  # MI355X dense bf16 MFMA, published
MALL_BYTES = 256 << 20       # Infinity Cache

# The pages' timing context (H100, FlashAttention varlen + the unfused key-0
# correction): ms per call for the same window workloads.  Another machine and
# another design: reported beside the result (page_context), never as its
# baseline.
PAGE_MS = {("window_4k", "key0_bias"): 0.248, ("window_4k", "none"): 0.038,
           ("window_16k", "key0_bias"): 0.289, ("window_16k", "none"): 0.134}

KERNEL_SRC = {"window": "window_fwd.hip", "topk": "topk_mla_fwd.hip", "blocksel": "blocksel_fwd.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------- work accounting
def seg_starts_ends(cu, n):
    cu = np.asarray(cu, dtype=np.int64)
    lens = np.diff(cu)
    return np.repeat(cu[:-1], lens)[:n], np.repeat(cu[1:], lens)[:n]


def pairs_per_row(case) -> np.ndarray:
    """|S(i,h)| summed over heads, per query row (int64 [T])."""
    T, Hq = case["q"].shape[:2]
    kind = case["mask_kind"]
    if kind == "window":
        st, en = seg_starts_ends(case["cu_seqlens"], T)
        i = np.arange(T)
        W = case["window"]
        return (np.minimum(en - 1, i + W) - np.maximum(st, i - W) + 1) * Hq
    if kind == "topk":
        idx = case["topk_idx"]
        return ((idx >= 0) & (idx < case["k"].shape[0])).sum(1).astype(np.int64) * Hq
    tab = case["block_sel"][0]                       # [Hidx, T, NB]
    Hidx, _, NB = tab.shape
    bs = case["block_size"]
    st, _ = seg_starts_ends(case["cu_seqlens"], T)
    i = np.arange(T)[:, None]
    b0 = (np.arange(NB) * bs)[None, :]
    ov = np.clip(np.minimum(i, b0 + bs - 1) - np.maximum(st[:, None], b0) + 1, 0, None)
    out = np.zeros(T, dtype=np.int64)
    for h in range(Hidx):
        out += ((tab[h] != 0) * ov).sum(1)
    return out * (Hq // Hidx)


def algorithmic_bytes(case) -> int:
    q, k, v = case["q"], case["k"], case["v"]
    T, Hq, Dqk = q.shape
    Tk, Hkv, _ = k.shape
    Dv = v.shape[2]
    es = 2 if case["dtype"] == "bf16" else 4
    b = T * Hq * Dqk * es + T * Hq * Dv * es + Hq * T * 4
    kind = case["mask_kind"]
    if kind == "window":
        b += Tk * Hkv * (Dqk + Dv) * es + case["cu_seqlens"].nbytes
    elif kind == "topk":
        idx = case["topk_idx"]
        distinct = np.unique(idx[(idx >= 0) & (idx < Tk)]).size
        row = Dqk * es if case.get("v_aliases_k") else (Dqk + Dv) * es
        b += distinct * Hkv * row + idx.nbytes
    else:
        tab = case["block_sel"][0]
        used = (tab != 0).any(axis=1)                # [Hidx, NB] blocks any query selected
        bs = case["block_size"]
        keys_per_idx = np.minimum((np.arange(used.shape[1]) + 1) * bs, Tk) - np.arange(used.shape[1]) * bs
        keys = (used * keys_per_idx[None, :]).sum(1)  # per index head
        b += int(keys.sum()) * (Hkv // tab.shape[0]) * (Dqk + Dv) * es + case["block_sel"].nbytes
        b += case["cu_seqlens"].nbytes
    if case["sinks"] is not None:
        b += Hq * 4
    return int(b)


def _code_only(text: str) -> str:
    """Source text without comments and blank-line differences, so that a
    comment edit does not count as a kernel change."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_hash(kind: str) -> str:
    """Hash of the kernel's code (comments ignored) and of the extra compiler
    options its source is built with."""
    from __graft_entry__ import EXTRA_FLAGS
    h = hashlib.sha256()
    for f in ("common.hpp", KERNEL_SRC[kind]):
        h.update(_code_only(open(os.path.join(ROOT, "sink_aware_masked_amd", "csrc", f)).read()).encode())
    extra = EXTRA_FLAGS.get(KERNEL_SRC[kind])
    if extra:
        h.update(" ".join(extra).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kind: str):
    """HBM bytes per launch from committed rocprofv3 PMC counters, or None if
    absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sha") != kernel_hash(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------- workloads
def build_case(name: str, seed: int, sink_mode: str | None, gqa: bool = False):
    import workloads as W
    kw = {} if sink_mode is None else {"sink_mode": sink_mode}
    if gqa:
        kw["gqa"] = True
    return W.make_workload(name, seed=seed, **kw)


def describe(name, case, sets):
    q, k, v = case["q"], case["k"], case["v"]
    cfg = {"workload": name, "tokens": int(q.shape[0]), "q_heads": int(q.shape[1]),
           "kv_heads": int(k.shape[1]), "head_dim_qk": int(q.shape[2]), "head_dim_v": int(v.shape[2]),
           "mask": case["mask_kind"], "sink_mode": case["sink_mode"], "cold_cache_sets": sets}
    if case["mask_kind"] == "window":
        cfg.update(window=case["window"], seqs=len(case["cu_seqlens"]) - 1)
    elif case["mask_kind"] == "topk":
        cfg.update(kv_entries=int(k.shape[0]), topk=int(case["topk_idx"].shape[1]), shared_latent_kv=True)
    else:
        cfg.update(documents=len(case["cu_seqlens"]) - 1, block_size=case["block_size"],
                   index_heads=int(case["block_sel"].shape[1]))
    return cfg


# ------------------------------------------------------------------- timing
def time_gpu(case, sets_n, steps, warmup, use_graph=True):
    """Warm up eagerly, then time exactly `steps` launches.  The timed launches
    are captured once into a HIP graph (replayed once inside the timed region)
    so that host-side launch overhead does not pace a kernel of a few
    microseconds; HIP events on the launch stream bracket the replay."""
    import torch
    import sink_aware_masked_amd as sam
    torch.cuda.set_device(0)
    sets = []
    for _ in range(sets_n):
        d = sam.case_on_device(case, "cuda:0")
        T, Hq = d["q"].shape[:2]
        d["out"] = torch.empty((T, Hq, d["v"].shape[2]), dtype=d["q"].dtype, device="cuda:0")
        d["lse"] = torch.empty((Hq, T), dtype=torch.float32, device="cuda:0")
        sets.append(d)
    eager = [sam.prepared_fwd(**d) for d in sets]
    for s in range(warmup):
        eager[s % sets_n]()
    torch.cuda.synchronize()
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            captured = [sam.prepared_fwd(**d) for d in sets]   # bound to the capture stream
            for s in range(steps):
                captured[s % sets_n]()
        run = g.replay
    else:
        def run():
            for s in range(steps):
                eager[s % sets_n]()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()                                   # barrier: N = 1
    t0 = time.perf_counter()
    ev0.record()
    run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = ev0.elapsed_time(ev1) / steps                    # average launch duration
    counter = [0]

    def one():
        eager[counter[0] % sets_n]()
        counter[0] += 1
    stats = launch_stats(one, steps)
    if use_graph:  # a replayed launch must reproduce the eager result bit for bit
        ref_out = torch.empty_like(sets[0]["out"])
        ref_lse = torch.empty_like(sets[0]["lse"])
        sam.fwd(**{k: v for k, v in sets[0].items() if k not in ("out", "lse")}, out=ref_out, lse=ref_lse)
        torch.cuda.synchronize()
        assert torch.equal(ref_out, sets[0]["out"]) and torch.equal(ref_lse, sets[0]["lse"]), \
            "graph replay differs from the eager launch"
    return wall * 1e3 / steps, kern_ms, sets[0], stats


def launch_stats(fn, n):
    """Median, p10 and p90 (ms) of n launches of fn, each bracketed by HIP
    events on torch's current stream (the stream the binding launches on)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    return {"launches": int(n), "median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90))}


def graph_ms(step, steps, warmup):
    """Average ms of one `step` (a zero-argument callable that enqueues its
    launches on torch's current stream): warm up eagerly, capture `steps`
    repetitions into one HIP graph, replay it once between HIP events."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def compare_unfused(case, steps, warmup, fused_ms):
    """The MiMo page's unfused design on this GPU: the no-sink window kernel
    followed by the closed-form key-0 correction of the first W + 1 rows of
    each sequence, against the fused key0_bias kernel."""
    import torch
    import sink_aware_masked_amd as sam
    d = sam.case_on_device(case, "cuda:0")
    T, Hq = d["q"].shape[:2]
    out = torch.empty((T, Hq, d["v"].shape[2]), dtype=d["q"].dtype, device="cuda:0")
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda:0")
    nosink = dict(d, sink_mode="none", sinks=None)

    def fwd_none():
        sam.fwd(**nosink, out=out, lse=lse)

    def fwd_fused():
        sam.fwd(**d, out=out, lse=lse)

    def correction():
        sam.attn_sink_key0_correct(d["q"], d["k"], d["v"], d["cu_seqlens"], case["window"], d["sinks"],
                                   case["scale"], out, lse)

    def unfused():
        fwd_none()
        correction()
    ms_fused = graph_ms(fwd_fused, steps, warmup)
    ms_none = graph_ms(fwd_none, steps, warmup)
    ms_unfused = graph_ms(unfused, steps, warmup)
    ms_corr = graph_ms(correction, steps, warmup)
    return {"fused_kernel_ms": ms_fused, "nosink_kernel_ms": ms_none, "correction_kernel_ms": ms_corr,
            "unfused_ms": ms_unfused, "unfused_over_fused": ms_unfused / ms_fused,
            "fused_over_nosink": ms_fused / ms_none, "fused_kernel_ms_cold": fused_ms,
            "note": "hot cache (one input set) except fused_kernel_ms_cold; "
                    "unfused = no-sink kernel + key-0 correction kernel"}


def measure_merge(case, steps, warmup, fused_ms):
    """Split-KV composition on this GPU: the top-k lists cut into two column
    halves, each half through the no-sink kernel, then the LSE merge with the
    null-logit sink folded in after it.  The merge alone is HBM bound: its
    bytes are two partial (out, lse) pairs read and one written."""
    import torch
    import sink_aware_masked_amd as sam
    d = sam.case_on_device(case, "cuda:0")
    T, Hq = d["q"].shape[:2]
    Dv = d["v"].shape[2]
    idx = d["topk_idx"]
    half = idx.shape[1] // 2
    pieces = [idx[:, :half], idx[:, half:]]
    parts = [(torch.empty((T, Hq, Dv), dtype=d["q"].dtype, device="cuda:0"),
              torch.empty((Hq, T), dtype=torch.float32, device="cuda:0")) for _ in pieces]
    out = torch.empty_like(parts[0][0])
    lse = torch.empty_like(parts[0][1])
    halves = [dict(d, sink_mode="none", sinks=None, topk_idx=pc, out=po, lse=pl)
              for pc, (po, pl) in zip(pieces, parts)]

    def merge():
        sam.attn_sink_merge(parts, d["sinks"], case["sink_mode"], out, lse)

    def split_path():  # the binding launches on torch's current stream at call time
        for h in halves:
            sam.fwd(**h)
        merge()
    for h in halves:
        sam.fwd(**h)
    ms_merge = graph_ms(merge, steps, warmup)
    ms_split = graph_ms(split_path, max(1, steps // 4), max(1, warmup // 4))
    es = out.element_size()
    nbytes = 3 * (T * Hq * Dv * es + Hq * T * 4) + Hq * 4
    ach = nbytes / (ms_merge * 1e-3) / 1e9
    return {"merge_kernel_ms": ms_merge, "merge_bytes": nbytes, "merge_GBps": ach,
            "merge_frac_hbm": ach / PEAK_HBM_GBS, "split2_fwd_plus_merge_ms": ms_split,
            "fused_kernel_ms": fused_ms, "split_over_fused": ms_split / fused_ms}


def measure_cp(case, steps, warmup, cp_size=8):
    """Context-parallel reorder on this GPU: K and V of the workload as an
    all-gather of cp_size load-balanced shards would hold them, put into global
    token order (two row scatters), and the document segments derived from the
    reordered position ids.  The scatters are HBM bound: each row is read once
    and written once, plus the int64 index."""
    import torch
    import sink_aware_masked_amd as sam
    d = sam.case_on_device(case, "cuda:0")
    T = d["q"].shape[0]
    slots = torch.empty(T, dtype=torch.int64, device="cuda:0")
    sam.attn_sink_cp_slots(cp_size, T // cp_size, -1, slots)
    lens = np.diff(case["cu_seqlens"])
    pos = torch.from_numpy(np.concatenate([np.arange(n) for n in lens]).astype(np.int64)).to("cuda:0")
    gathered = [d["k"][slots], d["v"][slots]]
    glob = [torch.empty_like(x) for x in gathered]
    pos_g, pos_glob = pos[slots], torch.empty_like(pos)
    cu = torch.empty(len(case["cu_seqlens"]), dtype=torch.int32, device="cuda:0")
    nd = torch.empty(1, dtype=torch.int32, device="cuda:0")

    def reorder():
        for src, dst in zip(gathered, glob):
            sam.attn_sink_cp_permute_rows(src, slots, True, dst)

    def documents():
        sam.attn_sink_cp_permute_rows(pos_g, slots, True, pos_glob)
        sam.attn_sink_cp_documents(pos_glob, None, cu, nd)
    ms_kv = graph_ms(reorder, steps, warmup)
    ms_doc = graph_ms(documents, steps, warmup)
    nbytes = sum(2 * x.numel() * x.element_size() for x in gathered) + 2 * slots.numel() * 8
    ach = nbytes / (ms_kv * 1e-3) / 1e9
    return {"cp_size": cp_size, "kv_reorder_ms": ms_kv, "kv_reorder_bytes": nbytes, "kv_reorder_GBps": ach,
            "kv_reorder_frac_hbm": ach / PEAK_HBM_GBS, "positions_reorder_and_documents_ms": ms_doc}


def cpu_baseline(case, pairs_row, dqk_dv, budget_s, out_dev, lse_dev):
    """The oracle as it stands, on a seeded row sample sized to ~budget_s."""
    import oracle
    T = case["q"].shape[0]
    g = np.random.default_rng(1234)
    kw = dict(mask_kind=case["mask_kind"], scale=case["scale"], cu_seqlens=case["cu_seqlens"],
              window=case["window"], topk_idx=case["topk_idx"], block_sel=case["block_sel"],
              block_size=case["block_size"], sinks=case["sinks"], sink_mode=case["sink_mode"])
    probe = np.sort(g.choice(T, size=min(T, 64), replace=False))
    t = time.perf_counter()
    oracle.attn_ref(case["q"], case["k"], case["v"], rows=probe, **kw)
    per_pair = max(time.perf_counter() - t, 1e-4) / max(1, int(pairs_row[probe].sum()))
    want_pairs = budget_s / per_pair
    order = g.permutation(T)
    csum = np.cumsum(pairs_row[order])
    n = int(min(T, max(64, np.searchsorted(csum, want_pairs) + 1)))
    rows = np.sort(order[:n])
    # the whole workload may take far less than the budget: repeat the sample
    # until the budget is spent (at most 1000 passes)
    reps, secs = 0, 0.0
    while True:
        t = time.perf_counter()
        ref_o, ref_l = oracle.attn_ref(case["q"], case["k"], case["v"], rows=rows, **kw)
        secs += time.perf_counter() - t
        reps += 1
        if secs >= 0.8 * budget_s or reps >= 1000:
            break
    flops = 2.0 * dqk_dv * float(pairs_row[rows].sum()) * reps
    out = out_dev.float().cpu().numpy().astype(np.float64)[rows]
    lse = lse_dev.cpu().numpy().astype(np.float64)[:, rows]
    fin = np.isfinite(ref_l.T)
    ref_n = np.linalg.norm(ref_o, axis=2)
    nz = fin & (ref_n > 0)
    rel = float((np.linalg.norm(out - ref_o, axis=2)[nz] / ref_n[nz]).max()) if nz.any() else 0.0
    # the pages' statistic: one relative L2 over the whole output tensor
    tens = float(np.linalg.norm(out - ref_o) / np.linalg.norm(ref_o)) if np.linalg.norm(ref_o) > 0 else 0.0
    dl = float(np.abs(lse.T[fin] - ref_l.T[fin]).max()) if fin.any() else 0.0
    assert np.all(out[~fin] == 0.0) and np.all(np.isneginf(lse.T[~fin]))
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} of {T} query rows (all heads), seeded, x{reps} passes; {secs:.1f} s wall; fp64 C enumerator",
            "ms_per_call_equiv": secs / reps * 1e3 * float(pairs_row.sum()) / float(pairs_row[rows].sum())}, \
        {"max_rel_l2": rel, "tensor_rel_l2": tens, "lse_max_abs": dl, "rows_checked": n}


def bench_decode(args, case):
    """The fp8 sparse-MLA decode: two launches per step (list pieces, then the
    LSE merge with the sink), inputs rotated over enough sets to exceed the
    Infinity Cache.  Useful FLOPs count valid (row, key) pairs only; the
    algorithmic bytes are q, out, lse, every distinct cache row touched
    (576 fp8 bytes + its fp32 scale), the index lists and the sinks."""
    import torch
    import sink_aware_masked_amd as sam
    idx = case["topk_idx"]
    T, Hq = case["q"].shape[:2]
    Tk = case["kv_fp8"].shape[0]
    valid = (idx >= 0) & (idx < Tk)
    prow = valid.sum(1).astype(np.int64) * Hq
    F = 2.0 * (576 + 512) * float(prow.sum())
    distinct = np.unique(idx[valid]).size
    B = int(T * Hq * 576 * 2 + T * Hq * 512 * 2 + Hq * T * 4 + distinct * (576 + 4) + idx.nbytes + Hq * 4)
    one = B + int(case["kv_fp8"].nbytes) - distinct * 576  # the whole cache is resident per set
    sets_n = args.sets or max(1, min(16, math.ceil(1.25 * MALL_BYTES / one)))
    log(f"[bench] decode: useful FLOPs {F:.4e}, algorithmic bytes {B:.4e}, sets {sets_n}")
    sets = [sam.decode_case_on_device(case, "cuda:0") for _ in range(sets_n)]
    counter = [0]

    def step():
        d = sets[counter[0] % sets_n]
        counter[0] += 1
        sam.attn_sink_mla_decode_fp8(d["q"], d["kv"], d["kv_scale"], d["topk_idx"], d["sinks"], d["sink_mode"],
                                     d["scale"], d["out"], d["lse"], d["workspace"])
    t0 = time.perf_counter()
    kern_ms = graph_ms(step, args.steps, args.warmup)
    ms = kern_ms  # the graph replay is the whole timed job
    ach = F / (kern_ms * 1e-3) / 1e12
    res = {"metric": METRIC, "value": F / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16 (fp8 e4m3 cache)", "data": "synthetic",
           "config": {"workload": "mla_decode_fp8", "rows": int(T), "q_heads": int(Hq), "kv_entries": int(Tk),
                      "topk": int(idx.shape[1]), "head_dim_qk": 576, "head_dim_v": 512, "cache": "fp8 e4m3 + fp32 row scale",
                      "sink_mode": case["sink_mode"], "cold_cache_sets": sets_n},
           "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_MFMA_BF16_TFS, "unit": "TFLOP/s",
                        "frac": ach / PEAK_MFMA_BF16_TFS, "traffic": None, "kernel_ms": kern_ms,
                        "algorithmic_bytes": B, "useful_flops": F, **both_roofs(F, B, kern_ms)},
           "device": device_facts(), "wall_s": time.perf_counter() - t0}
    d = sets[0]
    sam.attn_sink_mla_decode_fp8(d["q"], d["kv"], d["kv_scale"], d["topk_idx"], d["sinks"], d["sink_mode"],
                                 d["scale"], d["out"], d["lse"], d["workspace"])
    torch.cuda.synchronize()
    if args.cpu_seconds > 0:
        from oracle import fp8
        g = np.random.default_rng(1234)
        rows = np.sort(g.choice(T, size=min(T, 8), replace=False))
        reps, secs = 0, 0.0
        while secs < 0.8 * args.cpu_seconds and reps < 100:
            t = time.perf_counter()
            ref_o, ref_l = fp8.decode_ref(case, rows=rows)
            secs += time.perf_counter() - t
            reps += 1
        import oracle
        flops = 2.0 * 1088 * float(prow[rows].sum()) * reps
        out = d["out"].float().cpu().numpy().astype(np.float64)[rows]
        num = np.linalg.norm(out - ref_o, axis=2)
        den = np.linalg.norm(ref_o, axis=2)
        nz = den > 0
        res["cpu_baseline"] = {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
                               "kind": "oracle",
                               "sample": f"{len(rows)} of {T} rows (all heads), seeded, x{reps} passes; {secs:.1f} s wall; "
                                         "fp64 C enumerator after an fp64 NumPy dequantization of the cache"}
        res["parity_sample"] = {"max_rel_l2": float((num[nz] / den[nz]).max()),
                                "tensor_rel_l2": float(np.linalg.norm(out - ref_o) / np.linalg.norm(ref_o)),
                                "lse_max_abs": float(np.abs(d["lse"].cpu().numpy()[:, rows] - ref_l).max()),
                                "rows_checked": int(len(rows))}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


def both_roofs(F: float, B: float, kern_ms: float) -> dict:
    """The launch against both roofs: useful FLOP/s against the MFMA peak and
    algorithmic bytes/s against the HBM peak (the binding one is `frac`)."""
    t = kern_ms * 1e-3
    return {"hbm_GBps": B / t / 1e9, "hbm_frac": B / t / 1e9 / PEAK_HBM_GBS,
            "mfma_TFLOPs": F / t / 1e12, "mfma_frac": F / t / 1e12 / PEAK_MFMA_BF16_TFS}


def device_facts(copy_bytes: int = 1 << 30, reps: int = 10) -> dict:
    """What the device reports (name, compute units, architecture) and the HBM
    bandwidth two plain copies of copy_bytes reach here (bytes read + written
    per second): torch's device copy, and the library's row gather
    (attn_sink_cp_permute_rows) with the identity index over 64 KB rows."""
    import torch
    import sink_aware_masked_amd as sam
    props = torch.cuda.get_device_properties(0)
    a = torch.empty(copy_bytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    rows = copy_bytes // 65536
    a2, b2 = a.view(rows, 65536), b.view(rows, 65536)
    ident = torch.arange(rows, dtype=torch.int64, device="cuda:0")

    def rate(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 2 * copy_bytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9

    torch_gbs = rate(lambda: b.copy_(a))
    rows_gbs = rate(lambda: sam.attn_sink_cp_permute_rows(a2, ident, False, b2))
    assert torch.equal(a, b)
    del a, b, a2, b2, ident
    torch.cuda.empty_cache()
    return {"name": props.name, "compute_units": props.multi_processor_count,
            "arch": getattr(props, "gcnArchName", None), "copy_bytes": 2 * copy_bytes,
            "copy_GBps_torch": torch_gbs, "copy_GBps_row_gather": rows_gbs, "latent_gather": latent_gather()}


def latent_gather(rows: int = 65536, row_bytes: int = 1152, n: int = 1 << 18, reps: int = 10) -> dict:
    """The access pattern of the sparse-MLA kernel's gathered stream, timed
    through the library's row gather (attn_sink_cp_permute_rows, gather mode):
    n uniformly random 1152-byte rows (one bf16 latent row of 576 values) of a
    65536-row table, written densely.  read_GBps counts the gathered bytes
    only; rw_GBps adds the dense writes, which the attention kernel does not
    make."""
    import torch
    import sink_aware_masked_amd as sam
    tbl = torch.randint(0, 255, (rows, row_bytes), dtype=torch.uint8, device="cuda:0")
    g = torch.Generator(device="cpu").manual_seed(7)
    idx = torch.randint(0, rows, (n,), generator=g, dtype=torch.int64).to("cuda:0")
    dst = torch.empty((n, row_bytes), dtype=torch.uint8, device="cuda:0")
    for _ in range(2):
        sam.attn_sink_cp_permute_rows(tbl, idx, False, dst)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        sam.attn_sink_cp_permute_rows(tbl, idx, False, dst)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    probe = torch.randint(0, n, (64,), generator=g)
    assert torch.equal(dst[probe.to("cuda:0")], tbl[idx[probe.to("cuda:0")]])
    del tbl, dst, idx
    torch.cuda.empty_cache()
    return {"table_rows": rows, "row_bytes": row_bytes, "gathered_rows": n, "ms": t * 1e3,
            "read_GBps": n * row_bytes / t / 1e9, "rw_GBps": 2 * n * row_bytes / t / 1e9}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="blocksparse_32k",
                    choices=["window_4k", "window_16k", "mla_topk", "blocksparse_32k", "blocksparse_32k_coherent",
                             "mla_decode_fp8"])
    ap.add_argument("--sink-mode", default=None, choices=[None, "none", "key0_bias", "null_logit"],
                    help="default: the workload's own (key0_bias for window, null_logit for the others; "
                         "blocksparse_32k: null_logit)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--gqa", action="store_true", help="window_4k: the GQA variant (16 query heads over 4 kv heads)")
    ap.add_argument("--sets", type=int, default=0, help="input sets to rotate (0: enough to exceed the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample budget (0: skip)")
    ap.add_argument("--compare-sink-none", action="store_true",
                    help="also time the same workload without a sink and report the ratio "
                         "(always on for the default block-sparse workload)")
    ap.add_argument("--compare-unfused", action="store_true",
                    help="window workloads: also time the no-sink kernel + closed-form key-0 correction")
    ap.add_argument("--measure-merge", action="store_true",
                    help="top-k workload: also time the split-in-two path and the LSE merge kernel")
    ap.add_argument("--measure-cp", action="store_true",
                    help="block-sparse workload: also time the context-parallel K/V reorder and document derivation")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps one by one instead of replaying a captured graph")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this size (PMC scaling reference)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path (each GPU runs the same kernels on its own share); "
              "run with --gpus 1", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    lib = os.path.join(ROOT, "sink_aware_masked_amd", "libattn_sink.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.build()

    if args.gqa and args.workload != "window_4k":
        print("--gqa applies to the window_4k workload only", file=sys.stderr)
        return 2
    workload = args.workload + ("_gqa" if args.gqa else "")
    sink_mode = args.sink_mode
    if sink_mode is None and args.workload.startswith("blocksparse_32k"):
        sink_mode = "null_logit"      # the layer's sink pass; the no-sink pass is timed beside it
        args.compare_sink_none = True
    log(f"[bench] building workload {workload} seed {args.seed}")
    case = build_case(args.workload, args.seed, sink_mode, args.gqa)
    if case["mask_kind"] == "topk_fp8":
        return bench_decode(args, case)
    prow = pairs_per_row(case)
    dqk, dv = case["q"].shape[2], case["v"].shape[2]
    F = 2.0 * (dqk + dv) * float(prow.sum())
    B = algorithmic_bytes(case)
    sets_n = args.sets or max(1, min(16, math.ceil(1.25 * MALL_BYTES / B)))
    log(f"[bench] useful FLOPs {F:.4e}, algorithmic bytes {B:.4e}, sets {sets_n}")

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calibrate_copy} MiB done")

    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup")
    ms, kern_ms, dev0, stats = time_gpu(case, sets_n, args.steps, args.warmup, use_graph=not args.no_graph)
    kind = case["mask_kind"]
    bound = "hbm" if kind == "window" else "mfma"
    if bound == "hbm":
        ach = B / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS}
    else:
        ach = F / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_MFMA_BF16_TFS, "unit": "TFLOP/s",
                "frac": ach / PEAK_MFMA_BF16_TFS}
    roof["traffic"] = load_traffic(workload + ":" + case["sink_mode"], kind)
    roof.update(both_roofs(F, B, kern_ms))
    roof["kernel_ms"] = kern_ms
    roof["launch_ms"] = stats
    roof["algorithmic_bytes"] = B
    roof["useful_flops"] = F

    value = F / (ms * 1e-3) / 1e12
    page = PAGE_MS.get((workload, case["sink_mode"]))
    res = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": case["dtype"], "data": "synthetic",
           "config": describe(workload, case, sets_n), "roofline": roof, "device": device_facts()}
    if page:
        res["page_context"] = {"page_ms": page, "page_over_ours": page / ms,
                               "note": "the MiMo page's H100 time for the same shape (FlashAttention varlen"
                                       + (" + the unfused key-0 correction" if case["sink_mode"] == "key0_bias" else "")
                                       + "); another machine and design, context only"}

    if args.compare_sink_none and case["sink_mode"] != "none":
        base = dict(case, sink_mode="none", sinks=None)
        ms0, kern0, _, stats0 = time_gpu(base, sets_n, args.steps, args.warmup, use_graph=not args.no_graph)
        res["sink_vs_none"] = {"kernel_ms_sink": kern_ms, "kernel_ms_none": kern0,
                               "ratio": kern_ms / kern0, "ms_per_step_none": ms0,
                               "median_ms_sink": stats["median_ms"], "median_ms_none": stats0["median_ms"],
                               "median_ratio": stats["median_ms"] / stats0["median_ms"]}

    if args.compare_unfused:
        if kind != "window" or case["sink_mode"] != "key0_bias":
            print("--compare-unfused needs a window workload with the key0_bias sink", file=sys.stderr)
            return 2
        log("[bench] unfused key-0 correction")
        res["unfused_key0"] = compare_unfused(case, args.steps, args.warmup, kern_ms)
    if args.measure_merge:
        if kind != "topk":
            print("--measure-merge needs the top-k workload", file=sys.stderr)
            return 2
        log("[bench] split-in-two + merge")
        res["split_merge"] = measure_merge(case, args.steps, args.warmup, kern_ms)

    if args.measure_cp:
        if kind != "blocksel":
            print("--measure-cp needs the block-sparse workload", file=sys.stderr)
            return 2
        log("[bench] context-parallel reorder")
        res["cp_reorder"] = measure_cp(case, args.steps, args.warmup)

    if args.cpu_seconds > 0:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cb, parity = cpu_baseline(case, prow, dqk + dv, args.cpu_seconds, dev0["out"], dev0["lse"])
        res["cpu_baseline"] = cb
        res["parity_sample"] = parity
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
