"""Seeded synthetic inputs for sink-aware masked attention.

This module only draws random inputs; it holds none of the method's arithmetic
(no logits, masks or softmax).  Both sides of every comparison -- the CPU
oracle and the HIP library -- read the arrays it returns, so they see the same
bits.  Every draw comes from ``numpy.random.Generator(PCG64(seed))``; bf16
inputs are drawn in float32 and rounded to bf16 (round to nearest even), then
kept as float32 arrays whose values are exactly representable in bf16.

A *case* is a plain dict:

    name, dtype ('bf16' | 'f32'), q [T,Hq,Dqk], k [Tk,Hkv,Dqk], v [Tk,Hkv,Dv]
    (for the shared-latent MLA layout ``v`` is a view of ``k[..., :Dv]`` and
    ``v_aliases_k`` is True), mask_kind ('window' | 'topk' | 'blocksel'),
    cu_seqlens (int32), window, topk_idx (int32 [T,topk], -1 padding),
    block_sel (uint8 [1,Hidx,T,NB]), block_size, sinks (float32 [Hq] or None),
    sink_mode ('none' | 'key0_bias' | 'null_logit'), scale.

The five named workloads follow the shapes, value ranges and structure of the
three source pages (see ``WORKLOADS``); none of them reads any data file.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "rng", "round_bf16", "bf16_bits", "window_case", "topk_case", "blocksel_case",
    "tiny_window", "tiny_wide_window", "c3_seqlens", "c5_doc_lens", "WORKLOADS", "make_workload",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def round_bf16(x, inplace: bool = False) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    if not (inplace and isinstance(x, np.ndarray) and x.dtype == np.float32 and x.flags.c_contiguous):
        x = np.array(x, dtype=np.float32, copy=True, order="C")
    flat = x.reshape(-1).view(np.uint32)
    step = 1 << 22
    lsb = np.empty(min(step, flat.size), dtype=np.uint32)
    for s in range(0, flat.size, step):
        u = flat[s:s + step]
        t = lsb[:u.size]
        # finite inputs only: u <= 0xFF7FFFFF, so adding at most 0x8000 cannot wrap
        np.bitwise_and(u, np.uint32(0x10000), out=t)
        t >>= np.uint32(16)
        u += np.uint32(0x7FFF)
        u += t
        u &= np.uint32(0xFFFF0000)
    return x


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of bf16-representable float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _values(g: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_bf16(x, inplace=True) if dtype == "bf16" else x


def _sinks(g, Hq: int, sink_mode: str, sink_range) -> np.ndarray | None:
    if sink_mode == "none":
        return None
    lo, hi = sink_range
    return g.uniform(lo, hi, size=Hq).astype(np.float32)


def _cu(lens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


def window_case(seqlens, Hq: int, Hkv: int, D: int, W: int, *, dtype: str = "bf16",
                sink_mode: str = "key0_bias", sink_range=(-0.1, 0.6), seed: int = 0,
                scale: float | None = None, Dv: int | None = None, name: str = "window") -> dict:
    g = rng(seed)
    T = int(np.sum(seqlens))
    Dv = D if Dv is None else Dv
    q = _values(g, (T, Hq, D), 1.0, dtype)
    k = _values(g, (T, Hkv, D), 1.0, dtype)
    v = _values(g, (T, Hkv, Dv), 1.0, dtype)
    return dict(name=name, dtype=dtype, q=q, k=k, v=v, v_aliases_k=False, mask_kind="window",
                cu_seqlens=_cu(seqlens), window=int(W), topk_idx=None, block_sel=None,
                block_size=None, sinks=_sinks(g, Hq, sink_mode, sink_range), sink_mode=sink_mode,
                scale=float(1.0 / math.sqrt(D) if scale is None else scale))


def _distinct(g, N: int, n: int) -> np.ndarray:
    """n distinct indices drawn uniformly from [0, N), in draw order."""
    if 4 * n > N:
        return g.permutation(N)[:n].astype(np.int32)
    out = np.empty(0, dtype=np.int64)
    while len(out) < n:
        x = np.concatenate([out, g.integers(0, N, size=n + n // 8 + 8)])
        _, first = np.unique(x, return_index=True)
        out = x[np.sort(first)]
    return out[:n].astype(np.int32)


def topk_case(T: int, Tk: int, Hq: int, Dqk: int, Dv: int, topk: int, *, counts=(1, 4, 16, 128, 512, 2048),
              shuffled: bool = False, mla: bool = True, Hkv: int = 1, std: float = 0.5, dtype: str = "bf16",
              sink_mode: str = "null_logit", sink_range=(-2.20, 2.49), seed: int = 0,
              scale: float | None = None, out_of_range: bool = False, name: str = "topk") -> dict:
    """Per-row top-k lists: the valid count is uniform over ``counts`` (clipped to
    topk and Tk); indices are distinct and uniform in [0, Tk); valid entries come
    first, then -1 -- or, with ``shuffled``, -1 entries are interleaved at random
    positions.  ``out_of_range`` also plants indices >= Tk and < -1 among the
    padding (both are padding by the library's contract)."""
    g = rng(seed)
    q = _values(g, (T, Hq, Dqk), std, dtype)
    if mla:
        kv = _values(g, (Tk, 1, Dqk), std, dtype)
        k, v = kv, kv[:, :, :Dv]
    else:
        k = _values(g, (Tk, Hkv, Dqk), std, dtype)
        v = _values(g, (Tk, Hkv, Dv), std, dtype)
    idx = np.full((T, topk), -1, dtype=np.int32)
    cnt = np.minimum(np.asarray(counts)[g.integers(0, len(counts), size=T)], min(topk, Tk))
    for i in range(T):
        n = int(cnt[i])
        sel = _distinct(g, Tk, n)
        if shuffled:
            pos = np.sort(g.choice(topk, size=n, replace=False))
            idx[i, pos] = sel
        else:
            idx[i, :n] = sel
        if out_of_range and n < topk:
            pad = np.flatnonzero(idx[i] == -1)
            bad = g.choice(pad, size=max(1, len(pad) // 3), replace=False)
            idx[i, bad] = np.where(g.random(len(bad)) < 0.5, Tk + g.integers(0, 1000, len(bad)),
                                   -2 - g.integers(0, 1000, len(bad)))
    return dict(name=name, dtype=dtype, q=q, k=k, v=v, v_aliases_k=bool(mla), mask_kind="topk",
                cu_seqlens=None, window=None, topk_idx=idx, block_sel=None, block_size=None,
                sinks=_sinks(g, Hq, sink_mode, sink_range), sink_mode=sink_mode,
                scale=float(1.0 / math.sqrt(Dqk) if scale is None else scale))


def _block_table(g, doc_lens, Hidx: int, block_size: int, n_random: int, coherent: bool = False) -> np.ndarray:
    """[1, Hidx, T, NB] uint8: per (index head, query) the query's own block
    i // block_size plus min(n_random, c) distinct uniform picks among the c
    earlier blocks that overlap the query's document.  With ``coherent`` the
    picks are drawn once per (index head, query block, document) and shared by
    its queries (a labelled extra, not the per-query workload)."""
    if coherent:
        return _block_table_coherent(g, doc_lens, Hidx, block_size, n_random)
    T = int(np.sum(doc_lens))
    NB = -(-T // block_size)
    cu = _cu(doc_lens)
    doc_start = np.repeat(cu[:-1], np.asarray(doc_lens)).astype(np.int64)      # per token
    diag = np.arange(T, dtype=np.int64) // block_size
    lo = doc_start // block_size
    table = np.zeros((1, Hidx, T, NB), dtype=np.uint8)
    cols = np.arange(NB, dtype=np.int64)[None, :]
    chunk = 4096
    for hi in range(Hidx):
        for r0 in range(0, T, chunk):
            r1 = min(T, r0 + chunk)
            key = g.random((r1 - r0, NB))
            cand = (cols >= lo[r0:r1, None]) & (cols < diag[r0:r1, None])
            key = np.where(cand, key, 2.0)
            k_sel = min(n_random, NB)
            pick = np.argpartition(key, k_sel - 1, axis=1)[:, :k_sel] if k_sel < NB else np.argsort(key, axis=1)
            ok = np.take_along_axis(key, pick, axis=1) < 1.0
            rows = np.broadcast_to(np.arange(r0, r1)[:, None], pick.shape)
            table[0, hi, rows[ok], pick[ok]] = 1
            table[0, hi, np.arange(r0, r1), diag[r0:r1]] = 1
    return table


def _block_table_coherent(g, doc_lens, Hidx: int, block_size: int, n_random: int) -> np.ndarray:
    T = int(np.sum(doc_lens))
    NB = -(-T // block_size)
    cu = _cu(doc_lens)
    table = np.zeros((1, Hidx, T, NB), dtype=np.uint8)
    for hi in range(Hidx):
        for d in range(len(doc_lens)):
            s0, s1 = int(cu[d]), int(cu[d + 1])
            lo = s0 // block_size
            for qb in range(s0 // block_size, (s1 - 1) // block_size + 1):
                r0, r1 = max(s0, qb * block_size), min(s1, (qb + 1) * block_size)
                cand = np.arange(lo, qb)
                pick = g.permutation(cand)[:min(n_random, len(cand))]
                table[0, hi, r0:r1, pick] = 1
                table[0, hi, r0:r1, qb] = 1
    return table


def blocksel_case(doc_lens, Hq: int, Hkv: int, D: int, *, block_size: int = 64, n_random: int = 15,
                  Hidx: int | None = None, dtype: str = "bf16", sink_mode: str = "none",
                  sink_range=(-2.0, 2.0), seed: int = 0, scale: float | None = None,
                  coherent: bool = False, name: str = "blocksel") -> dict:
    g = rng(seed)
    T = int(np.sum(doc_lens))
    Hidx = Hkv if Hidx is None else Hidx
    q = _values(g, (T, Hq, D), 1.0, dtype)
    k = _values(g, (T, Hkv, D), 1.0, dtype)
    v = _values(g, (T, Hkv, D), 1.0, dtype)
    table = _block_table(g, doc_lens, Hidx, block_size, n_random, coherent=coherent)
    return dict(name=name, dtype=dtype, q=q, k=k, v=v, v_aliases_k=False, mask_kind="blocksel",
                cu_seqlens=_cu(doc_lens), window=None, topk_idx=None, block_sel=table,
                block_size=int(block_size), sinks=_sinks(g, Hq, sink_mode, sink_range),
                sink_mode=sink_mode, scale=float(1.0 / math.sqrt(D) if scale is None else scale))


def mla_decode_fp8_case(T: int, Tk: int, Hq: int, topk: int, *, counts=(2048,), shuffled: bool = False,
                        out_of_range: bool = False, sink_mode: str = "null_logit", sink_range=(-2.20, 2.49),
                        std: float = 0.5, seed: int = 0, name: str = "mla_decode_fp8") -> dict:
    """Decode rows over an fp8 latent cache: q bf16 N(0, std^2) [T, Hq, 576];
    cache rows drawn N(0, std^2) in fp32, each stored as 576 fp8 e4m3 bytes
    (round to nearest even, by torch's float8_e4m3fn conversion) with one fp32
    scale per row, amax / 448 rounded up to an 8-bit mantissa (so scale times
    any e4m3 value is exact in fp32).  Top-k lists as in topk_case.  The fp32
    rows before rounding are kept as ``kv_source`` [Tk, 576]."""
    import torch
    base = topk_case(T, Tk, Hq, 576, 512, topk, counts=counts, shuffled=shuffled, mla=True, std=std,
                     sink_mode=sink_mode, sink_range=sink_range, seed=seed, out_of_range=out_of_range, name=name)
    g = rng(50_000 + seed)
    x = g.standard_normal((Tk, 576), dtype=np.float32) * np.float32(std)
    amax = np.maximum(np.abs(x).max(axis=1), np.float32(1e-6))
    sc = (amax / np.float32(448.0)).astype(np.float32)
    bits = sc.view(np.uint32)
    up = (bits & np.uint32(0xFFFF)) != 0
    sc = ((bits & np.uint32(0xFFFF0000)) + (up.astype(np.uint32) << np.uint32(16))).view(np.float32)  # round up
    q8 = torch.from_numpy(x / sc[:, None]).to(torch.float8_e4m3fn)
    fp8 = q8.view(torch.uint8).numpy().reshape(Tk, 1, 576).copy()
    base.update(kv_fp8=fp8, kv_scale=sc.astype(np.float32), kv_source=x, k=None, v=None, v_aliases_k=True,
                mask_kind="topk_fp8")
    return base


def c3_seqlens(seed: int, total: int = 16384, nseq: int = 8, W: int = 64) -> list[int]:
    """One length uniform in 1..W-1 (shorter than the window); the other nseq-1
    lengths from nseq-2 sorted uniform cut points over the remainder; the short
    sequence sits at a seeded random position."""
    g = rng(10_000 + seed)
    short = int(g.integers(1, W))
    rest = total - short
    while True:
        cuts = np.sort(g.choice(np.arange(1, rest), size=nseq - 2, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [rest]])).astype(int).tolist()
        if min(lens) >= W:
            break
    pos = int(g.integers(0, nseq))
    lens.insert(pos, short)
    return lens


def c5_doc_lens(seed: int, total: int = 32768, ndoc: int = 4, block: int = 64, min_len: int = 256) -> list[int]:
    """ndoc seeded random document lengths summing to total, no boundary on a
    multiple of the key block size."""
    g = rng(20_000 + seed)
    while True:
        cuts = np.sort(g.choice(np.arange(1, total), size=ndoc - 1, replace=False))
        if np.any(cuts % block == 0):
            continue
        lens = np.diff(np.concatenate([[0], cuts, [total]])).astype(int).tolist()
        if min(lens) >= min_len:
            return lens


def tiny_window(seed: int = 0, **kw) -> dict:
    return window_case([96, 160], 4, 4, 64, 16, **{"dtype": "f32", "sink_range": (-0.1, 0.6),
                                                   "scale": 0.125, "seed": seed, **kw})


def tiny_wide_window(seed: int = 0, **kw) -> dict:
    return window_case([5, 40, 19], 4, 2, 32, 1 << 20, **{"dtype": "f32", "seed": seed, **kw})


# The five named workloads.  Values: bf16 draws from N(0, std^2) rounded to
# bf16 (fp32 for the tiny case); sinks uniform in the stated range.
WORKLOADS = {
    # MiMo page (window attention sink fix): its unit test uses one sequence
    # shorter than the window and one longer; tiny fp32 case.
    "tiny_window_f32": lambda seed=0, **kw: tiny_window(seed, **kw),
    # MiMo page "Cost" paragraph: 4096 tokens, 16 heads, head dim 80, window 64.
    "window_4k": lambda seed=0, sink_range=(-0.1, 0.6), gqa=False, sink_mode="key0_bias": window_case(
        [2048, 2048], 16, 4 if gqa else 16, 80, 64, dtype="bf16", sink_mode=sink_mode,
        sink_range=sink_range, seed=seed, name="window_4k" + ("_gqa" if gqa else "")),
    # Same paragraph's 16384-token point, as 8 packed sequences, one shorter than W.
    "window_16k": lambda seed=0, sink_mode="key0_bias": window_case(
        c3_seqlens(seed), 16, 16, 80, 64, dtype="bf16", sink_mode=sink_mode,
        sink_range=(-2.0, 2.0), seed=seed, name="window_16k"),
    # DeepSeek-V4 sparse-MLA page: 64 heads over one latent KV (576 = 512 + 64),
    # top-k 2048 with the page's valid-key buckets, sinks in [-2.20, 2.49].
    "mla_topk": lambda seed=0, sink_mode="null_logit", **kw: topk_case(
        4096, 65536, 64, 576, 512, 2048, sink_mode=sink_mode, seed=seed, name="mla_topk", **kw),
    # Same page, decode call site: 128 decode rows x 64 heads over an fp8 latent
    # cache of 65536 rows, full 2048-entry lists (steady-state decode).
    "mla_decode_fp8": lambda seed=0, sink_mode="null_logit", **kw: mla_decode_fp8_case(
        128, 65536, 64, 2048, sink_mode=sink_mode, seed=seed, **kw),
    # MiniMax-M3 CP sparse-attention page: block-sparse causal over 4 packed
    # documents, 32 q heads / 8 kv heads, head dim 128, 64-token key blocks.
    "blocksparse_32k": lambda seed=0, sink_mode="none": blocksel_case(
        c5_doc_lens(seed), 32, 8, 128, block_size=64, n_random=15, sink_mode=sink_mode,
        sink_range=(-2.0, 2.0), seed=seed, name="blocksparse_32k"),
    # Labelled extra: the same layer with the 15 earlier blocks drawn once per
    # 64-query block (shared by its queries), as a selection that neighbouring
    # queries agree on would look; not the per-query workload above.
    "blocksparse_32k_coherent": lambda seed=0, sink_mode="none": blocksel_case(
        c5_doc_lens(seed), 32, 8, 128, block_size=64, n_random=15, sink_mode=sink_mode,
        sink_range=(-2.0, 2.0), seed=seed, coherent=True, name="blocksparse_32k_coherent"),
}


def make_workload(name: str, seed: int = 0, **kw) -> dict:
    return WORKLOADS[name](seed=seed, **kw)
