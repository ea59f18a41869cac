"""CPU oracle for sink-aware masked attention (forward): TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and the two share no code.

Two independent fp64 implementations of the same plain definition:

* :func:`attn_ref` -- ``ref.c``, a C enumerator (OpenMP over (row, head)) that
  lists each row's valid keys and sums over them in double.  It runs on all
  rows of small cases, on sampled rows of full-size cases, and it is the timed
  CPU baseline.
* :func:`oracle.dense.attn_dense` -- a NumPy twin that builds explicit dense
  mask / bias / null-key matrices and applies a textbook softmax.

Both take the same keyword arguments and return ``(out[R, Hq, Dv], lse[Hq, R])``
in float64, where R is the number of evaluated rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .dense import MASK_KINDS, SINK_MODES, attn_dense  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ref.c")
_LIB = os.path.join(_HERE, "libattn_oracle.so")
_lib = None


def build_oracle(force: bool = False) -> str:
    """Compile ref.c with gcc (plain -O2, no fast-math) into libattn_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-Wall", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build_oracle()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_fwd.argtypes = [
            P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, ctypes.c_double, P,
            ctypes.c_int64, P, P]
        lib.oracle_blocksel_offset.restype = ctypes.c_int64
        lib.oracle_blocksel_offset.argtypes = [ctypes.c_int64] * 7
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def blocksel_flat_offset(b, h, q, kb, H, S, NB) -> int:
    """64-bit flat offset of [b, h, q, kb] in a [B, H, S, NB] table (as ref.c uses it)."""
    return int(_load().oracle_blocksel_offset(b, h, q, kb, H, S, NB))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def attn_ref(q, k, v, *, mask_kind: str, scale: float, cu_seqlens=None, window=None,
             topk_idx=None, block_sel=None, block_size=None, sinks=None,
             sink_mode: str = "none", rows=None):
    """fp64 oracle via the C enumerator.  Inputs: float32-representable arrays."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    T, Hq, Dqk = q.shape
    Tk, Hkv, Dk = k.shape
    Dv = v.shape[2]
    if Dk != Dqk or v.shape[0] != Tk or v.shape[1] != Hkv:
        raise ValueError("q/k/v shapes disagree")
    kind = MASK_KINDS.index(mask_kind)
    mode = SINK_MODES.index(sink_mode)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ti = None if topk_idx is None else np.ascontiguousarray(topk_idx, dtype=np.int32)
    bsel = None if block_sel is None else np.ascontiguousarray(block_sel, dtype=np.uint8)
    sk = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float64)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = T if r is None else len(r)
    out = np.empty((nrows, Hq, Dv), dtype=np.float64)
    lse = np.empty((Hq, nrows), dtype=np.float64)
    if nrows == 0:
        return out, lse
    rc = lib.oracle_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), T, Tk, Hq, Hkv, Dqk, Dv,
        _ptr(cu), 0 if cu is None else len(cu) - 1, kind, int(window or 0),
        _ptr(ti), 0 if ti is None else ti.shape[1],
        _ptr(bsel), 0 if bsel is None else bsel.shape[1], 0 if bsel is None else bsel.shape[3],
        int(block_size or 0), _ptr(sk), mode, float(scale), _ptr(r), nrows, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd rejected its arguments (rc={rc})")
    return out, lse
