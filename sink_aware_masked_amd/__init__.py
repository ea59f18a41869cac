"""Python binding of the sink-aware masked attention forward library (gfx950).

Argument marshalling only: torch tensors supply device pointers, sizes,
strides and the current HIP stream; every step of the computation runs in the
HIP kernels of ``libattn_sink.so`` behind the C ABI declared in
``include/attn_sink.h``.  There is no fallback: if the library is missing the
import fails, and if a call is rejected the C status is raised.

Names mirror the C ABI: :func:`attn_sink_fwd`, :func:`attn_sink_check`,
:func:`attn_sink_strerror`, :func:`attn_sink_abi_version`.  :func:`fwd` is the
same call with keyword arguments that also allocates ``out`` / ``lse``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_sink.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python __graft_entry__.py` (hipcc, gfx950) first")
_lib = ctypes.CDLL(LIB_PATH)

MASK_KINDS = {"window": 0, "topk": 1, "blocksel": 2}
SINK_MODES = {"none": 0, "key0_bias": 1, "null_logit": 2}
DTYPE_BF16, DTYPE_F32, DTYPE_I32, DTYPE_U8, DTYPE_I64, DTYPE_FP8_E4M3 = 0, 1, 2, 3, 4, 5
STATUS = {0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_ENUM", -3: "ATTN_ERR_SHAPE",
          -4: "ATTN_ERR_STRIDE", -5: "ATTN_ERR_HEADS", -6: "ATTN_ERR_DTYPE",
          -7: "ATTN_ERR_UNSUPPORTED", -8: "ATTN_ERR_RANGE", -9: "ATTN_ERR_LAUNCH"}
EXPORTS = ("attn_sink_fwd", "attn_sink_check", "attn_sink_key0_correct", "attn_sink_key0_correct_check",
           "attn_sink_merge", "attn_sink_merge_check", "attn_sink_cp_slots", "attn_sink_cp_slots_check",
           "attn_sink_cp_permute_rows", "attn_sink_cp_permute_rows_check", "attn_sink_cp_documents",
           "attn_sink_cp_documents_check", "attn_sink_mla_decode_fp8", "attn_sink_mla_decode_fp8_check",
           "attn_sink_mla_decode_fp8_workspace", "attn_sink_mla_decode_fp8_noalloc", "attn_sink_strerror",
           "attn_sink_abi_version")
DECODE_SCRATCH_BYTES = 96 << 20
MERGE_MAX_PARTS = 8


class AttnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class AttnMaskArg(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("topk_idx", ctypes.POINTER(AttnTensor)), ("block_sel", ctypes.POINTER(AttnTensor))]


_P = ctypes.c_void_p
_T = ctypes.POINTER(AttnTensor)
_lib.attn_sink_fwd.restype = ctypes.c_int
_lib.attn_sink_fwd.argtypes = [_T, _T, _T, _P, ctypes.c_int32, ctypes.c_int32,
                               ctypes.POINTER(AttnMaskArg), _P, ctypes.c_int32, ctypes.c_float,
                               _T, _P, _P]
_lib.attn_sink_check.restype = ctypes.c_int
_lib.attn_sink_check.argtypes = [_T, _T, _T, _P, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.POINTER(AttnMaskArg), _P, ctypes.c_int32, ctypes.c_float,
                                 _T, _P]
_K0 = [_T, _T, _T, _P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_float, _T, _P]
_lib.attn_sink_key0_correct.restype = ctypes.c_int
_lib.attn_sink_key0_correct.argtypes = _K0 + [_P]
_lib.attn_sink_key0_correct_check.restype = ctypes.c_int
_lib.attn_sink_key0_correct_check.argtypes = _K0
_MG = [_T, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, _P, ctypes.c_int32, _T, _P]
_lib.attn_sink_merge.restype = ctypes.c_int
_lib.attn_sink_merge.argtypes = _MG + [_P]
_lib.attn_sink_merge_check.restype = ctypes.c_int
_lib.attn_sink_merge_check.argtypes = _MG
_I64, _I32 = ctypes.c_int64, ctypes.c_int32
_lib.attn_sink_cp_slots.restype = ctypes.c_int
_lib.attn_sink_cp_slots.argtypes = [_I32, _I64, _I32, _P, _P]
_lib.attn_sink_cp_slots_check.restype = ctypes.c_int
_lib.attn_sink_cp_slots_check.argtypes = [_I32, _I64, _I32, _P]
_lib.attn_sink_cp_permute_rows.restype = ctypes.c_int
_lib.attn_sink_cp_permute_rows.argtypes = [_T, _P, _I64, _I32, _T, _P]
_lib.attn_sink_cp_permute_rows_check.restype = ctypes.c_int
_lib.attn_sink_cp_permute_rows_check.argtypes = [_T, _P, _I64, _I32, _T]
_lib.attn_sink_cp_documents.restype = ctypes.c_int
_lib.attn_sink_cp_documents.argtypes = [_P, _I64, _P, _P, _I32, _P, _P]
_lib.attn_sink_cp_documents_check.restype = ctypes.c_int
_lib.attn_sink_cp_documents_check.argtypes = [_P, _I64, _P, _P, _I32, _P]
_DEC = [_T, _T, _P, _T, _P, _I32, ctypes.c_float, _T, _P, _P, _I64]
_lib.attn_sink_mla_decode_fp8.restype = ctypes.c_int
_lib.attn_sink_mla_decode_fp8.argtypes = _DEC + [_P]
_lib.attn_sink_mla_decode_fp8_check.restype = ctypes.c_int
_lib.attn_sink_mla_decode_fp8_check.argtypes = _DEC
_lib.attn_sink_mla_decode_fp8_noalloc.restype = ctypes.c_int
_lib.attn_sink_mla_decode_fp8_noalloc.argtypes = [_T, _T, _P, _T, _P, _I32, ctypes.c_float, _T, _P, _P]
_lib.attn_sink_mla_decode_fp8_workspace.restype = ctypes.c_int
_lib.attn_sink_mla_decode_fp8_workspace.argtypes = [_I64, _I64, _I64, ctypes.POINTER(ctypes.c_int64)]
_lib.attn_sink_strerror.restype = ctypes.c_char_p
_lib.attn_sink_strerror.argtypes = [ctypes.c_int]
_lib.attn_sink_abi_version.restype = ctypes.c_int
_lib.attn_sink_abi_version.argtypes = []


class AttnSinkError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {attn_sink_strerror(status)}")


def attn_sink_strerror(status: int) -> str:
    return _lib.attn_sink_strerror(int(status)).decode()


def attn_sink_abi_version() -> int:
    return int(_lib.attn_sink_abi_version())


def _dtype_code(t) -> int:
    import torch
    codes = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32, torch.int32: DTYPE_I32,
             torch.uint8: DTYPE_U8, torch.bool: DTYPE_U8, torch.int64: DTYPE_I64,
             torch.float8_e4m3fn: DTYPE_FP8_E4M3}
    if t.dtype not in codes:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return codes[t.dtype]


def desc(t, *, data=None, dtype=None, shape=None, stride=None) -> AttnTensor:
    """Descriptor of a torch tensor (or of explicit fields, for host-side checks)."""
    d = AttnTensor()
    if t is not None:
        data = t.data_ptr() if data is None else data
        dtype = _dtype_code(t) if dtype is None else dtype
        shape = tuple(t.shape) if shape is None else shape
        stride = tuple(t.stride()) if stride is None else stride
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    for i, (s, st) in enumerate(zip(shape, stride)):
        d.shape[i] = int(s)
        d.stride[i] = int(st)
    return d


def _ptr(t):
    return None if t is None else (t if isinstance(t, int) else t.data_ptr())


def _ref(x):
    return None if x is None else ctypes.byref(x)


def _on_device(name, t, device):
    """Raise unless t is a torch tensor on `device` (a host pointer handed to a
    kernel would fault the GPU)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor on {device}, got {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _aux(name, t, dtype, numel, device, *, optional=False, at_least=False):
    """Check a buffer the C ABI takes as a bare pointer: a contiguous torch
    tensor on `device` with the given dtype and element count (or at least
    that many elements), checked before anything is enqueued."""
    import torch
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    _on_device(name, t, device)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if (t.numel() < numel) if at_least else (t.numel() != numel):
        raise ValueError(f"{name} has {t.numel()} elements, expected {'at least ' if at_least else ''}{numel}")


def _check_fwd_buffers(q, k, v, out, cu_seqlens, sinks, lse, topk_idx, block_sel, sink_mode):
    import torch
    dev = q.device
    for name, t in (("k", k), ("v", v), ("out", out)):
        _on_device(name, t, dev)
    for name, t in (("topk_idx", topk_idx), ("block_sel", block_sel)):
        if t is not None and not isinstance(t, AttnTensor):
            _on_device(name, t, dev)
    T, Hq = q.shape[0], q.shape[1]
    if cu_seqlens is not None:
        _aux("cu_seqlens", cu_seqlens, torch.int32, max(cu_seqlens.numel(), 1), dev)
    _aux("sinks", sinks, torch.float32, Hq, dev, optional=(sink_mode == 0))
    _aux("lse", lse, torch.float32, Hq * T, dev)
    _need_gpu(q)


def _need_gpu(t):
    """Non-empty calls launch kernels, which need device memory (an empty call
    enqueues nothing and is accepted anywhere)."""
    if t.numel() > 0 and t.device.type != "cuda":
        raise ValueError(f"the kernels need device memory; got tensors on {t.device}")


def _as_desc(x):
    if x is None or isinstance(x, AttnTensor):
        return x
    return desc(x)


def _mask(mask_kind, window, block_size, topk_idx, block_sel):
    m = AttnMaskArg()
    m.window = int(window or 0)
    m.block_size = int(block_size or 0)
    ti, bs = _as_desc(topk_idx), _as_desc(block_sel)
    m.topk_idx = ctypes.pointer(ti) if ti is not None else None
    m.block_sel = ctypes.pointer(bs) if bs is not None else None
    return m, (ti, bs)


def _codes(mask_kind, sink_mode):
    mk = MASK_KINDS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    sm = SINK_MODES[sink_mode] if isinstance(sink_mode, str) else int(sink_mode)
    return mk, sm


def attn_sink_check(q, k, v, cu_seqlens, num_seqs, mask_kind, mask: dict, sinks, sink_mode,
                    scale, out, lse) -> int:
    """Host-side validation only (no device access); returns the C status."""
    mk, sm = _codes(mask_kind, sink_mode)
    m, keep = _mask(mk, mask.get("window"), mask.get("block_size"), mask.get("topk_idx"),
                    mask.get("block_sel"))
    dq, dk, dv, do = (_as_desc(x) for x in (q, k, v, out))
    return int(_lib.attn_sink_check(_ref(dq), _ref(dk), _ref(dv), _ptr(cu_seqlens), int(num_seqs), mk,
                                    ctypes.byref(m), _ptr(sinks), sm, float(scale), _ref(do), _ptr(lse)))


def attn_sink_fwd(q, k, v, cu_seqlens, mask_kind, mask: dict, sinks, sink_mode, scale, out, lse,
                  stream=None) -> None:
    """Enqueue the forward on `stream` (default: torch's current stream on q's device).

    q, k, v, out: torch tensors on the GPU; cu_seqlens: int32 device tensor or
    None; mask: {"window": W} | {"topk_idx": int32 [T, topk]} |
    {"block_sel": uint8/bool [1, Hidx, T, NB], "block_size": bs}; sinks: f32
    device tensor [Hq] or None; lse: f32 device tensor [Hq, T].
    Raises AttnSinkError on a non-zero status."""
    import torch
    mk, sm = _codes(mask_kind, sink_mode)
    _check_fwd_buffers(q, k, v, out, cu_seqlens, sinks, lse, mask.get("topk_idx"), mask.get("block_sel"), sm)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    m, keep = _mask(mk, mask.get("window"), mask.get("block_size"), mask.get("topk_idx"),
                    mask.get("block_sel"))
    num_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    dq, dk, dv, do = desc(q), desc(k), desc(v), desc(out)
    rc = _lib.attn_sink_fwd(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _ptr(cu_seqlens),
                            num_seqs, mk, ctypes.byref(m), _ptr(sinks), sm, float(scale),
                            ctypes.byref(do), _ptr(lse), ctypes.c_void_p(stream))
    if rc != 0:
        raise AttnSinkError(rc)


def prepared_fwd(q, k, v, *, mask_kind: str, scale: float, out, lse, cu_seqlens=None, window=None,
                 topk_idx=None, block_sel=None, block_size=None, sinks=None, sink_mode: str = "none",
                 stream=None):
    """Marshal the arguments once and return a zero-argument callable that
    re-issues the same attn_sink_fwd call (for timing loops and graph capture,
    where per-call Python marshalling would dominate a microsecond kernel)."""
    import torch
    mk, sm = _codes(mask_kind, sink_mode)
    _check_fwd_buffers(q, k, v, out, cu_seqlens, sinks, lse, topk_idx, block_sel, sm)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    m, keep = _mask(mk, window, block_size, topk_idx, block_sel)
    num_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    dq, dk, dv, do = desc(q), desc(k), desc(v), desc(out)
    args = (ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _ptr(cu_seqlens), num_seqs, mk,
            ctypes.byref(m), _ptr(sinks), sm, float(scale), ctypes.byref(do), _ptr(lse),
            ctypes.c_void_p(stream))
    hold = (dq, dk, dv, do, m, keep, q, k, v, out, lse, cu_seqlens, sinks, topk_idx, block_sel)
    fn = _lib.attn_sink_fwd

    def call():
        rc = fn(*args)
        if rc != 0:
            raise AttnSinkError(rc)
    call._hold = hold
    return call


def fwd(q, k, v, *, mask_kind: str, scale: float, cu_seqlens=None, window=None, topk_idx=None,
        block_sel=None, block_size=None, sinks=None, sink_mode: str = "none", out=None, lse=None,
        stream=None):
    """Keyword form of :func:`attn_sink_fwd`; allocates out [T, Hq, Dv] and
    lse [Hq, T] (float32) with torch when not given.  Returns (out, lse)."""
    import torch
    T, Hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((T, Hq, v.shape[2]), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    mask = {"window": window, "topk_idx": topk_idx, "block_sel": block_sel, "block_size": block_size}
    attn_sink_fwd(q, k, v, cu_seqlens, mask_kind, mask, sinks, sink_mode, scale, out, lse, stream)
    return out, lse


def _stream(stream, dev):
    import torch
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def attn_sink_key0_correct_check(q, k, v, cu_seqlens, num_seqs, window, sinks, scale, out, lse) -> int:
    """Host-side validation of the unfused key-0 correction only; returns the C status."""
    dq, dk, dv, do = (_as_desc(x) for x in (q, k, v, out))
    return int(_lib.attn_sink_key0_correct_check(_ref(dq), _ref(dk), _ref(dv), _ptr(cu_seqlens), int(num_seqs),
                                                 int(window), _ptr(sinks), float(scale), _ref(do), _ptr(lse)))


def attn_sink_key0_correct(q, k, v, cu_seqlens, window, sinks, scale, out, lse, stream=None) -> None:
    """Rewrite, in place, the out / lse of a no-sink window attention with the
    closed-form key-0 sink (only the first window + 1 rows of each sequence).
    Raises AttnSinkError on a non-zero status."""
    import torch
    _check_fwd_buffers(q, k, v, out, cu_seqlens, sinks, lse, None, None, 1)
    num_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    dq, dk, dv, do = desc(q), desc(k), desc(v), desc(out)
    rc = _lib.attn_sink_key0_correct(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _ptr(cu_seqlens),
                                     num_seqs, int(window), _ptr(sinks), float(scale), ctypes.byref(do),
                                     _ptr(lse), ctypes.c_void_p(_stream(stream, q.device)))
    if rc != 0:
        raise AttnSinkError(rc)


def _merge_args(parts, sinks, sink_mode, out, lse):
    n = len(parts)
    outs = (AttnTensor * max(n, 1))()
    lses = (ctypes.c_void_p * max(n, 1))()
    for i, (o, l) in enumerate(parts):
        outs[i] = _as_desc(o)
        lses[i] = _ptr(l)
    sm = SINK_MODES[sink_mode] if isinstance(sink_mode, str) else int(sink_mode)
    do = _as_desc(out)
    return (outs, lses, n, _ptr(sinks), sm, _ref(do), _ptr(lse)), (outs, lses, do)


def attn_sink_merge_check(parts, sinks, sink_mode, out, lse) -> int:
    """Host-side validation of the merge only; parts = [(out_p, lse_p), ...]."""
    args, keep = _merge_args(parts, sinks, sink_mode, out, lse)
    return int(_lib.attn_sink_merge_check(*args))


def attn_sink_merge(parts, sinks, sink_mode, out, lse, stream=None) -> None:
    """Merge partial results over disjoint key sets, parts = [(out_p, lse_p), ...]
    (each from a no-sink attn_sink_fwd), into out / lse, folding in a
    null_logit sink after the merge.  Raises AttnSinkError on a non-zero status."""
    import torch
    dev = out.device
    T, Hq = out.shape[0], out.shape[1]
    sm = SINK_MODES[sink_mode] if isinstance(sink_mode, str) else int(sink_mode)
    for i, (po, pl) in enumerate(parts):
        _on_device(f"parts[{i}].out", po, dev)
        _aux(f"parts[{i}].lse", pl, torch.float32, Hq * T, dev)
    _aux("sinks", sinks, torch.float32, Hq, dev, optional=(sm != SINK_MODES["null_logit"]))
    _aux("lse", lse, torch.float32, Hq * T, dev)
    _need_gpu(out)
    args, keep = _merge_args(parts, sinks, sink_mode, out, lse)
    rc = _lib.attn_sink_merge(*args, ctypes.c_void_p(_stream(stream, out.device)))
    if rc != 0:
        raise AttnSinkError(rc)


def _check_rc(rc):
    if rc != 0:
        raise AttnSinkError(rc)


def attn_sink_cp_slots_check(cp_size, t_local, rank, slots) -> int:
    return int(_lib.attn_sink_cp_slots_check(int(cp_size), int(t_local), int(rank), _ptr(slots)))


def attn_sink_cp_slots(cp_size, t_local, rank, slots, stream=None) -> None:
    """Global slot of every local slot under load-balanced causal CP (rank -1:
    all ranks, rank-major) into the int64 device tensor `slots`."""
    import torch
    n = int(cp_size) * int(t_local) if int(rank) < 0 else int(t_local)
    if slots is not None:
        _aux("slots", slots, torch.int64, n, slots.device, at_least=True)
    _check_rc(_lib.attn_sink_cp_slots(int(cp_size), int(t_local), int(rank), _ptr(slots),
                                      ctypes.c_void_p(_stream(stream, slots.device))))


def attn_sink_cp_permute_rows_check(src, index, n, scatter, dst) -> int:
    ds, dd = _as_desc(src), _as_desc(dst)
    return int(_lib.attn_sink_cp_permute_rows_check(_ref(ds), _ptr(index), int(n), int(scatter), _ref(dd)))


def attn_sink_cp_permute_rows(src, index, scatter, dst, stream=None) -> None:
    """scatter: dst[index[i]] = src[i] (order_by_positions); gather:
    dst[i] = src[index[i]] (restore_by_positions).  index: int64 device tensor."""
    import torch
    _on_device("dst", dst, src.device)
    _aux("index", index, torch.int64, index.numel() if isinstance(index, torch.Tensor) else 0, src.device)
    ds, dd = desc(src), desc(dst)
    _check_rc(_lib.attn_sink_cp_permute_rows(ctypes.byref(ds), _ptr(index), int(index.numel()), int(bool(scatter)),
                                             ctypes.byref(dd), ctypes.c_void_p(_stream(stream, src.device))))


def attn_sink_cp_documents_check(positions, T, doc_ids, cu_seqlens, max_docs, num_docs) -> int:
    return int(_lib.attn_sink_cp_documents_check(_ptr(positions), int(T), _ptr(doc_ids), _ptr(cu_seqlens),
                                                 int(max_docs), _ptr(num_docs)))


def attn_sink_cp_documents(positions, doc_ids=None, cu_seqlens=None, num_docs=None, stream=None) -> None:
    """Document ids (cumsum(positions == 0) - 1) and segment boundaries of
    global-ordered int64 position ids; cu_seqlens holds max_docs + 1 entries."""
    import torch
    dev = positions.device
    _aux("positions", positions, torch.int64, positions.numel(), dev)
    _aux("doc_ids", doc_ids, torch.int32, positions.numel(), dev, optional=True, at_least=True)
    _aux("num_docs", num_docs, torch.int32, 1, dev, optional=True)
    if cu_seqlens is not None:
        _aux("cu_seqlens", cu_seqlens, torch.int32, max(cu_seqlens.numel(), 1), dev)
    max_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    _check_rc(_lib.attn_sink_cp_documents(_ptr(positions), int(positions.numel()), _ptr(doc_ids),
                                          _ptr(cu_seqlens), int(max_docs), _ptr(num_docs),
                                          ctypes.c_void_p(_stream(stream, positions.device))))


def attn_sink_mla_decode_fp8_workspace(T, Hq, topk) -> int:
    """Workspace bytes the fp8 decode needs (host-only)."""
    n = ctypes.c_int64(0)
    _check_rc(_lib.attn_sink_mla_decode_fp8_workspace(int(T), int(Hq), int(topk), ctypes.byref(n)))
    return int(n.value)


def attn_sink_mla_decode_fp8_check(q, kv, kv_scale, topk_idx, sinks, sink_mode, scale, out, lse, workspace,
                                   workspace_bytes) -> int:
    sm = SINK_MODES[sink_mode] if isinstance(sink_mode, str) else int(sink_mode)
    dq, dk, di, do = (_as_desc(x) for x in (q, kv, topk_idx, out))
    return int(_lib.attn_sink_mla_decode_fp8_check(_ref(dq), _ref(dk), _ptr(kv_scale), _ref(di), _ptr(sinks), sm,
                                                   float(scale), _ref(do), _ptr(lse), _ptr(workspace),
                                                   int(workspace_bytes)))


def attn_sink_mla_decode_fp8(q, kv, kv_scale, topk_idx, sinks, sink_mode, scale, out, lse, workspace,
                             stream=None) -> None:
    """Sparse-MLA decode over an fp8 e4m3 latent cache kv [Tk, 1, 576] with
    per-row fp32 scales; workspace: a device tensor of at least
    attn_sink_mla_decode_fp8_workspace(T, Hq, topk) bytes."""
    sm = SINK_MODES[sink_mode] if isinstance(sink_mode, str) else int(sink_mode)
    import torch
    dev = q.device
    T, Hq = q.shape[0], q.shape[1]
    for name, t in (("kv", kv), ("topk_idx", topk_idx), ("out", out)):
        _on_device(name, t, dev)
    _aux("kv_scale", kv_scale, torch.float32, kv.shape[0], dev)
    _aux("sinks", sinks, torch.float32, Hq, dev, optional=(sm != SINK_MODES["null_logit"]))
    _aux("lse", lse, torch.float32, Hq * T, dev)
    _on_device("workspace", workspace, dev)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _need_gpu(q)
    dq, dk, di, do = desc(q), desc(kv), desc(topk_idx), desc(out)
    nbytes = workspace.numel() * workspace.element_size()
    _check_rc(_lib.attn_sink_mla_decode_fp8(ctypes.byref(dq), ctypes.byref(dk), _ptr(kv_scale), ctypes.byref(di),
                                            _ptr(sinks), sm, float(scale), ctypes.byref(do), _ptr(lse),
                                            _ptr(workspace), int(nbytes), ctypes.c_void_p(_stream(stream, q.device))))


def attn_sink_mla_decode_fp8_noalloc(q, kv, kv_scale, topk_idx, sinks, sink_mode, scale, out, lse,
                                     stream=None) -> None:
    """The fp8 sparse-MLA decode without a workspace: its partial results go to
    the library's static per-GPU scratch (DECODE_SCRATCH_BYTES; larger calls
    raise ATTN_ERR_RANGE).  Calls that overlap on one GPU race."""
    import torch
    sm = SINK_MODES[sink_mode] if isinstance(sink_mode, str) else int(sink_mode)
    dev = q.device
    T, Hq = q.shape[0], q.shape[1]
    for name, t in (("kv", kv), ("topk_idx", topk_idx), ("out", out)):
        _on_device(name, t, dev)
    _aux("kv_scale", kv_scale, torch.float32, kv.shape[0], dev)
    _aux("sinks", sinks, torch.float32, Hq, dev, optional=(sm != SINK_MODES["null_logit"]))
    _aux("lse", lse, torch.float32, Hq * T, dev)
    _need_gpu(q)
    dq, dk, di, do = desc(q), desc(kv), desc(topk_idx), desc(out)
    _check_rc(_lib.attn_sink_mla_decode_fp8_noalloc(ctypes.byref(dq), ctypes.byref(dk), _ptr(kv_scale),
                                                    ctypes.byref(di), _ptr(sinks), sm, float(scale),
                                                    ctypes.byref(do), _ptr(lse),
                                                    ctypes.c_void_p(_stream(stream, q.device))))


def decode_case_on_device(case: dict, device="cuda:0") -> dict:
    """Device tensors of a generated fp8 decode case (fp8 bytes viewed as
    torch.float8_e4m3fn) plus out / lse / workspace buffers."""
    import torch
    T, Hq = case["q"].shape[:2]
    topk = case["topk_idx"].shape[1]
    d = dict(q=torch.from_numpy(case["q"]).to(device=device, dtype=torch.bfloat16),
             kv=torch.from_numpy(case["kv_fp8"]).to(device).view(torch.float8_e4m3fn),
             kv_scale=torch.from_numpy(case["kv_scale"]).to(device),
             topk_idx=torch.from_numpy(case["topk_idx"]).to(device),
             sinks=None if case["sinks"] is None else torch.from_numpy(case["sinks"]).to(device),
             sink_mode=case["sink_mode"], scale=case["scale"])
    d["out"] = torch.empty((T, Hq, 512), dtype=torch.bfloat16, device=device)
    d["lse"] = torch.empty((Hq, T), dtype=torch.float32, device=device)
    d["workspace"] = torch.empty(attn_sink_mla_decode_fp8_workspace(T, Hq, topk), dtype=torch.uint8, device=device)
    return d


def case_on_device(case: dict, device="cuda:0") -> dict:
    """Copy a generated input case (NumPy arrays) to device tensors: bf16 or f32
    values (bit-exact), int32 / uint8 metadata.  The shared-latent layout keeps
    v as a view of k."""
    import torch
    dt = torch.bfloat16 if case["dtype"] == "bf16" else torch.float32

    def t(a, dtype):
        return None if a is None else torch.from_numpy(a).to(device=device, dtype=dtype)

    q = t(case["q"], dt)
    k = t(case["k"], dt)
    if case.get("v_aliases_k"):
        v = k[:, :, :case["v"].shape[2]]
    else:
        v = t(case["v"].copy(), dt)
    return dict(q=q, k=k, v=v, mask_kind=case["mask_kind"], scale=case["scale"],
                cu_seqlens=t(case["cu_seqlens"], torch.int32), window=case["window"],
                topk_idx=t(case["topk_idx"], torch.int32), block_sel=t(case["block_sel"], torch.uint8),
                block_size=case["block_size"], sinks=t(case["sinks"], torch.float32),
                sink_mode=case["sink_mode"])


def run_case(case: dict, device="cuda:0", **over):
    """Run a generated case on the GPU; returns (out, lse) device tensors."""
    d = case_on_device(case, device)
    d.update(over)
    return fwd(**d)
