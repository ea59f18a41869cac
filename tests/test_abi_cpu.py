"""The C-ABI library on a host without a GPU: it loads, exports exactly what
include/attn_sink.h declares, and its host-side validation accepts every
supported call and rejects each class of bad argument with the documented
status (no device access: attn_sink_check never touches memory)."""
from __future__ import annotations

import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_sink.h")


@pytest.fixture(scope="module")
def sam():
    lib = os.path.join(ROOT, "sink_aware_masked_amd", "libattn_sink.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.build_library()
    import sink_aware_masked_amd
    return sink_aware_masked_amd


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_sink_\w+)\s*\(", src, flags=re.M)))


def test_exports_match_header(sam):
    decl = declared_functions()
    assert decl == sorted(sam.EXPORTS)
    for name in decl:
        assert hasattr(sam._lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", sam.LIB_PATH], capture_output=True, text=True, check=True)
    exported = sorted(ln.split()[-1] for ln in nm.stdout.splitlines() if " T " in ln and ln.split()[-1].startswith("attn_"))
    assert exported == decl


def test_version_and_strerror(sam):
    m = re.search(r"#define ATTN_SINK_ABI_VERSION (\d+)", open(HEADER).read())
    assert sam.attn_sink_abi_version() == int(m.group(1))
    for code in list(sam.STATUS) + [-100, 7]:
        s = sam.attn_sink_strerror(code)
        assert isinstance(s, str) and s
    assert sam.attn_sink_strerror(0) == "ok"


# ------------------------------------------------------------ validation
def window_args(T=256, Hq=16, Hkv=4, D=80, dtype=torch.bfloat16, W=64, sink="key0_bias"):
    q = torch.empty(T, Hq, D, dtype=dtype)
    k = torch.empty(T, Hkv, D, dtype=dtype)
    v = torch.empty(T, Hkv, D, dtype=dtype)
    out = torch.empty(T, Hq, D, dtype=dtype)
    lse = torch.empty(Hq, T, dtype=torch.float32)
    cu = torch.tensor([0, 100, T], dtype=torch.int32)
    sinks = torch.zeros(Hq, dtype=torch.float32)
    return dict(q=q, k=k, v=v, cu_seqlens=cu, num_seqs=2, mask_kind="window", mask={"window": W},
                sinks=sinks, sink_mode=sink, scale=0.1, out=out, lse=lse)


def mla_args(T=8, Hq=64, Tk=100, topk=16):
    q = torch.empty(T, Hq, 576, dtype=torch.bfloat16)
    kv = torch.empty(Tk, 1, 576, dtype=torch.bfloat16)
    return dict(q=q, k=kv, v=kv[:, :, :512], cu_seqlens=None, num_seqs=0, mask_kind="topk",
                mask={"topk_idx": torch.empty(T, topk, dtype=torch.int32)},
                sinks=torch.zeros(Hq), sink_mode="null_logit", scale=0.04,
                out=torch.empty(T, Hq, 512, dtype=torch.bfloat16), lse=torch.empty(Hq, T))


def bsel_args(T=300, Hq=32, Hkv=8, D=128, bs=64):
    NB = (T + bs - 1) // bs
    return dict(q=torch.empty(T, Hq, D, dtype=torch.bfloat16), k=torch.empty(T, Hkv, D, dtype=torch.bfloat16),
                v=torch.empty(T, Hkv, D, dtype=torch.bfloat16), cu_seqlens=torch.tensor([0, 120, T], dtype=torch.int32),
                num_seqs=2, mask_kind="blocksel",
                mask={"block_sel": torch.empty(1, Hkv, T, NB, dtype=torch.uint8), "block_size": bs},
                sinks=None, sink_mode="none", scale=0.088, out=torch.empty(T, Hq, D, dtype=torch.bfloat16),
                lse=torch.empty(Hq, T))


def check(sam, a):
    return sam.attn_sink_check(a["q"], a["k"], a["v"], a["cu_seqlens"], a["num_seqs"], a["mask_kind"], a["mask"],
                               a["sinks"], a["sink_mode"], a["scale"], a["out"], a["lse"])


@pytest.mark.parametrize("D", [64, 80, 96, 128])
@pytest.mark.parametrize("sink", ["none", "key0_bias", "null_logit"])
def test_supported_window(sam, D, sink):
    assert check(sam, window_args(D=D, sink=sink)) == 0


def test_supported_others(sam):
    assert check(sam, mla_args()) == 0
    assert check(sam, bsel_args()) == 0
    a = bsel_args()
    a.update(sink_mode="null_logit", sinks=torch.zeros(32))
    assert check(sam, a) == 0
    for kind, args in (("window", window_args(D=48, dtype=torch.float32)),):
        assert check(sam, args) == 0
    f = mla_args()
    for key in ("q", "k", "out"):
        f[key] = f[key].float()
    f["v"] = f["k"][:, :, :512]
    assert check(sam, f) == 0
    e = window_args(T=0)
    e["cu_seqlens"] = torch.tensor([0], dtype=torch.int32)
    e["num_seqs"] = 0
    assert check(sam, e) == 0


def _bad(sam, base, expect, **over):
    a = dict(base)
    a.update(over)
    rc = check(sam, a)
    assert sam.STATUS[rc] == expect, (sam.STATUS.get(rc), expect, over.keys())


def test_rejections(sam):
    E = sam
    w = window_args()
    _bad(E, w, "ATTN_ERR_NULL", q=None)
    _bad(E, w, "ATTN_ERR_NULL", lse=None)
    _bad(E, w, "ATTN_ERR_NULL", sinks=None)
    _bad(E, w, "ATTN_ERR_NULL", cu_seqlens=None)
    _bad(E, w, "ATTN_ERR_ENUM", mask_kind=3)
    _bad(E, w, "ATTN_ERR_ENUM", sink_mode=-1)
    _bad(E, w, "ATTN_ERR_SHAPE", k=torch.empty(255, 4, 80, dtype=torch.bfloat16))
    _bad(E, w, "ATTN_ERR_SHAPE", out=torch.empty(256, 16, 64, dtype=torch.bfloat16))
    _bad(E, w, "ATTN_ERR_SHAPE", q=torch.empty(256, 16, 80, 1, dtype=torch.bfloat16))
    _bad(E, w, "ATTN_ERR_HEADS", k=torch.empty(256, 3, 80, dtype=torch.bfloat16),
         v=torch.empty(256, 3, 80, dtype=torch.bfloat16))
    _bad(E, w, "ATTN_ERR_DTYPE", out=torch.empty(256, 16, 80, dtype=torch.float32))
    _bad(E, w, "ATTN_ERR_DTYPE", q=torch.empty(256, 16, 80, dtype=torch.int32))
    _bad(E, w, "ATTN_ERR_STRIDE", q=torch.empty(256, 80, 16, dtype=torch.bfloat16).transpose(1, 2))
    _bad(E, w, "ATTN_ERR_STRIDE", q=torch.empty(256, 16, 84, dtype=torch.bfloat16)[:, :, :80])
    _bad(E, w, "ATTN_ERR_RANGE", mask={"window": -1})
    _bad(E, w, "ATTN_ERR_RANGE", scale=float("nan"))
    _bad(E, w, "ATTN_ERR_RANGE", scale=3.0e38)   # finite, but scale * log2(e) overflows
    _bad(E, w, "ATTN_ERR_RANGE", scale=-3.0e38)
    _bad(E, w, "ATTN_ERR_UNSUPPORTED", **{k_: torch.empty(256, h, 48, dtype=torch.bfloat16)
                                         for k_, h in (("q", 16), ("k", 4), ("v", 4), ("out", 16))})
    m = mla_args()
    _bad(E, m, "ATTN_ERR_UNSUPPORTED", sink_mode="key0_bias")
    _bad(E, m, "ATTN_ERR_UNSUPPORTED", v=torch.empty(100, 1, 512, dtype=torch.bfloat16))
    _bad(E, m, "ATTN_ERR_DTYPE", mask={"topk_idx": torch.empty(8, 16, dtype=torch.float32)})
    _bad(E, m, "ATTN_ERR_SHAPE", mask={"topk_idx": torch.empty(9, 16, dtype=torch.int32)})
    _bad(E, m, "ATTN_ERR_NULL", mask={})
    b = bsel_args()
    _bad(E, b, "ATTN_ERR_SHAPE", mask={"block_sel": torch.empty(1, 8, 300, 4, dtype=torch.uint8), "block_size": 64})
    _bad(E, b, "ATTN_ERR_HEADS", mask={"block_sel": torch.empty(1, 3, 300, 5, dtype=torch.uint8), "block_size": 64})
    _bad(E, b, "ATTN_ERR_RANGE", mask={"block_sel": torch.empty(1, 8, 300, 5, dtype=torch.uint8), "block_size": 0})
    _bad(E, b, "ATTN_ERR_DTYPE", mask={"block_sel": torch.empty(1, 8, 300, 5, dtype=torch.int32), "block_size": 64})
    _bad(E, b, "ATTN_ERR_UNSUPPORTED", mask={"block_sel": torch.empty(1, 8, 300, 10, dtype=torch.uint8), "block_size": 32})
    _bad(E, b, "ATTN_ERR_SHAPE", k=torch.empty(301, 8, 128, dtype=torch.bfloat16),
         v=torch.empty(301, 8, 128, dtype=torch.bfloat16))


def test_binding_fails_loudly_without_library(tmp_path):
    """Importing the binding from a copy of the package without the built
    library raises instead of falling back to anything."""
    import shutil
    import sys
    pkg = tmp_path / "sink_aware_masked_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "sink_aware_masked_amd", "__init__.py"), pkg / "__init__.py")
    code = "import sink_aware_masked_amd"
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "not built" in r.stderr


# --------------------------------------------- unfused key-0 correction / merge
def key0_args(T=256, Hq=16, Hkv=4, D=80, dtype=torch.bfloat16, W=64):
    a = window_args(T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, W=W)
    return dict(q=a["q"], k=a["k"], v=a["v"], cu_seqlens=a["cu_seqlens"], num_seqs=2, window=W,
                sinks=torch.zeros(Hq), scale=0.1, out=a["out"], lse=a["lse"])


def key0_check(sam, a):
    return sam.attn_sink_key0_correct_check(a["q"], a["k"], a["v"], a["cu_seqlens"], a["num_seqs"], a["window"],
                                            a["sinks"], a["scale"], a["out"], a["lse"])


def test_key0_correct_validation(sam):
    for D in (64, 80, 128):
        assert key0_check(sam, key0_args(D=D)) == 0
    assert key0_check(sam, key0_args(D=48, dtype=torch.float32)) == 0
    a = key0_args()
    for over, expect in (({"sinks": None}, "ATTN_ERR_NULL"), ({"cu_seqlens": None}, "ATTN_ERR_NULL"),
                         ({"lse": None}, "ATTN_ERR_NULL"), ({"window": -1}, "ATTN_ERR_RANGE"),
                         ({"scale": float("inf")}, "ATTN_ERR_RANGE"), ({"scale": 3.0e38}, "ATTN_ERR_RANGE"),
                         ({"out": torch.empty(256, 16, 80, dtype=torch.float32)}, "ATTN_ERR_DTYPE"),
                         ({"k": torch.empty(255, 4, 80, dtype=torch.bfloat16)}, "ATTN_ERR_SHAPE"),
                         ({"k": torch.empty(256, 3, 80, dtype=torch.bfloat16),
                           "v": torch.empty(256, 3, 80, dtype=torch.bfloat16)}, "ATTN_ERR_HEADS"),
                         ({"q": torch.empty(256, 16, 84, dtype=torch.bfloat16)[:, :, :80]}, "ATTN_ERR_STRIDE")):
        b = dict(a)
        b.update(over)
        assert sam.STATUS[key0_check(sam, b)] == expect, (over.keys(), expect)
    # an f32 head dim of 6 is not a whole number of 16-byte chunks
    f = key0_args(D=4, dtype=torch.float32)
    for k_, h in (("q", 16), ("k", 4), ("v", 4), ("out", 16)):
        f[k_] = torch.empty(256, h, 8, dtype=torch.float32)[:, :, :6]
    assert sam.STATUS[key0_check(sam, f)] in ("ATTN_ERR_UNSUPPORTED", "ATTN_ERR_STRIDE")


def merge_args(P=2, T=64, Hq=8, Dv=128, dtype=torch.bfloat16):
    parts = [(torch.empty(T, Hq, Dv, dtype=dtype), torch.empty(Hq, T)) for _ in range(P)]
    return dict(parts=parts, sinks=torch.zeros(Hq), sink_mode="null_logit",
                out=torch.empty(T, Hq, Dv, dtype=dtype), lse=torch.empty(Hq, T))


def merge_check(sam, a):
    return sam.attn_sink_merge_check(a["parts"], a["sinks"], a["sink_mode"], a["out"], a["lse"])


def test_merge_validation(sam):
    for P in (1, 2, sam.MERGE_MAX_PARTS):
        assert merge_check(sam, merge_args(P=P)) == 0
    assert merge_check(sam, merge_args(dtype=torch.float32, Dv=4)) == 0
    a = merge_args()
    a["sink_mode"], a["sinks"] = "none", None
    assert merge_check(sam, a) == 0

    def bad(expect, **over):
        b = merge_args()
        b.update(over)
        assert sam.STATUS[merge_check(sam, b)] == expect, (over.keys(), expect)

    bad("ATTN_ERR_RANGE", parts=[])
    bad("ATTN_ERR_RANGE", parts=merge_args(P=sam.MERGE_MAX_PARTS + 1)["parts"])
    bad("ATTN_ERR_UNSUPPORTED", sink_mode="key0_bias")
    bad("ATTN_ERR_ENUM", sink_mode=3)
    bad("ATTN_ERR_NULL", sinks=None)
    bad("ATTN_ERR_NULL", lse=None)
    bad("ATTN_ERR_DTYPE", out=torch.empty(64, 8, 128, dtype=torch.float32))
    bad("ATTN_ERR_SHAPE", parts=[(torch.empty(64, 8, 64, dtype=torch.bfloat16), torch.empty(8, 64))] * 2)
    bad("ATTN_ERR_NULL", parts=[(torch.empty(64, 8, 128, dtype=torch.bfloat16), None)] * 2)
    b = merge_args()
    b["out"] = b["parts"][1][0]  # writing into a partial is refused
    assert sam.STATUS[merge_check(sam, b)] == "ATTN_ERR_RANGE"
    b = merge_args()
    b["lse"] = b["parts"][0][1]
    assert sam.STATUS[merge_check(sam, b)] == "ATTN_ERR_RANGE"


# ------------------------------------------------ context-parallel reorder
def test_cp_validation(sam):
    slots = torch.empty(64, dtype=torch.int64)
    assert sam.attn_sink_cp_slots_check(4, 16, -1, slots) == 0
    assert sam.attn_sink_cp_slots_check(4, 16, 3, slots) == 0
    assert sam.attn_sink_cp_slots_check(1, 0, 0, None) == 0
    for args, expect in (((0, 16, -1, slots), "ATTN_ERR_RANGE"), ((4, 15, -1, slots), "ATTN_ERR_RANGE"),
                         ((4, 16, 4, slots), "ATTN_ERR_RANGE"), ((4, 16, -2, slots), "ATTN_ERR_RANGE"),
                         ((4, 16, -1, None), "ATTN_ERR_NULL")):
        assert sam.STATUS[sam.attn_sink_cp_slots_check(*args)] == expect, (args[:3], expect)

    src = torch.empty(32, 8, 128, dtype=torch.bfloat16)
    dst = torch.empty(32, 8, 128, dtype=torch.bfloat16)
    idx = torch.empty(32, dtype=torch.int64)
    chk = sam.attn_sink_cp_permute_rows_check
    assert chk(src, idx, 32, 1, dst) == 0 and chk(src, idx, 32, 0, dst) == 0
    assert chk(torch.empty(32, dtype=torch.int64), idx, 32, 1, torch.empty(32, dtype=torch.int64)) == 0
    assert chk(torch.empty(10, 3, dtype=torch.int32), idx[:10], 10, 0, torch.empty(10, 3, dtype=torch.int32)) == 0
    assert chk(src, idx[:20], 20, 0, torch.empty(20, 8, 128, dtype=torch.bfloat16)) == 0  # gather a subset
    for over, expect in (({"scatter": 2}, "ATTN_ERR_ENUM"), ({"index": None}, "ATTN_ERR_NULL"),
                         ({"dst": torch.empty(32, 8, 128, dtype=torch.float32)}, "ATTN_ERR_DTYPE"),
                         ({"dst": torch.empty(32, 8, 64, dtype=torch.bfloat16)}, "ATTN_ERR_SHAPE"),
                         ({"n": 31}, "ATTN_ERR_SHAPE"), ({"dst": src}, "ATTN_ERR_RANGE"),
                         ({"src": torch.empty(32, 128, 8, dtype=torch.bfloat16).transpose(1, 2)}, "ATTN_ERR_STRIDE"),
                         ({"src": torch.empty(32, 3, dtype=torch.uint8), "dst": torch.empty(32, 3, dtype=torch.uint8)},
                          "ATTN_ERR_UNSUPPORTED")):
        a = dict(src=src, index=idx, n=32, scatter=1, dst=dst)
        a.update(over)
        assert sam.STATUS[chk(a["src"], a["index"], a["n"], a["scatter"], a["dst"])] == expect, (over.keys(), expect)

    pos = torch.empty(100, dtype=torch.int64)
    ids, cu, nd = torch.empty(100, dtype=torch.int32), torch.empty(9, dtype=torch.int32), torch.empty(1, dtype=torch.int32)
    dchk = sam.attn_sink_cp_documents_check
    assert dchk(pos, 100, ids, cu, 8, nd) == 0 and dchk(pos, 100, None, None, 0, None) == 0
    assert dchk(None, 0, None, cu, 8, nd) == 0
    assert sam.STATUS[dchk(None, 100, ids, cu, 8, nd)] == "ATTN_ERR_NULL"
    assert sam.STATUS[dchk(pos, -1, ids, cu, 8, nd)] == "ATTN_ERR_RANGE"
    assert sam.STATUS[dchk(pos, 100, ids, cu, -1, nd)] == "ATTN_ERR_RANGE"


# ------------------------------------------------------------ fp8 decode
def decode_args(T=8, Hq=64, Tk=100, topk=32):
    return dict(q=torch.empty(T, Hq, 576, dtype=torch.bfloat16),
                kv=torch.empty(Tk, 1, 576, dtype=torch.float8_e4m3fn), kv_scale=torch.empty(Tk),
                topk_idx=torch.empty(T, topk, dtype=torch.int32), sinks=torch.zeros(Hq), sink_mode="null_logit",
                scale=0.04, out=torch.empty(T, Hq, 512, dtype=torch.bfloat16), lse=torch.empty(Hq, T))


def decode_check(sam, a, ws_bytes=None):
    T, Hq, topk = a["q"].shape[0], a["q"].shape[1], a["topk_idx"].shape[1]
    need = sam.attn_sink_mla_decode_fp8_workspace(T, Hq, topk) if Hq % 64 == 0 and Hq > 0 else 16
    ws = torch.empty(max(need, 16), dtype=torch.uint8)
    return sam.attn_sink_mla_decode_fp8_check(a["q"], a["kv"], a["kv_scale"], a["topk_idx"], a["sinks"], a["sink_mode"],
                                              a["scale"], a["out"], a["lse"], ws,
                                              need if ws_bytes is None else ws_bytes)


def test_decode_validation(sam):
    assert sam.attn_sink_mla_decode_fp8_workspace(128, 64, 2048) > 0
    assert decode_check(sam, decode_args()) == 0
    a = decode_args()
    a.update(sink_mode="none", sinks=None)
    assert decode_check(sam, a) == 0
    assert decode_check(sam, decode_args(Hq=128)) == 0
    for over, expect in (({"sink_mode": "key0_bias"}, "ATTN_ERR_UNSUPPORTED"), ({"sinks": None}, "ATTN_ERR_NULL"),
                         ({"kv": torch.empty(100, 1, 576, dtype=torch.bfloat16)}, "ATTN_ERR_DTYPE"),
                         ({"kv": torch.empty(100, 1, 512, dtype=torch.float8_e4m3fn)}, "ATTN_ERR_UNSUPPORTED"),
                         ({"kv_scale": None}, "ATTN_ERR_NULL"),
                         ({"out": torch.empty(8, 64, 576, dtype=torch.bfloat16)}, "ATTN_ERR_UNSUPPORTED"),
                         ({"topk_idx": torch.empty(9, 32, dtype=torch.int32)}, "ATTN_ERR_SHAPE"),
                         ({"scale": float("nan")}, "ATTN_ERR_RANGE"), ({"scale": -3.0e38}, "ATTN_ERR_RANGE")):
        b = decode_args()
        b.update(over)
        assert sam.STATUS[decode_check(sam, b)] == expect, (over.keys(), expect)
    assert sam.STATUS[decode_check(sam, decode_args(), ws_bytes=64)] == "ATTN_ERR_RANGE"
    b = decode_args(Hq=32)
    assert sam.STATUS[decode_check(sam, b)] == "ATTN_ERR_UNSUPPORTED"


def test_empty_inputs_return_without_launching(sam):
    """T == 0 (or n == 0) is a valid call that enqueues nothing: every entry
    point returns ATTN_OK on a host without a GPU, because it never reaches a
    launch."""
    a = merge_args(T=0)
    assert sam.attn_sink_merge_check(a["parts"], a["sinks"], a["sink_mode"], a["out"], a["lse"]) == 0
    sam.attn_sink_merge(a["parts"], a["sinks"], a["sink_mode"], a["out"], a["lse"], stream=0)
    k = key0_args(T=0)
    k["cu_seqlens"] = torch.tensor([0], dtype=torch.int32)
    k["num_seqs"] = 0
    sam.attn_sink_key0_correct(k["q"], k["k"], k["v"], k["cu_seqlens"], k["window"], k["sinks"], k["scale"],
                               k["out"], k["lse"], stream=0)
    empty = torch.empty(0, 8, dtype=torch.float32)
    sam.attn_sink_cp_permute_rows(empty, torch.empty(0, dtype=torch.int64), True, torch.empty(0, 8), stream=0)
    sam.attn_sink_cp_slots(3, 0, -1, torch.empty(0, dtype=torch.int64), stream=0)
    d = decode_args(T=0)
    ws = torch.empty(16, dtype=torch.uint8)
    sam.attn_sink_mla_decode_fp8(d["q"], d["kv"], d["kv_scale"], d["topk_idx"], d["sinks"], d["sink_mode"], d["scale"],
                                 d["out"], d["lse"], ws, stream=0)


def test_row_stride_limit_of_a_64_row_tile(sam):
    """64 rows of q, k, v or out must span less than 2^31 bytes (kernels
    address inside a 64-row tile with 32-bit offsets): a bf16 row stride of
    2^24 elements is refused with ATTN_ERR_RANGE, one 64 elements shorter is
    accepted.  Single-row tensors carry the stride without any storage."""
    base = window_args(T=1, Hq=4, Hkv=4, D=64)
    base.update(cu_seqlens=torch.tensor([0, 1], dtype=torch.int32), num_seqs=1)

    def strided(t, s0):
        return t.as_strided(t.shape, (s0,) + tuple(t.stride()[1:]))

    for key in ("q", "k", "v", "out"):
        ok = dict(base, **{key: strided(base[key], (1 << 24) - 64)})
        assert check(sam, ok) == 0, key
        _bad(sam, base, "ATTN_ERR_RANGE", **{key: strided(base[key], 1 << 24)})


# ---------------------------------------------------------------- binding argument checks
# The binding passes cu_seqlens, sinks, lse, kv_scale and workspace to the C
# ABI as bare pointers; it must refuse a wrong device, dtype or size before any
# call reaches the library (a host pointer or an undersized buffer would reach
# a kernel otherwise).

def _fwd_args(dev="cpu"):
    import torch
    T, Hq, Hkv, D = 8, 4, 2, 64
    q = torch.zeros((T, Hq, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((T, Hkv, D), dtype=torch.bfloat16, device=dev)
    v = torch.zeros((T, Hkv, D), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    cu = torch.tensor([0, 3, 8], dtype=torch.int32, device=dev)
    sinks = torch.zeros(Hq, dtype=torch.float32, device=dev)
    return dict(q=q, k=k, v=v, cu_seqlens=cu, mask_kind="window", window=2, scale=0.125,
                sinks=sinks, sink_mode="key0_bias", out=out, lse=lse)


@pytest.mark.parametrize("bad", ["cu_int64", "lse_bf16", "lse_short", "sinks_short", "sinks_missing",
                                 "sinks_f64", "lse_strided", "cpu_tensors"])
def test_binding_refuses_bad_buffers(sam, bad):
    import torch
    a = _fwd_args()
    if bad == "cu_int64":
        a["cu_seqlens"] = a["cu_seqlens"].to(torch.int64)
        err = TypeError
    elif bad == "lse_bf16":
        a["lse"] = a["lse"].to(torch.bfloat16)
        err = TypeError
    elif bad == "lse_short":
        a["lse"] = a["lse"][:, :4]
        err = ValueError
    elif bad == "sinks_short":
        a["sinks"] = a["sinks"][:2]
        err = ValueError
    elif bad == "sinks_missing":
        a["sinks"] = None
        err = ValueError
    elif bad == "sinks_f64":
        a["sinks"] = a["sinks"].double()
        err = TypeError
    elif bad == "lse_strided":
        a["lse"] = torch.empty((a["lse"].shape[1], a["lse"].shape[0]), dtype=torch.float32).t()
        err = ValueError
    else:  # everything consistent, but in host memory: the kernels need device memory
        err = ValueError
    with pytest.raises(err):
        sam.fwd(**a)
    with pytest.raises(err):
        sam.prepared_fwd(**a)


def test_binding_refuses_mixed_devices(sam):
    import torch
    a = _fwd_args()
    meta = {k: (v.to("meta") if isinstance(v, torch.Tensor) and k in ("q", "k", "v", "out") else v)
            for k, v in a.items()}
    with pytest.raises(ValueError, match="is on"):
        sam.fwd(**meta)


def test_binding_refuses_bad_decode_buffers(sam):
    import torch
    T, Hq, Tk = 2, 64, 16
    q = torch.zeros((T, Hq, 576), dtype=torch.bfloat16)
    kv = torch.zeros((Tk, 1, 576), dtype=torch.uint8).view(torch.float8_e4m3fn)
    idx = torch.zeros((T, 4), dtype=torch.int32)
    out = torch.empty((T, Hq, 512), dtype=torch.bfloat16)
    lse = torch.empty((Hq, T), dtype=torch.float32)
    ws = torch.empty(1 << 20, dtype=torch.uint8)
    with pytest.raises(TypeError):   # kv_scale in fp64
        sam.attn_sink_mla_decode_fp8(q, kv, torch.ones(Tk, dtype=torch.float64), idx, None, "none", 0.1,
                                     out, lse, ws)
    with pytest.raises(ValueError):  # one scale short
        sam.attn_sink_mla_decode_fp8(q, kv, torch.ones(Tk - 1), idx, None, "none", 0.1, out, lse, ws)
    with pytest.raises(ValueError):  # null_logit without sinks
        sam.attn_sink_mla_decode_fp8(q, kv, torch.ones(Tk), idx, None, "null_logit", 0.1, out, lse, ws)


def test_binding_refuses_bad_merge_buffers(sam):
    import torch
    T, Hq, Dv = 4, 2, 16
    parts = [(torch.zeros((T, Hq, Dv)), torch.zeros((Hq, T))) for _ in range(2)]
    out = torch.empty((T, Hq, Dv))
    with pytest.raises(TypeError):   # a partial LSE in bf16
        sam.attn_sink_merge([parts[0], (parts[1][0], parts[1][1].bfloat16())], None, "none", out,
                            torch.empty((Hq, T)))
    with pytest.raises(ValueError):  # output LSE too small
        sam.attn_sink_merge(parts, None, "none", out, torch.empty((Hq, T - 1)))


def _fake(shape, dtype=0, data=1 << 20):
    """Host-side descriptor of a dense array that is never touched."""
    import sink_aware_masked_amd as m
    stride, acc = [], 1
    for n in reversed(shape):
        stride.insert(0, acc)
        acc *= n
    return m.desc(None, data=data, dtype=dtype, shape=tuple(shape), stride=tuple(stride))


def test_grid_limit_boundary(sam):
    """The window launch uses ceil(T / 128) * Hq workgroups of 256 lanes; a call
    whose grid exceeds 2^32 - 1 work items is refused by the check (not at
    launch), and the largest one that fits is accepted."""
    def win(T, Hq=1):
        q, out = _fake((T, Hq, 64)), _fake((T, Hq, 64))
        k, v = _fake((T, 1, 64)), _fake((T, 1, 64))
        return sam.attn_sink_check(q, k, v, 1 << 20, 1, "window", {"window": 4}, None, "none", 0.125, out, 1 << 20)
    fits = 128 * ((1 << 24) - 1)
    assert win(fits) == 0
    assert sam.STATUS[win(fits + 1)] == "ATTN_ERR_RANGE"
    assert sam.STATUS[win(fits // 2 + 1, Hq=2)] == "ATTN_ERR_RANGE"


def test_unbounded_window_accepted(sam):
    """W = INT32_MAX (an unbounded window) is valid on both precisions: the
    library clamps it to T, so no row + W sum leaves the int32 range."""
    for dt in (torch.bfloat16, torch.float32):
        a = window_args(D=64, dtype=dt)
        a["mask"] = {"window": 2 ** 31 - 1}
        assert check(sam, a) == 0
    k0 = window_args(D=64)
    rc = sam.attn_sink_key0_correct_check(k0["q"], k0["k"], k0["v"], k0["cu_seqlens"], 2, 2 ** 31 - 1,
                                          k0["sinks"], 0.1, k0["out"], k0["lse"])
    assert rc == 0
