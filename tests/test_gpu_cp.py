"""GPU parity of the context-parallel reorder primitives against oracle/cp.py
(NeMo AutoModel 'cp_sparse_attn' page): bit-exact slots, row permutations and
document ids / segment starts, and a block-sparse layer run end to end on
K/V reordered from a load-balanced CP layout."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import cp
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def sam():
    return G.sam()


@pytest.mark.parametrize("cp_size,t_local", [(1, 2), (2, 4), (3, 6), (8, 4096), (16, 2048), (5, 0)])
def test_slots_bit_exact(cp_size, t_local):
    for rank in [-1] + list(range(min(cp_size, 4))) + [cp_size - 1]:
        n = cp_size * t_local if rank < 0 else t_local
        out = torch.full((max(n, 1),), -7, dtype=torch.int64, device=DEV)
        sam().attn_sink_cp_slots(cp_size, t_local, rank, out)
        got = out[:n].cpu().numpy()
        want = cp.load_balanced_slots(cp_size, t_local, None if rank < 0 else rank)
        assert np.array_equal(got, want), (cp_size, t_local, rank)


TENSORS = [((4096, 8, 128), torch.bfloat16), ((1000, 3), torch.int32), ((777,), torch.int64),
           ((300, 16, 80), torch.bfloat16), ((64, 2, 6), torch.float32), ((512, 576), torch.bfloat16)]


@pytest.mark.parametrize("shape,dtype", TENSORS)
def test_order_and_restore_bit_exact(shape, dtype):
    """order_by_positions (scatter) and restore_by_positions (gather) on rows,
    against the oracle, for row lengths that take 16-, 8- and 4-byte chunks."""
    g = np.random.default_rng(shape[0])
    T = shape[0] - shape[0] % 2
    x = torch.from_numpy(g.integers(-2 ** 15, 2 ** 15, size=(T,) + shape[1:]).astype(np.int64)).to(dtype)
    cp_size = 2 if T % 4 else 4
    t_local = T // cp_size
    if t_local % 2:
        cp_size, t_local = 1, T
    pos = cp.load_balanced_slots(cp_size, t_local)
    gathered = x[torch.from_numpy(pos)]
    want_glob, _ = cp.order_by_positions(gathered.numpy() if dtype != torch.bfloat16 else gathered.view(torch.int16).numpy(), pos)
    dg, dpos = gathered.to(DEV), torch.from_numpy(pos).to(DEV)
    glob = torch.empty_like(dg)
    sam().attn_sink_cp_permute_rows(dg, dpos, True, glob)
    torch.cuda.synchronize()
    assert torch.equal(glob.cpu(), x)
    got = glob.cpu() if dtype != torch.bfloat16 else glob.cpu().view(torch.int16)
    assert np.array_equal(got.numpy(), want_glob)
    for r in range(cp_size):
        mine = cp.load_balanced_slots(cp_size, t_local, r)
        local = torch.empty((t_local,) + tuple(shape[1:]), dtype=dtype, device=DEV)
        sam().attn_sink_cp_permute_rows(glob, torch.from_numpy(mine).to(DEV), False, local)
        torch.cuda.synchronize()
        assert torch.equal(local.cpu(), gathered[r * t_local:(r + 1) * t_local])


def test_permute_out_of_range_rows():
    """Gather: an index outside the source gives a zero row; scatter: a target
    outside the destination drops the row and leaves the destination alone."""
    src = torch.arange(6 * 8, dtype=torch.float32, device=DEV).reshape(6, 8) + 1
    idx = torch.tensor([2, -1, 6, 0], dtype=torch.int64, device=DEV)
    out = torch.full((4, 8), 5.0, device=DEV)
    sam().attn_sink_cp_permute_rows(src, idx, False, out)
    dst = torch.full((6, 8), 5.0, device=DEV)
    sam().attn_sink_cp_permute_rows(src[:4], idx, True, dst)
    torch.cuda.synchronize()
    assert torch.equal(out[0], src[2]) and torch.equal(out[3], src[0])
    assert torch.all(out[1] == 0) and torch.all(out[2] == 0)
    assert torch.equal(dst[2], src[0]) and torch.equal(dst[0], src[3])
    assert torch.all(dst[[1, 3, 4, 5]] == 5.0)


def doc_positions(lens):
    return np.concatenate([np.arange(n) for n in lens]).astype(np.int64)


@pytest.mark.parametrize("positions", [
    doc_positions([3, 2, 4]), doc_positions([5]), np.array([3, 4, 0, 1, 0], dtype=np.int64),
    doc_positions(W.c5_doc_lens(0)), doc_positions([1] * 3000 + [7000, 1, 2]),
    np.random.default_rng(4).integers(0, 3, size=100_000).astype(np.int64), np.zeros(0, dtype=np.int64)])
def test_documents_bit_exact(positions):
    T = len(positions)
    want_ids = cp.document_ids(positions)
    want_cu = cp.segment_starts(positions)
    nseg = len(want_cu) - 1
    dpos = torch.from_numpy(positions).to(DEV)
    ids = torch.full((max(T, 1),), -9, dtype=torch.int32, device=DEV)
    cu = torch.full((nseg + 1,), -9, dtype=torch.int32, device=DEV)
    nd = torch.full((1,), -9, dtype=torch.int32, device=DEV)
    sam().attn_sink_cp_documents(dpos, ids, cu, nd)
    torch.cuda.synchronize()
    assert np.array_equal(ids[:T].cpu().numpy(), want_ids)
    assert np.array_equal(cu.cpu().numpy(), want_cu) and int(nd.item()) == nseg
    if nseg > 1:  # room for nseg - 1 boundaries only: those are written, then nothing, and the true count
        small = torch.full((nseg,), -9, dtype=torch.int32, device=DEV)
        sam().attn_sink_cp_documents(dpos, None, small, nd)
        torch.cuda.synchronize()
        got = small.cpu().numpy()
        assert np.array_equal(got[:nseg - 1], want_cu[:nseg - 1]) and got[nseg - 1] == -9
        assert int(nd.item()) == nseg


def test_cp_layout_block_sparse_end_to_end():
    """The block-sparse workload sharded as load-balanced CP over 8 ranks: the
    all-gathered K, V and position ids (rank-major) are put into global order
    on the GPU, the documents are derived from the positions, and the layer
    then gives exactly the same bytes as on the unsharded inputs."""
    case = W.make_workload("blocksparse_32k", seed=0, sink_mode="null_logit")
    d = sam().case_on_device(case, DEV)
    T = d["q"].shape[0]
    cp_size = 8
    slots = torch.empty(T, dtype=torch.int64, device=DEV)
    sam().attn_sink_cp_slots(cp_size, T // cp_size, -1, slots)
    positions = torch.from_numpy(doc_positions(np.diff(case["cu_seqlens"]))).to(DEV)
    gathered = {n: d[n][slots] for n in ("k", "v")}
    gathered_pos = positions[slots]
    glob = {n: torch.empty_like(gathered[n]) for n in gathered}
    for n in glob:
        sam().attn_sink_cp_permute_rows(gathered[n], slots, True, glob[n])
    pos_glob = torch.empty_like(gathered_pos)
    sam().attn_sink_cp_permute_rows(gathered_pos, slots, True, pos_glob)
    cu = torch.empty(len(case["cu_seqlens"]), dtype=torch.int32, device=DEV)
    nd = torch.empty(1, dtype=torch.int32, device=DEV)
    sam().attn_sink_cp_documents(pos_glob, None, cu, nd)
    ref_o, ref_l = sam().fwd(**d)
    o, l = sam().fwd(**dict(d, k=glob["k"], v=glob["v"], cu_seqlens=cu))
    torch.cuda.synchronize()
    assert int(nd.item()) == len(case["cu_seqlens"]) - 1
    assert torch.equal(cu.cpu(), d["cu_seqlens"].cpu())
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
