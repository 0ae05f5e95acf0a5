"""Layout compiler invariants, read back through bsmm_debug_lut (CPU only)."""
import itertools

import numpy as np
import pytest

import block_sparse_matrix_amd as bs
import synth

COORDS, COLPTR, COLENT, ROWPTR, ROWENT, COLORDER, ROWORDER, COLWORK, ROWWORK = range(9)
COLREC, ROWREC = 10, 11


def check_layout(L, b=8, fa=1):
    L = np.ascontiguousarray(L, dtype=np.uint8)
    R, S = L.shape
    m = bs.BlocksparseMatMul(L, block_size=b, feature_axis=fa)
    h = m.handle
    nnz = int(L.sum())
    cs, ks = np.nonzero(L)
    coords = bs.bsmm_debug_lut(h, COORDS).reshape(-1, 2)
    assert np.array_equal(coords, np.stack([cs, ks], 1).reshape(-1, 2))
    id_of = -np.ones((R, S), dtype=np.int64)
    id_of[cs, ks] = np.arange(nnz)

    colptr = bs.bsmm_debug_lut(h, COLPTR)
    assert np.array_equal(colptr, np.concatenate([[0], np.cumsum(L.sum(0))]))
    colent = bs.bsmm_debug_lut(h, COLENT).reshape(-1, 2)
    seen = np.zeros(nnz, dtype=int)
    for k in range(S):
        ent = colent[colptr[k]:colptr[k + 1]]
        assert np.all(np.diff(ent[:, 0]) > 0)             # ascending c, no repeats
        assert np.array_equal(ent[:, 0], np.flatnonzero(L[:, k]))
        assert np.array_equal(ent[:, 1], id_of[ent[:, 0], k])
        seen[ent[:, 1]] += 1
    assert np.all(seen == 1)

    rowptr = bs.bsmm_debug_lut(h, ROWPTR)
    assert np.array_equal(rowptr, np.concatenate([[0], np.cumsum(L.sum(1))]))
    rowent = bs.bsmm_debug_lut(h, ROWENT).reshape(-1, 2)
    seen[:] = 0
    for c in range(R):
        ent = rowent[rowptr[c]:rowptr[c + 1]]
        assert np.array_equal(ent[:, 0], np.flatnonzero(L[c]))
        assert np.array_equal(ent[:, 1], id_of[c, ent[:, 0]])
        seen[ent[:, 1]] += 1
    assert np.all(seen == 1)

    for which, counts in ((COLORDER, L.sum(0)), (ROWORDER, L.sum(1))):
        order = bs.bsmm_debug_lut(h, which)
        assert sorted(order.tolist()) == list(range(len(counts)))
        key = [(-int(counts[i]), int(i)) for i in order]
        assert key == sorted(key)

    # records: the work descriptor of each list in processing order, then its first
    # entries inline (zero padded to the common stride)
    for ow, ww, rw, ptr, ent in ((COLORDER, COLWORK, COLREC, colptr, colent),
                                 (ROWORDER, ROWWORK, ROWREC, rowptr, rowent)):
        order = bs.bsmm_debug_lut(h, ow)
        work = bs.bsmm_debug_lut(h, ww).reshape(-1, 4)
        lens = np.diff(ptr)
        rs = max(2, (min(int(lens.max(initial=0)), 1024) + 1) // 2 * 2)
        rec = bs.bsmm_debug_lut(h, rw).reshape(len(order), 4 + 2 * rs)
        assert np.array_equal(work[:, 0], order)
        assert np.array_equal(work[:, 1], ptr[order])
        assert np.array_equal(work[:, 2], lens[order])
        assert np.array_equal(rec[:, :4], work)
        for i, o in enumerate(order):
            n = min(int(lens[o]), rs)
            inline = rec[i, 4:].reshape(-1, 2)
            assert np.array_equal(inline[:n], ent[ptr[o]:ptr[o] + n])
            assert np.all(inline[n:] == 0)


def test_every_tiny_layout():
    for R, S in [(1, 1), (1, 2), (2, 1), (2, 2), (2, 3), (3, 2), (3, 3)]:
        for bits in itertools.product([0, 1], repeat=R * S):
            check_layout(np.array(bits).reshape(R, S))


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_workload_layouts(name):
    wl = synth.WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    R = wl.hidden // wl.block
    L = synth.make_layout(wl.layout_kind, R, R, rng)
    check_layout(L, wl.block, wl.fa)
    if name == "hidden4096_b16_n512":
        assert L.sum(0).min() >= 1 and L.sum(1).min() >= 1
    if name == "hidden8192_b8_n1024":
        assert np.all(np.diag(L) == 1)
    if name == "hidden8192_b32_n4096_g8":
        assert int(L.sum()) == round(0.03 * R * R)
        c, k = np.meshgrid(np.arange(R), np.arange(R), indexing="ij")
        assert np.all(L[np.abs(c - k) <= 2] == 1)


def test_updat_groups_cover_every_block_once():
    rng = np.random.default_rng(3)
    for R, S, p in [(5, 40, 0.5), (17, 9, 0.3), (1, 1, 1.0), (6, 6, 0.0)]:
        L = (rng.random((R, S)) < p).astype(np.uint8)
        m = bs.BlocksparseMatMul(L, block_size=8)
        g = bs.bsmm_debug_lut(m.handle, 9).reshape(-1, 4)
        coords = bs.bsmm_debug_lut(m.handle, 0).reshape(-1, 2)
        seen = np.zeros(int(L.sum()), dtype=int)
        for id0, cnt, c, _ in g:
            assert 1 <= cnt <= 8
            assert np.all(coords[id0:id0 + cnt, 0] == c)
            seen[id0:id0 + cnt] += 1
        assert np.all(seen == 1)
        assert list(g[:, 0]) == sorted(g[:, 0])


def test_records_of_lists_longer_than_the_inline_cap():
    # a column (fprop list) of 1100 blocks keeps only its first 1024 entries inline
    L = np.zeros((1100, 3), dtype=np.uint8)
    L[:, 1] = 1
    L[::7, 2] = 1
    check_layout(L)
    check_layout(L.T.copy())
