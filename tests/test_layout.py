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


def check_groups(L, m):
    """Output-block groups of 8 (block size 32): every present block appears exactly
    once, under its contraction index, with its id; contraction indices ascend."""
    h = m.handle
    R, S = L.shape
    cs, ks = np.nonzero(L)
    id_of = -np.ones((R, S), dtype=np.int64)
    id_of[cs, ks] = np.arange(len(cs))
    for pw, ew, Lo in ((12, 13, L), (14, 15, L.T)):   # fprop: (c, k); bprop: (k, c)
        gptr = bs.bsmm_debug_lut(h, pw)
        gent = bs.bsmm_debug_lut(h, ew).reshape(-1, 12)
        nout = Lo.shape[1]
        assert len(gptr) == (nout + 7) // 8 + 1 and gptr[0] == 0 and gptr[-1] == len(gent)
        seen = np.zeros(L.shape, dtype=int)
        for g in range(len(gptr) - 1):
            ent = gent[gptr[g]:gptr[g + 1]]
            assert np.all(np.diff(ent[:, 0]) > 0)
            blk = Lo[:, 8 * g:8 * g + 8]
            assert np.array_equal(ent[:, 0], np.flatnonzero(blk.any(1)))
            for u, mask, *rest in ent:
                ids = rest[:8]
                for j in range(8):
                    o = 8 * g + j
                    present = o < nout and Lo[u, o] == 1
                    assert bool(mask >> j & 1) == present
                    if present:
                        ref = id_of[u, o] if pw == 12 else id_of[o, u]
                        assert ids[j] == ref
                        if pw == 12:
                            seen[u, o] += 1
                        else:
                            seen[o, u] += 1
                    else:
                        assert ids[j] == 0
                assert rest[8] == 0 and rest[9] == 0
        assert np.array_equal(seen, L.astype(int))


def test_groups_of_32_blocks():
    rng = np.random.default_rng(5)
    for R, S, p in [(5, 40, 0.5), (17, 9, 0.3), (1, 1, 1.0), (6, 6, 0.0), (33, 64, 0.05)]:
        L = (rng.random((R, S)) < p).astype(np.uint8)
        check_groups(L, bs.BlocksparseMatMul(L, block_size=32))
    for b in (8, 16):   # only built for block size 32
        m = bs.BlocksparseMatMul(np.ones((3, 3), np.uint8), block_size=b)
        assert all(len(bs.bsmm_debug_lut(m.handle, w)) == 0 for w in (12, 13, 14, 15))


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


def test_weight_gradient_tiles_and_rest_cover_every_block_once():
    """32x32 blocks: dense 8x8 tiles (>= 16 blocks) plus row groups of the rest hold
    every block exactly once, with the right coordinates."""
    rng = np.random.default_rng(9)
    for R, S, p in [(20, 27, 0.5), (16, 16, 0.03), (9, 40, 0.3), (1, 1, 1.0), (8, 8, 1.0), (5, 5, 0.0)]:
        L = (rng.random((R, S)) < p).astype(np.uint8)
        if R >= 16:
            L[np.abs(np.subtract.outer(np.arange(R), np.arange(S))) <= 2] = 1
        m = bs.BlocksparseMatMul(L, block_size=32)
        coords = bs.bsmm_debug_lut(m.handle, 0).reshape(-1, 2)
        tiles = bs.bsmm_debug_lut(m.handle, 16).reshape(-1, 4)
        tblk = bs.bsmm_debug_lut(m.handle, 17)
        rest = bs.bsmm_debug_lut(m.handle, 18).reshape(-1, 4)
        rids = bs.bsmm_debug_lut(m.handle, 19)
        seen = np.zeros(int(L.sum()), dtype=int)
        for ti, (r0, c0, n, first) in enumerate(tiles):
            assert r0 % 8 == 0 and c0 % 8 == 0 and n >= 16 and first == 64 * ti
            assert n == int(L[r0:r0 + 8, c0:c0 + 8].sum())
            pos = tblk[first:first + 64].reshape(8, 8)
            for lr in range(8):
                for lc in range(8):
                    bid = pos[lr, lc]
                    inside = r0 + lr < R and c0 + lc < S
                    if inside and L[r0 + lr, c0 + lc]:
                        assert bid >= 0 and tuple(coords[bid]) == (r0 + lr, c0 + lc)
                        seen[bid] += 1
                    else:
                        assert bid == -1
        sizes = {}
        for first, n, c, flag in rest:
            assert flag == 1 and 1 <= n <= 2
            ids = rids[first:first + n]
            assert np.all(coords[ids, 0] == c) and np.all(np.diff(coords[ids, 1]) > 0)
            seen[ids] += 1
            sizes.setdefault(int(c), []).append(int(n))
        assert np.all(seen == 1)
        for c, sz in sizes.items():   # fewest groups of <= 2, sizes within 1 of each other
            assert len(sz) == (sum(sz) + 1) // 2 and max(sz) - min(sz) <= 1
    m8 = bs.BlocksparseMatMul(np.ones((16, 16), np.uint8), block_size=16)
    assert all(len(bs.bsmm_debug_lut(m8.handle, w)) == 0 for w in (16, 17, 18, 19))


def test_small_block_gradient_tiles_cover_every_block_once():
    """8x8 and 16x16 blocks: the 256 x 256-feature weight-gradient tiles list every
    block exactly once at its own quad, with per-quad-row lists of exactly the quads
    that hold a block (ascending), tiles without blocks left out, tiles in
    super-blocks of 4 x 8 tiles."""
    rng = np.random.default_rng(11)
    for b in (8, 16):
        TB = 256 // b
        QB = 2 if b == 8 else 1
        for R, S, p in [(40, 70, 0.1), (TB, TB, 1.0), (3, 5, 0.5), (2 * TB + 3, 9 * TB + 1, 0.004), (4, 4, 0.0)]:
            L = (rng.random((R, S)) < p).astype(np.uint8)
            m = bs.BlocksparseMatMul(L, block_size=b)
            coords = bs.bsmm_debug_lut(m.handle, 0).reshape(-1, 2)
            tiles = bs.bsmm_debug_lut(m.handle, 20).reshape(-1, 4)
            plans = bs.bsmm_debug_lut(m.handle, 21).reshape(-1, 16, 8)
            ids = bs.bsmm_debug_lut(m.handle, 22).reshape(-1, 16, 16, QB, QB)
            assert len(tiles) == len(plans) == len(ids)
            seen = np.zeros(int(L.sum()), dtype=int)
            cells = []
            for t, (f0, g0, first, zero) in enumerate(tiles):
                assert f0 % 256 == 0 and g0 % 256 == 0 and zero == 0
                assert first == t * 256 * QB * QB
                tr, tc = f0 // 256, g0 // 256
                cells.append((tr, tc))
                n = 0
                for qi in range(16):
                    for qj in range(16):
                        blk = ids[t, qi, qj]
                        for di in range(QB):
                            for dj in range(QB):
                                r, c = tr * TB + qi * QB + di, tc * TB + qj * QB + dj
                                if r < R and c < S and L[r, c]:
                                    bid = blk[di, dj]
                                    assert bid >= 0 and tuple(coords[bid]) == (r, c)
                                    seen[bid] += 1
                                    n += 1
                                else:
                                    assert blk[di, dj] == -1
                counts = [sum(np.any(ids[t, qi, qj] >= 0) for qj in range(16)) for qi in range(16)]
                assert sorted(int(r) for r in plans[t, :, 5]) == list(range(16))   # every row once
                for wv in range(16):
                    qi = int(plans[t, wv, 5])
                    present = [qj for qj in range(16) if np.any(ids[t, qi, qj] >= 0)]
                    cnt = int(plans[t, wv, 0])
                    cols = plans[t, wv, 1:5].astype(np.uint32).view(np.uint8)   # little-endian bytes
                    assert cnt == len(present) and list(cols[:cnt]) == present
                    assert np.all(cols[cnt:] == 0) and np.all(plans[t, wv, 6:] == 0)
                # waves w, w+4, w+8, w+12 share a SIMD: dealt fullest row first to the
                # least-loaded SIMD, no SIMD ends more than one row's count above another
                simd = [sum(counts[int(plans[t, wv, 5])] for wv in range(sm, 16, 4)) for sm in range(4)]
                assert max(simd) - min(simd) <= max(counts)
                assert n > 0
            assert np.all(seen == 1)
            key = [(tr // 4, tc // 8, tr, tc) for tr, tc in cells]
            assert key == sorted(key)
    m = bs.BlocksparseMatMul(np.ones((3, 3), np.uint8), block_size=32)
    assert all(len(bs.bsmm_debug_lut(m.handle, w)) == 0 for w in (20, 21, 22))
