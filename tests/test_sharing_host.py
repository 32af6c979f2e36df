"""Prefix sharing on the host: the oracle's bookkeeping check against planted
mistakes, the library's share / copy-on-write / release calls over seeded
walks (checked with the oracle's rules and a CPU model of the pools), and
their argument errors.  No GPU."""
import os

import numpy as np
import pytest

import paged_kv_attention_17_amd as pkv
from paged_kv_attention_17_amd import _abi
from oracle import paging

from sharing_walk import SharingWalk

FAKE = 1 << 20


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.LIB_PATH):
        from paged_kv_attention_17_amd import build
        build.build()
    return pkv.load()


# ------------------------------------------------------------ oracle pins --

def test_refcount_problems_catches_planted_mistakes():
    bt = np.array([[0, 1, -1], [0, 2, -1], [3, -1, -1]], np.int32)
    rc = np.array([2, 1, 1, 1, 0, 0], np.int32)
    free = np.array([4, 5], np.int32)
    assert paging.refcount_problems([bt], rc, free) == []
    # a count one short (block 0 listed twice, counted once)
    rc2 = rc.copy()
    rc2[0] = 1
    assert paging.refcount_problems([bt], rc2, free)
    # a listed block also on the free list
    assert paging.refcount_problems([bt], rc, np.array([4, 3], np.int32))
    # a free block with a stale count
    rc3 = rc.copy()
    rc3[5] = 1
    assert paging.refcount_problems([bt], rc3, free)
    # the free list holding a block twice
    assert paging.refcount_problems([bt], rc, np.array([4, 4], np.int32))
    # an entry outside the pool
    bt2 = bt.copy()
    bt2[2, 1] = 6
    assert paging.refcount_problems([bt2], rc, free)
    # counts summed over several table views (layers)
    assert paging.refcount_problems([bt[:2], bt[2:]], rc, free) == []


def test_copy_blocks_keeps_what_rows_read():
    """Moving a row's entry to a copy of its block leaves what the row gathers
    unchanged, and no other block changes."""
    rng = np.random.default_rng(3)
    k = rng.integers(0, 1 << 16, (6, 16, 2, 64), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, (6, 16, 2, 64), dtype=np.uint16)
    k_in, v_in = k.copy(), v.copy()
    row = np.array([2, 4, -1], np.int32)
    before_k = paging.gather(k, row, 29)
    before_v = paging.gather(v, row, 29)
    k2, v2 = paging.copy_blocks(k, v, [4, 2], [5, 0])
    moved = np.array([0, 5, -1], np.int32)
    np.testing.assert_array_equal(paging.gather(k2, moved, 29), before_k)
    np.testing.assert_array_equal(paging.gather(v2, moved, 29), before_v)
    for b in (1, 2, 3, 4):
        np.testing.assert_array_equal(k2[b], k[b])
        np.testing.assert_array_equal(v2[b], v[b])
    np.testing.assert_array_equal(k, k_in)
    np.testing.assert_array_equal(v, v_in)


# --------------------------------------------------------------- the walk --

@pytest.mark.parametrize("seed", [1, 2, 3])
def test_sharing_walk_host(lib, seed):
    w = SharingWalk(seed)
    saved = 0
    for _ in range(80):
        w.step()
        w.check()
        # blocks in use vs table entries listing blocks
        saved = max(saved, int(np.count_nonzero(w.bt >= 0)) - int(np.count_nonzero(w.refcount)))
    assert w.n_copies > 0 and w.n_forks > 0 and saved > 0


def test_fork_then_both_append_same_block(lib):
    """Two rows sharing a partly filled block both append in one call: the
    first one reached moves to a copy, the second then holds the block alone
    and writes it in place."""
    bt = np.full((3, 4), -1, np.int32)
    rc = np.zeros(8, np.int32)
    free = np.arange(8, dtype=np.int32)[::-1].copy()        # pops 0, 1, 2, ...
    nf, _, _ = pkv.pkv_blocks_assign(bt, free, 8, np.zeros(20, np.int32), np.arange(20, dtype=np.int32))
    rc[bt[0][bt[0] >= 0]] = 1
    off, val = pkv.pkv_blocks_share(bt, 0, 1, 20, rc)
    assert list(bt[1, :2]) == list(bt[0, :2]) and list(rc[:2]) == [2, 2]
    assert list(off) == [4, 5] and list(val) == list(bt[0, :2])
    shared_tail = int(bt[0, 1])
    nf, off, val, cs, cd = pkv.pkv_blocks_assign_shared(bt, free, nf, rc, np.array([0, 1], np.int32),
                                                        np.array([20, 20], np.int32))
    assert list(cs) == [shared_tail] and len(cd) == 1
    assert bt[0, 1] == cd[0] and bt[1, 1] == shared_tail
    assert rc[shared_tail] == 1 and rc[cd[0]] == 1 and rc[bt[0, 0]] == 2
    assert list(off) == [1] and list(val) == [cd[0]]
    assert paging.refcount_problems([bt], rc, free[:nf]) == []
    # releasing row 1 frees nothing that row 0 still lists
    nf2, _, _ = pkv.pkv_blocks_release_shared(bt, 1, free, nf, rc)
    assert nf2 == nf + 1 and free[nf2 - 1] == shared_tail and rc[bt[0, 0]] == 1
    assert paging.refcount_problems([bt], rc, free[:nf2]) == []


def test_sharing_calls_are_all_or_nothing(lib):
    bt = np.full((3, 4), -1, np.int32)
    rc = np.zeros(6, np.int32)
    free = np.arange(6, dtype=np.int32)
    nf, _, _ = pkv.pkv_blocks_assign(bt, free, 6, np.zeros(40, np.int32), np.arange(40, dtype=np.int32))
    rc[bt[0][bt[0] >= 0]] = 1
    pkv.pkv_blocks_share(bt, 0, 1, 40, rc)
    snap = (bt.copy(), rc.copy(), free.copy(), nf)
    # rows 0 and 1 both write into their shared third block (only the first
    # moves to a copy) and row 1 opens a fourth: two blocks, one free
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.pkv_blocks_assign_shared(bt, free, 1, rc, np.array([0, 1, 1], np.int32), np.array([40, 40, 48], np.int32))
    assert e.value.status == _abi.PKV_ERR_CAPACITY
    np.testing.assert_array_equal(bt, snap[0])
    np.testing.assert_array_equal(rc, snap[1])
    np.testing.assert_array_equal(free, snap[2])
    # sharing into a row that already holds blocks
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.pkv_blocks_share(bt, 0, 1, 16, rc)
    assert e.value.status == _abi.PKV_ERR_INVALID_ARG
    # sharing tokens the source does not hold
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.pkv_blocks_share(bt, 0, 2, 60, rc)
    assert e.value.status == _abi.PKV_ERR_BAD_BLOCK
    # a count that does not cover the row's entries
    rc_bad = rc.copy()
    rc_bad[bt[1, 0]] = 1
    bt_c = bt.copy()
    pkv.pkv_blocks_release_shared(bt_c, 0, free.copy(), nf, rc_bad)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.pkv_blocks_release_shared(bt_c, 1, free.copy(), nf + 0, rc_bad)
    assert e.value.status == _abi.PKV_ERR_INVALID_ARG
    np.testing.assert_array_equal(bt, snap[0])


def test_blocks_copy_argument_errors(lib):
    E = _abi

    def call(src, dst, nb=8, n_kv=8, hd=64, kp=FAKE, vp=FAKE):
        s = np.array(src, np.int32)
        d = np.array(dst, np.int32)
        return lib.pkv_blocks_copy(kp, vp, nb, n_kv, hd, s.ctypes.data, d.ctypes.data, len(s), None)

    assert call([], []) == E.PKV_OK
    assert call([0], [1], hd=32) == E.PKV_ERR_UNSUPPORTED
    assert call([0], [1], kp=None) == E.PKV_ERR_NULL
    assert call([0], [1], vp=FAKE + 8) == E.PKV_ERR_MISALIGNED
    assert call([0], [8]) == E.PKV_ERR_BAD_BLOCK
    assert call([-1], [2]) == E.PKV_ERR_BAD_BLOCK
    assert call([0, 1], [2, 2]) == E.PKV_ERR_INVALID_ARG        # block written twice
    assert call([0, 2], [2, 3]) == E.PKV_ERR_INVALID_ARG        # block both written and read
    assert call([2, 0], [3, 2]) == E.PKV_ERR_INVALID_ARG        # same, other order
    assert lib.pkv_blocks_copy(FAKE, FAKE, 8, 8, 64, None, None, 1, None) == E.PKV_ERR_NULL
    assert lib.pkv_blocks_copy(FAKE, FAKE, 8, 8, 64, None, None, -1, None) == E.PKV_ERR_INVALID_ARG
