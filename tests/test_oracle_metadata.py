"""Pins of the paging-metadata definitions in oracle/metadata.py against
hand-worked cases (lucebox PR #555, Summary: resident block table updated
entry by entry; Roadmap item 6: prefix blocks shared under reference counts
and copied on write)."""
import numpy as np
import pytest

from oracle.metadata import PrefixPoolModel, copy_blocks, table_update


def test_table_update_hand_worked():
    table = np.zeros((2, 3), dtype=np.int32)
    seq = np.array([5, 6], dtype=np.int32)
    t, s = table_update(table, seq, [(0, 1, 7), (1, -1, 33), (1, 2, 5)])
    assert t.tolist() == [[0, 7, 0], [0, 0, 5]]
    assert s.tolist() == [5, 33]
    assert table.tolist() == [[0, 0, 0], [0, 0, 0]] and seq.tolist() == [5, 6]   # inputs untouched
    with pytest.raises(ValueError):
        table_update(table, seq, [(0, 1, 7), (0, 1, 8)])
    with pytest.raises(IndexError):
        table_update(table, seq, [(0, 3, 1)])


def test_copy_blocks_hand_worked():
    pool = np.arange(4 * 3, dtype=np.uint8).reshape(4, 3)       # block i holds 3i, 3i+1, 3i+2
    out = copy_blocks(pool, [0, 3], [2, 1])
    assert out.tolist() == [[0, 1, 2], [9, 10, 11], [0, 1, 2], [9, 10, 11]]
    # sources are read as they were before any copy
    out = copy_blocks(pool, [1, 2], [2, 3])
    assert out[3].tolist() == [6, 7, 8] and out[2].tolist() == [3, 4, 5]


def test_prefix_model_hand_worked():
    m = PrefixPoolModel(5)
    m.alloc(1, [0, 1, 2])
    m.fork(1, 2, 2)
    assert [m.refcount(i) for i in range(5)] == [2, 2, 1, 0, 0]
    assert m.cow(2, 1, 3) == (3, 1)
    assert m.allocs[2] == [0, 3]
    assert [m.refcount(i) for i in range(5)] == [2, 1, 1, 1, 0]
    m.release(1)
    assert [m.refcount(i) for i in range(5)] == [1, 0, 0, 1, 0]
    assert m.free() == {1, 2, 4}
    assert m.cow(2, 0, None) == (0, -1)                          # private now: write in place
    with pytest.raises(ValueError):
        m.alloc(3, [0])                                          # 0 is held
    m.fork(2, 2, 4)
    with pytest.raises(ValueError):
        m.cow(4, 1, 3)                                           # 3 is held by 2 and 4
    m.reset()
    assert m.free() == set(range(5))
