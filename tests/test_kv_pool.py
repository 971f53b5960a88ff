"""The fixed-block allocator (kv_pool_*) against a plain Python model:
transactional allocation, exact block counts, immediate release, stale-handle
detection and reset (lucebox PR #555, Summary and Validation)."""
import random

import pytest

from oracle.metadata import PrefixPoolModel
from test_lib_cpu import pa  # builds the library if needed


def test_fresh_pool_hands_out_ids_in_order_and_exactly():
    p = pa.KvPool(10)
    h, ids = p.alloc(3)
    assert ids == [0, 1, 2] and p.count(h) == 3 and p.free_count() == 7
    h2, ids2 = p.alloc(2, h)
    assert h2 == h and ids2 == [3, 4] and p.blocks(h) == [0, 1, 2, 3, 4]


def test_capacity_failure_changes_nothing():
    p = pa.KvPool(5)
    h, _ = p.alloc(4)
    with pytest.raises(pa.PaError) as e:
        p.alloc(2, h)
    assert e.value.code == pa.PA_ERR_CAPACITY and "kv_pool_alloc" in str(e.value)
    assert p.count(h) == 4 and p.free_count() == 1
    with pytest.raises(pa.PaError):
        p.alloc(2)                      # new allocation refused too, no slot leaked
    assert p.free_count() == 1
    h2, ids = p.alloc(1)
    assert ids == [4]


def test_release_is_immediate_and_handles_go_stale():
    p = pa.KvPool(8)
    h, ids = p.alloc(5)
    p.release(h)
    assert p.free_count() == 8
    for op in (lambda: p.release(h), lambda: p.count(h), lambda: p.alloc(1, h),
               lambda: p.blocks(h)):
        with pytest.raises(pa.PaError) as e:
            op()
        assert e.value.code == pa.PA_ERR_STALE_HANDLE
    h2, ids2 = p.alloc(5)
    assert h2 != h and sorted(ids2) == sorted(ids)


def test_reset_invalidates_every_handle():
    p = pa.KvPool(6)
    hs = [p.alloc(2)[0] for _ in range(3)]
    p.reset()
    assert p.free_count() == 6
    for h in hs:
        with pytest.raises(pa.PaError) as e:
            p.release(h)
        assert e.value.code == pa.PA_ERR_STALE_HANDLE
    h, ids = p.alloc(6)
    assert sorted(ids) == list(range(6)) and h not in hs


def test_invalid_handles_and_arguments():
    p = pa.KvPool(4)
    for h in (0, 1, 12345, (7 << 32) | 1):
        with pytest.raises(pa.PaError) as e:
            p.release(h)
        assert e.value.code == pa.PA_ERR_STALE_HANDLE
    with pytest.raises(pa.PaError) as e:
        p.alloc(-1)
    assert e.value.code == pa.PA_ERR_INVALID


def test_model_based_fuzz():
    rng = random.Random(1234)
    N = 64
    p = pa.KvPool(N)
    model = {}                     # handle -> list of ids
    free = set(range(N))
    stale = []
    for step in range(4000):
        op = rng.random()
        if op < 0.45:
            n = rng.randint(0, 9)
            grow = model and rng.random() < 0.5
            h = rng.choice(list(model)) if grow else 0
            if n > len(free):
                with pytest.raises(pa.PaError) as e:
                    p.alloc(n, h)
                assert e.value.code == pa.PA_ERR_CAPACITY
            else:
                h2, ids = p.alloc(n, h)
                assert len(ids) == n and set(ids) <= free and len(set(ids)) == n
                free -= set(ids)
                if grow:
                    assert h2 == h
                    model[h] += ids
                else:
                    model[h2] = list(ids)
        elif op < 0.8 and model:
            h = rng.choice(list(model))
            p.release(h)
            free |= set(model.pop(h))
            stale.append(h)
        elif op < 0.9 and stale:
            h = rng.choice(stale)
            with pytest.raises(pa.PaError) as e:
                p.alloc(1, h) if rng.random() < 0.5 else p.release(h)
            assert e.value.code == pa.PA_ERR_STALE_HANDLE
        elif op < 0.92:
            p.reset()
            stale += list(model)
            model.clear()
            free = set(range(N))
        assert p.free_count() == len(free)
        for h, ids in model.items():
            assert p.blocks(h) == ids


def test_fork_shares_the_prefix_and_counts_references():
    """lucebox PR #555, Roadmap item 6: prefix blocks shared under reference
    counts."""
    p = pa.KvPool(8)
    h, ids = p.alloc(3)
    f = p.fork(h, 2)
    assert p.blocks(f) == ids[:2] and p.count(f) == 2
    assert [p.refcount(i) for i in ids] == [2, 2, 1]
    assert p.free_count() == 5
    _, more = p.alloc(2, f)                      # the fork grows privately
    assert set(more).isdisjoint(ids) and p.blocks(f) == ids[:2] + more
    p.release(h)                                 # shared blocks stay with f
    assert [p.refcount(i) for i in ids] == [1, 1, 0] and p.free_count() == 4
    p.release(f)
    assert p.free_count() == 8 and all(p.refcount(i) == 0 for i in range(8))


def test_cow_replaces_only_shared_blocks_and_is_all_or_nothing():
    p = pa.KvPool(4)
    h, ids = p.alloc(2)
    assert p.cow(h, 1) == (ids[1], -1)           # private: write in place
    f = p.fork(h, 2)
    new, old = p.cow(f, 1)
    assert old == ids[1] and new not in ids and p.blocks(f) == [ids[0], new]
    assert p.refcount(old) == 1 and p.refcount(new) == 1
    g = p.fork(f, 2)
    p.alloc(1, g)                                # pool is now full
    assert p.free_count() == 0
    with pytest.raises(pa.PaError) as e:
        p.cow(g, 0)
    assert e.value.code == pa.PA_ERR_CAPACITY and "kv_pool_cow" in str(e.value)
    assert p.blocks(g)[:2] == [ids[0], new] and p.refcount(ids[0]) == 3
    for bad in (-1, 3):
        with pytest.raises(pa.PaError) as e:
            p.cow(g, bad)
        assert e.value.code == pa.PA_ERR_INVALID
    with pytest.raises(pa.PaError) as e:
        p.fork(h, 3)
    assert e.value.code == pa.PA_ERR_INVALID
    p.release(h)
    with pytest.raises(pa.PaError) as e:
        p.fork(h, 0)
    assert e.value.code == pa.PA_ERR_STALE_HANDLE
    with pytest.raises(pa.PaError) as e:
        p.refcount(4)
    assert e.value.code == pa.PA_ERR_INVALID


def test_model_based_fuzz_with_prefix_sharing():
    """Random alloc / fork / cow / release / reset against the set model of
    oracle/metadata.py, which recounts every reference from the block lists."""
    rng = random.Random(4321)
    N = 48
    p = pa.KvPool(N)
    m = PrefixPoolModel(N)
    stale = []
    for step in range(3000):
        op = rng.random()
        live = list(m.allocs)
        free = m.free()
        if op < 0.3:
            n = rng.randint(0, 6)
            h = rng.choice(live) if live and rng.random() < 0.5 else 0
            if n > len(free):
                with pytest.raises(pa.PaError) as e:
                    p.alloc(n, h)
                assert e.value.code == pa.PA_ERR_CAPACITY
            else:
                h2, ids = p.alloc(n, h)
                m.alloc(h2, ids)
        elif op < 0.45 and live:
            src = rng.choice(live)
            k = rng.randint(0, len(m.allocs[src]))
            h2 = p.fork(src, k)
            m.fork(src, k, h2)
        elif op < 0.65 and live:
            h = rng.choice(live)
            if m.allocs[h]:
                i = rng.randrange(len(m.allocs[h]))
                shared = m.refcount(m.allocs[h][i]) > 1
                if shared and not free:
                    with pytest.raises(pa.PaError) as e:
                        p.cow(h, i)
                    assert e.value.code == pa.PA_ERR_CAPACITY
                else:
                    new, old = p.cow(h, i)
                    assert (new, old) == m.cow(h, i, new if shared else None)
        elif op < 0.85 and live:
            h = rng.choice(live)
            p.release(h)
            m.release(h)
            stale.append(h)
        elif op < 0.9 and stale:
            h = rng.choice(stale)
            with pytest.raises(pa.PaError) as e:
                p.fork(h, 0) if rng.random() < 0.5 else p.cow(h, 0)
            assert e.value.code == pa.PA_ERR_STALE_HANDLE
        elif op < 0.91:
            p.reset()
            stale += list(m.allocs)
            m.reset()
        assert p.free_count() == len(m.free())
        for h, ids in m.allocs.items():
            assert p.blocks(h) == ids
        for i in rng.sample(range(N), 6):
            assert p.refcount(i) == m.refcount(i)
