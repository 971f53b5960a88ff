"""Plain definitions of the paging-metadata operations.

TEST INFRASTRUCTURE ONLY. Only the tests may import this module; the product
path (the C-ABI library and its Python binding) never does, and shares no code
with it.

Sources (page titles and sections):
  * lucebox PR #555 "paged-attention monolithic decode-only AR foundation",
    Summary: the table and lengths live on the device beside the pool, so a
    step sends only the ids of newly allocated blocks rather than re-sending
    the table.
  * the same page, Roadmap item 6: prefix caching, where blocks of a common
    prefix are shared under reference counts and copied before a write.

Each function states the result directly: an update list applied entry by
entry, a block copy as array slicing, and allocator state as a set of block
lists from which every reference count is recounted on demand.
"""
from __future__ import annotations

import numpy as np

__all__ = ["table_update", "copy_blocks", "PrefixPoolModel"]


def table_update(table: np.ndarray, seq_len: np.ndarray, updates):
    """Return copies of table [B, max_blocks] and seq_len [B] with every
    (b, slot, value) triple applied: slot >= 0 writes table[b, slot], slot ==
    -1 writes seq_len[b]. Two triples naming the same entry raise (the result
    would depend on their order)."""
    t = np.array(table, dtype=np.int32, copy=True)
    s = np.array(seq_len, dtype=np.int32, copy=True)
    seen = set()
    for b, slot, value in updates:
        key = (int(b), int(slot))
        if key in seen:
            raise ValueError(f"entry {key} updated twice")
        seen.add(key)
        if slot == -1:
            s[b] = value
        elif 0 <= slot < t.shape[1]:
            t[b, slot] = value
        else:
            raise IndexError(f"slot {slot} outside [-1, {t.shape[1]})")
    return t, s


def copy_blocks(pool: np.ndarray, src_ids, dst_ids) -> np.ndarray:
    """Return a copy of pool [nblocks, ...] in which block dst_ids[i] holds the
    bytes of block src_ids[i] (taken from the pool as it was before any copy)."""
    before = np.array(pool, copy=True)
    out = np.array(pool, copy=True)
    for s, d in zip(src_ids, dst_ids):
        out[d] = before[s]
    return out


class PrefixPoolModel:
    """Allocator state as plain data: each live allocation is a list of block
    ids; the reference count of a block is the number of allocations that
    list it, recounted every time; a block is free when its count is 0."""

    def __init__(self, nblocks: int):
        self.nblocks = nblocks
        self.allocs: dict[int, list[int]] = {}

    def refcount(self, block: int) -> int:
        return sum(ids.count(block) for ids in self.allocs.values())

    def free(self) -> set[int]:
        return {i for i in range(self.nblocks) if self.refcount(i) == 0}

    def alloc(self, handle: int, ids) -> None:
        """Record that `ids` (which must all be free) were appended to
        allocation `handle` (created if new)."""
        ids = list(ids)
        if len(set(ids)) != len(ids) or not set(ids) <= self.free():
            raise ValueError("allocated ids must be distinct free blocks")
        self.allocs.setdefault(handle, []).extend(ids)

    def fork(self, src: int, n_shared: int, handle: int) -> None:
        """A new allocation whose blocks are the first n_shared of src."""
        if not 0 <= n_shared <= len(self.allocs[src]):
            raise ValueError("n_shared outside the source allocation")
        self.allocs[handle] = list(self.allocs[src][:n_shared])

    def cow(self, handle: int, index: int, new_id: int | None):
        """Copy-on-write of block `index`: a block listed by no other
        allocation stays (returns (id, -1)); otherwise it is replaced by
        new_id, a free block (returns (new_id, old id))."""
        old = self.allocs[handle][index]
        if self.refcount(old) == 1:
            return old, -1
        if new_id is None or new_id not in self.free():
            raise ValueError("copy-on-write of a shared block needs a free block")
        self.allocs[handle][index] = new_id
        return new_id, old

    def release(self, handle: int) -> None:
        del self.allocs[handle]

    def reset(self) -> None:
        self.allocs.clear()
