// Fixed-block K/V allocator over the block ids of a caller-owned pool.
//
// Behaviour from the lucebox PR #555 page (Summary; Validation): exact
// fixed-block allocation (an allocation holds exactly the blocks asked for),
// transactional allocation (all or nothing), stale-handle detection, immediate
// release, and a pool reset across requests.
//
// Prefix sharing with reference counts and copy-on-write (lucebox PR #555,
// Roadmap item 6): an allocation can start as a fork of another's first
// blocks; a shared block returns to the pool when the last allocation holding
// it is released, and an allocation about to write into a shared block first
// swaps in a private copy.
//
// Design: free ids sit on a stack (popped lowest-first on a fresh pool, so a
// fresh pool hands out 0, 1, 2, ...); every id has a reference count (0 =
// free). Allocations live in slots; a handle is (generation << 32) |
// (slot + 1). Releasing a slot bumps its generation and a reset bumps the
// generation of every slot, so every old handle stops matching.
#include <algorithm>
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/paged_attn.h"
#include "pa_host.h"

struct kv_pool {
  int32_t nblocks = 0;
  std::vector<int32_t> free_ids;  // stack; back() is handed out next
  std::vector<int32_t> refs;      // allocations holding each id (0 = free)
  struct Slot {
    uint32_t gen = 1;
    bool live = false;
    std::vector<int32_t> ids;
  };
  std::vector<Slot> slots;
  std::vector<uint32_t> free_slots;
  mutable std::mutex mu;
};

namespace {

inline uint64_t make_handle(uint32_t slot, uint32_t gen) {
  return (uint64_t(gen) << 32) | uint64_t(slot + 1);
}

// Returns the slot of a live handle or -1.
int64_t find_slot(const kv_pool* p, uint64_t h) {
  uint32_t lo = uint32_t(h & 0xffffffffu);
  uint32_t gen = uint32_t(h >> 32);
  if (lo == 0 || lo > p->slots.size()) return -1;
  const auto& s = p->slots[lo - 1];
  if (!s.live || s.gen != gen) return -1;
  return int64_t(lo - 1);
}

void refill(kv_pool* p) {
  p->free_ids.resize(size_t(p->nblocks));
  for (int32_t i = 0; i < p->nblocks; ++i) p->free_ids[size_t(i)] = p->nblocks - 1 - i;
  p->refs.assign(size_t(p->nblocks), 0);
}

// A live slot for a new allocation (reused or appended).
int64_t open_slot(kv_pool* p) {
  int64_t slot;
  if (p->free_slots.empty()) {
    p->slots.emplace_back();
    slot = int64_t(p->slots.size() - 1);
  } else {
    slot = p->free_slots.back();
    p->free_slots.pop_back();
  }
  p->slots[size_t(slot)].live = true;
  p->slots[size_t(slot)].ids.clear();
  return slot;
}

// Drops one reference to id; the block is free again when none is left.
void unref(kv_pool* p, int32_t id) {
  if (--p->refs[size_t(id)] == 0) p->free_ids.push_back(id);
}

}  // namespace

extern "C" int32_t kv_pool_create(int32_t nblocks, kv_pool** pool) {
  if (!pool || nblocks < 0) return pa::fail(PA_ERR_INVALID, "kv_pool_create: null out-pointer or nblocks < 0");
  kv_pool* p = new (std::nothrow) kv_pool();
  if (!p) return pa::fail(PA_ERR_CAPACITY, "kv_pool_create: out of host memory");
  p->nblocks = nblocks;
  refill(p);
  *pool = p;
  return PA_OK;
}

extern "C" int32_t kv_pool_destroy(kv_pool* pool) {
  if (!pool) return pa::fail(PA_ERR_INVALID, "kv_pool_destroy: null pool");
  delete pool;
  return PA_OK;
}

extern "C" int32_t kv_pool_alloc(kv_pool* pool, int32_t n, int32_t* ids_out, uint64_t* handle) {
  if (!pool || !handle || n < 0 || (n > 0 && !ids_out))
    return pa::fail(PA_ERR_INVALID, "kv_pool_alloc: null pool/handle/ids_out or n < 0");
  std::lock_guard<std::mutex> lk(pool->mu);
  int64_t slot = -1;
  if (*handle != 0) {
    slot = find_slot(pool, *handle);
    if (slot < 0) return pa::fail(PA_ERR_STALE_HANDLE, "kv_pool_alloc: stale or unknown handle");
  }
  if (size_t(n) > pool->free_ids.size())
    return pa::fail(PA_ERR_CAPACITY, "kv_pool_alloc: not enough free blocks");
  // Everything below succeeds; reserve first so no allocation can throw midway.
  if (slot < 0) slot = open_slot(pool);
  auto& s = pool->slots[size_t(slot)];
  s.ids.reserve(s.ids.size() + size_t(n));
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = pool->free_ids.back();
    pool->free_ids.pop_back();
    pool->refs[size_t(id)] = 1;
    s.ids.push_back(id);
    ids_out[i] = id;
  }
  *handle = make_handle(uint32_t(slot), s.gen);
  return PA_OK;
}

extern "C" int32_t kv_pool_release(kv_pool* pool, uint64_t handle) {
  if (!pool) return pa::fail(PA_ERR_INVALID, "kv_pool_release: null pool");
  std::lock_guard<std::mutex> lk(pool->mu);
  int64_t slot = find_slot(pool, handle);
  if (slot < 0) return pa::fail(PA_ERR_STALE_HANDLE, "kv_pool_release: stale or unknown handle");
  auto& s = pool->slots[size_t(slot)];
  // Blocks no other allocation holds go back so that the most recently
  // released is reused first.
  for (auto it = s.ids.rbegin(); it != s.ids.rend(); ++it) unref(pool, *it);
  s.ids.clear();
  s.live = false;
  s.gen += 1;
  if (s.gen == 0) s.gen = 1;
  pool->free_slots.push_back(uint32_t(slot));
  return PA_OK;
}

extern "C" int32_t kv_pool_reset(kv_pool* pool) {
  if (!pool) return pa::fail(PA_ERR_INVALID, "kv_pool_reset: null pool");
  std::lock_guard<std::mutex> lk(pool->mu);
  pool->free_slots.clear();
  for (size_t i = pool->slots.size(); i-- > 0;) {
    auto& s = pool->slots[i];
    s.ids.clear();
    s.live = false;
    s.gen += 1;
    if (s.gen == 0) s.gen = 1;
    pool->free_slots.push_back(uint32_t(i));
  }
  refill(pool);
  return PA_OK;
}

extern "C" int32_t kv_pool_free_count(const kv_pool* pool) {
  if (!pool) return pa::fail(PA_ERR_INVALID, "kv_pool_free_count: null pool");
  std::lock_guard<std::mutex> lk(pool->mu);
  return int32_t(pool->free_ids.size());
}

extern "C" int32_t kv_pool_count(const kv_pool* pool, uint64_t handle) {
  if (!pool) return pa::fail(PA_ERR_INVALID, "kv_pool_count: null pool");
  std::lock_guard<std::mutex> lk(pool->mu);
  int64_t slot = find_slot(pool, handle);
  if (slot < 0) return pa::fail(PA_ERR_STALE_HANDLE, "kv_pool_count: stale or unknown handle");
  return int32_t(pool->slots[size_t(slot)].ids.size());
}

extern "C" int32_t kv_pool_blocks(const kv_pool* pool, uint64_t handle, int32_t* ids_out,
                                  int32_t cap) {
  if (!pool || cap < 0 || (cap > 0 && !ids_out))
    return pa::fail(PA_ERR_INVALID, "kv_pool_blocks: null pool/ids_out or cap < 0");
  std::lock_guard<std::mutex> lk(pool->mu);
  int64_t slot = find_slot(pool, handle);
  if (slot < 0) return pa::fail(PA_ERR_STALE_HANDLE, "kv_pool_blocks: stale or unknown handle");
  const auto& ids = pool->slots[size_t(slot)].ids;
  size_t k = std::min(ids.size(), size_t(cap));
  std::copy(ids.begin(), ids.begin() + k, ids_out);
  return int32_t(ids.size());
}

extern "C" int32_t kv_pool_fork(kv_pool* pool, uint64_t src, int32_t n_shared, uint64_t* handle) {
  if (!pool || !handle || n_shared < 0)
    return pa::fail(PA_ERR_INVALID, "kv_pool_fork: null pool/handle or n_shared < 0");
  std::lock_guard<std::mutex> lk(pool->mu);
  const int64_t from = find_slot(pool, src);
  if (from < 0) return pa::fail(PA_ERR_STALE_HANDLE, "kv_pool_fork: stale or unknown source handle");
  if (size_t(n_shared) > pool->slots[size_t(from)].ids.size())
    return pa::fail(PA_ERR_INVALID, "kv_pool_fork: n_shared %d exceeds the %zu blocks of the source",
                    n_shared, pool->slots[size_t(from)].ids.size());
  std::vector<int32_t> shared(pool->slots[size_t(from)].ids.begin(),
                              pool->slots[size_t(from)].ids.begin() + n_shared);
  const int64_t slot = open_slot(pool);    // may grow slots: index, do not hold references
  auto& s = pool->slots[size_t(slot)];
  s.ids = std::move(shared);
  for (int32_t id : s.ids) ++pool->refs[size_t(id)];
  *handle = make_handle(uint32_t(slot), s.gen);
  return PA_OK;
}

extern "C" int32_t kv_pool_cow(kv_pool* pool, uint64_t handle, int32_t index, int32_t* id_out,
                               int32_t* copy_from) {
  if (!pool || !id_out || !copy_from)
    return pa::fail(PA_ERR_INVALID, "kv_pool_cow: null pool, id_out or copy_from");
  std::lock_guard<std::mutex> lk(pool->mu);
  const int64_t slot = find_slot(pool, handle);
  if (slot < 0) return pa::fail(PA_ERR_STALE_HANDLE, "kv_pool_cow: stale or unknown handle");
  auto& s = pool->slots[size_t(slot)];
  if (index < 0 || size_t(index) >= s.ids.size())
    return pa::fail(PA_ERR_INVALID, "kv_pool_cow: index %d outside the %zu blocks of the allocation",
                    index, s.ids.size());
  const int32_t old = s.ids[size_t(index)];
  if (pool->refs[size_t(old)] == 1) {      // already private: write in place
    *id_out = old;
    *copy_from = -1;
    return PA_OK;
  }
  if (pool->free_ids.empty())
    return pa::fail(PA_ERR_CAPACITY, "kv_pool_cow: no free block for the private copy");
  const int32_t id = pool->free_ids.back();
  pool->free_ids.pop_back();
  pool->refs[size_t(id)] = 1;
  --pool->refs[size_t(old)];               // still held by another allocation
  s.ids[size_t(index)] = id;
  *id_out = id;
  *copy_from = old;
  return PA_OK;
}

extern "C" int32_t kv_pool_refcount(const kv_pool* pool, int32_t id) {
  if (!pool) return pa::fail(PA_ERR_INVALID, "kv_pool_refcount: null pool");
  std::lock_guard<std::mutex> lk(pool->mu);
  if (id < 0 || id >= pool->nblocks)
    return pa::fail(PA_ERR_INVALID, "kv_pool_refcount: id %d outside [0, %d)", id, pool->nblocks);
  return pool->refs[size_t(id)];
}
