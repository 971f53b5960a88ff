// Fixed-block K/V allocator over the block ids of a caller-owned pool.
//
// Behaviour from the lucebox PR #555 page (Summary; Validation): exact
// fixed-block allocation (an allocation holds exactly the blocks asked for),
// transactional allocation (all or nothing), stale-handle detection, immediate
// release, and a pool reset across requests.
//
// Design: free ids sit on a stack (popped lowest-first on a fresh pool, so a
// fresh pool hands out 0, 1, 2, ...). Allocations live in slots; a handle is
// (generation << 32) | (slot + 1). Releasing a slot bumps its generation and a
// reset bumps the generation of every slot, so every old handle stops matching.
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
  if (slot < 0) {
    if (pool->free_slots.empty()) {
      pool->slots.emplace_back();
      slot = int64_t(pool->slots.size() - 1);
    } else {
      slot = pool->free_slots.back();
      pool->free_slots.pop_back();
    }
    pool->slots[size_t(slot)].live = true;
    pool->slots[size_t(slot)].ids.clear();
  }
  auto& s = pool->slots[size_t(slot)];
  s.ids.reserve(s.ids.size() + size_t(n));
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = pool->free_ids.back();
    pool->free_ids.pop_back();
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
  // Released blocks go back so that the most recently released is reused first.
  for (auto it = s.ids.rbegin(); it != s.ids.rend(); ++it) pool->free_ids.push_back(*it);
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
