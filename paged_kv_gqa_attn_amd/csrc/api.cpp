// C ABI of libpaged_attn: planning, host-side validation and dispatch of the
// decode, merge and gather kernels. Host-detectable problems are refused
// synchronously with a message naming the entry point (mlxcel issue #2153,
// Proposed Solution and Implementation Notes: refused launches report the
// entry point; the pool itself is never refused for its size).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/paged_attn.h"
#include "pa_host.h"
#include "wide_plan.h"

namespace pa {

namespace {
thread_local std::string g_err;

constexpr int kMaxB = 1024;
constexpr int kMaxR = 16;
constexpr int kTileTokens = 32;
constexpr int kWavesPerUnit = 4;
constexpr int kMaxChunk = 4096;   // query tokens per sequence in one chunk call
// MI355X dense f16 MFMA peak over HBM peak (2.5 PFLOP/s / 8 TB/s), flop per byte
constexpr double kFlopsPerByte = 2.5e15 / 8.0e12;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int ilog2_exact(int32_t v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int s = 0;
  while ((1 << s) != v) ++s;
  return s;
}

// Validates a shape; `who` names the entry point in messages.
int32_t check_shape(const pa_shape* s, const char* who) {
  if (!s) return fail(PA_ERR_INVALID, "%s: null shape", who);
  if (s->B < 1 || s->Hq < 1 || s->Hkv < 1 || s->D < 1 || s->nblocks < 1 || s->max_blocks < 1)
    return fail(PA_ERR_INVALID, "%s: B, Hq, Hkv, D, nblocks and max_blocks must be >= 1", who);
  if (s->Hq % s->Hkv)
    return fail(PA_ERR_INVALID, "%s: Hq (%d) is not a multiple of Hkv (%d)", who, s->Hq, s->Hkv);
  for (int32_t t : {s->k_type, s->v_type})
    if (t < PA_F16 || t > PA_Q4_0) return fail(PA_ERR_INVALID, "%s: unknown K/V type %d", who, t);
  const int bs_shift = ilog2_exact(s->block_size);
  if (bs_shift < 0) return fail(PA_ERR_INVALID, "%s: block_size %d is not a power of two", who, s->block_size);
  if (s->D != 128 && s->D != 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: head dimension D=%d is not compiled (supported: 128, 256)", who, s->D);
  if (s->Hq / s->Hkv > kMaxR)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d query heads per K/V head (at most %d)", who, s->Hq / s->Hkv, kMaxR);
  if (s->block_size < 16 || s->block_size > 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d outside [16, 256]", who, s->block_size);
  if (s->B > kMaxB) return fail(PA_ERR_UNSUPPORTED, "%s: B=%d above %d", who, s->B, kMaxB);
  if (int64_t(s->max_blocks) * s->block_size > INT32_MAX)
    return fail(PA_ERR_INVALID, "%s: max_blocks*block_size exceeds the int32 token range", who);
  return PA_OK;
}

// The LDS-staged kernel takes the shape: quads of kv heads, the batch prefix
// fits its LDS budget, and one step of both sides (16 or 8 token slots of
// four heads) fits a ring slot.
bool lds_path_ok(const pa_shape& s) {
  return s.Hkv % 4 == 0 && s.B <= kLdsMaxB && decode_group_slots(s.k_type, s.v_type, s.D) > 0;
}

// The single-launch merge runs the wide merge layout's slices; where the
// separate merge would take the row-per-thread layout, the step stays two
// launches (so that both paths give the same bits).
bool fused_merge_ok(const pa_shape& s, int p_max) {
  return !merge_rows_layout(int64_t(s.B) * s.Hq, p_max) && s.D % kMergeColsHost == 0;
}

int32_t check_plan(const pa_plan* p, const char* who) {
  if (!p) return fail(PA_ERR_INVALID, "%s: null plan", who);
  int32_t rc = check_shape(&p->shape, who);
  if (rc) return rc;
  if (p->psize < kTileTokens || p->psize % kTileTokens || p->p_max < 1 || p->grid < 1 ||
      !(p->scale == p->scale) || p->direct != (p->p_max == 1) || (p->path != 1 && p->path != 2) ||
      (p->fused != 0 && p->fused != 1) || p->part_offset != ws_part_offset(p->shape.B, p->shape.Hkv))
    return fail(PA_ERR_INVALID, "%s: plan was not produced by paged_attn_plan", who);
  if (p->path == 2 && !lds_path_ok(p->shape))
    return fail(PA_ERR_UNSUPPORTED, "%s: plan path 2 (LDS-staged kernel) does not take this shape", who);
  if (p->fused && (p->path != 2 || p->direct || !fused_merge_ok(p->shape, p->p_max)))
    return fail(PA_ERR_INVALID, "%s: a fused plan needs path 2, partitions and the wide merge layout "
                "(set fused = 0 for two launches)", who);
  return PA_OK;
}

uint64_t ws_bytes_for(const pa_shape& s, int p_max, bool direct) {
  uint64_t bytes = ws_part_offset(s.B, s.Hkv);
  if (!direct) bytes += uint64_t(s.B) * s.Hq * p_max * (2u * uint64_t(s.D) + 8u);
  return (bytes + 255) & ~uint64_t(255);
}

}  // namespace

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

void clear_error() { g_err.clear(); }

}  // namespace pa

using namespace pa;

extern "C" const char* pa_last_error(void) { return g_err.c_str(); }

extern "C" int32_t pa_row_bytes(int32_t type, int32_t D) {
  if (D < 1) return fail(PA_ERR_INVALID, "pa_row_bytes: D must be >= 1");
  switch (type) {
    case PA_F16: return 2 * D;
    case PA_Q8_0:
    case PA_Q4_0:
      if (D % 32) return fail(PA_ERR_INVALID, "pa_row_bytes: quantised rows need D %% 32 == 0");
      return (type == PA_Q8_0 ? 34 : 18) * (D / 32);
  }
  return fail(PA_ERR_INVALID, "pa_row_bytes: unknown type %d", type);
}

extern "C" int32_t paged_attn_plan(const pa_shape* shape, int32_t max_seq_len, int64_t total_tokens,
                                   int32_t num_cus, int32_t force_partitions,
                                   int32_t partition_tokens, float scale, pa_plan* plan) {
  const char* who = "paged_attn_plan";
  if (!plan) return fail(PA_ERR_INVALID, "%s: null plan", who);
  int32_t rc = check_shape(shape, who);
  if (rc) return rc;
  const pa_shape& s = *shape;
  const int64_t cap = int64_t(s.max_blocks) * s.block_size;
  if (max_seq_len < 0 || max_seq_len > cap)
    return fail(PA_ERR_INVALID, "%s: max_seq_len %d outside [0, max_blocks*block_size=%lld]", who,
                max_seq_len, (long long)cap);
  if (total_tokens < 0 || force_partitions < 0 || partition_tokens < 0)
    return fail(PA_ERR_INVALID, "%s: negative total_tokens/force_partitions/partition_tokens", who);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "%s: scale is not finite", who);
  if (num_cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return fail(PA_ERR_HIP, "%s: could not query the device's compute-unit count", who);
  }
  if (num_cus < 1) return fail(PA_ERR_INVALID, "%s: num_cus must be >= 1", who);

  const int64_t L = max_seq_len;
  const int64_t rbk = pa_row_bytes(s.k_type, s.D), rbv = pa_row_bytes(s.v_type, s.D);
  const bool lds = lds_path_ok(s);
  // units per (sequence, partition): one per kv head (register kernel) or per
  // quad of kv heads (LDS-staged kernel)
  const int64_t per_bp = lds ? s.Hkv / 4 : s.Hkv;
  const int64_t tok = total_tokens > 0 ? total_tokens : int64_t(s.B) * L;
  int64_t psize;
  if (partition_tokens > 0) {
    psize = round_up(partition_tokens, kTileTokens);
  } else if (force_partitions >= 1) {
    psize = round_up(std::max<int64_t>(1, ceil_div(L, force_partitions)), kTileTokens);
  } else if (lds) {
    // Occupancy-aware partitioning (lucebox PR #555, Summary). The LDS-staged
    // kernel runs two workgroups per compute unit and streams at full rate
    // only when every unit slot is busy, so the batch is cut into about
    // 2*num_cus equal units (at least 64 tokens each: two steps of the ring).
    // The partial results this adds are 2D+8 bytes per query head per
    // partition (binary16 o, fp32 m and l), written once and read once.
    // Sequences of at most 256 tokens stay in one partition: splitting them
    // saves less decode time than the merge launch costs.
    const int64_t units_target = int64_t(num_cus) * 2;
    psize = std::max<int64_t>(64, round_up(std::max<int64_t>(1, ceil_div(tok * per_bp, units_target)),
                                           kTileTokens));
    if (L <= 256) psize = L;
  } else {
    // Register kernel: about four workgroups per compute unit, but never split
    // so finely that partial results (written and read once more by the merge)
    // exceed ~4% of the K/V bytes of a partition.
    const int64_t units_target = int64_t(num_cus) * 4;
    const int64_t per_unit = int64_t(kTileTokens) * kWavesPerUnit;
    const int64_t bal = round_up(std::max<int64_t>(1, ceil_div(tok * per_bp, units_target)), per_unit);
    const double part_bytes = double(s.Hq) * (2.0 * s.D + 8.0) * 2.0;
    const double kv_per_token = double(s.Hkv) * double(rbk + rbv);
    const int64_t floor_tok = round_up(int64_t(std::ceil(part_bytes / (0.04 * kv_per_token))), per_unit);
    psize = std::max(bal, floor_tok);
  }
  if (psize >= L) psize = round_up(std::max<int64_t>(L, 1), kTileTokens);
  if (psize > INT32_MAX - kTileTokens) return fail(PA_ERR_INVALID, "%s: partition size overflows", who);
  const int64_t p_max = std::max<int64_t>(1, ceil_div(L, psize));
  const bool direct = p_max == 1;
  int64_t bp_upper = int64_t(s.B) * p_max;
  if (total_tokens > 0) bp_upper = std::min(bp_upper, ceil_div(total_tokens, psize) + s.B);
  const int64_t units = std::max<int64_t>(1, bp_upper * per_bp);
  // The single launch (fused) is left to the caller: on MI355X the separate
  // merge launch measured faster at every shape tried (the in-launch merge
  // runs at two workgroups per CU and behind its waits, where the merge
  // kernel spreads every slice over the whole GPU at once).
  const bool fused = false;
  const int64_t grid = std::min<int64_t>(units, int64_t(num_cus) * (lds ? 2 : 8));

  std::memset(plan, 0, sizeof *plan);
  plan->shape = s;
  plan->scale = scale == 0.0f ? float(1.0 / std::sqrt(double(s.D))) : scale;
  plan->psize = int32_t(psize);
  plan->p_max = int32_t(p_max);
  plan->max_seq_len = max_seq_len;
  plan->grid = int32_t(grid);
  plan->num_cus = num_cus;
  plan->direct = direct ? 1 : 0;
  plan->path = lds ? 2 : 1;
  plan->fused = fused ? 1 : 0;
  plan->ws_bytes = ws_bytes_for(s, int(p_max), direct);
  plan->part_offset = ws_part_offset(s.B, s.Hkv);
  clear_error();
  return PA_OK;
}

extern "C" int32_t paged_attn_decode(const pa_plan* plan, const float* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_table,
                                     const int32_t* seq_len, void* ws, uint64_t ws_bytes,
                                     float* out, void* stream) {
  const char* who = "paged_attn_decode";
  int32_t rc = check_plan(plan, who);
  if (rc) return rc;
  if (!q || !k_pool || !v_pool || !seq_len || !ws)
    return fail(PA_ERR_INVALID, "%s: null q, k_pool, v_pool, seq_len or ws", who);
  if ((plan->direct || plan->fused) && !out)
    return fail(PA_ERR_INVALID, "%s: direct mode and fused plans need out", who);
  if (ws_bytes < plan->ws_bytes)
    return fail(PA_ERR_INVALID, "%s: workspace of %llu bytes, plan needs %llu", who,
                (unsigned long long)ws_bytes, (unsigned long long)plan->ws_bytes);
  const pa_shape& s = plan->shape;
  DecodeArgs a{};
  a.q = q;
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.table = block_table;
  a.seq_len = seq_len;
  a.out = out;
  a.status = static_cast<uint32_t*>(ws);
  a.work = static_cast<uint32_t*>(ws) + 1;
  a.leave = static_cast<uint32_t*>(ws) + 2;
  a.done = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + kWsHeader);
  a.part_o = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + plan->part_offset);
  a.part_ml = reinterpret_cast<float*>(a.part_o + uint64_t(s.B) * s.Hq * plan->p_max * s.D);
  a.B = s.B; a.Hq = s.Hq; a.Hkv = s.Hkv; a.D = s.D; a.r = s.Hq / s.Hkv;
  a.nblocks = s.nblocks; a.max_blocks = s.max_blocks; a.block_size = s.block_size;
  a.bs_shift = ilog2_exact(s.block_size);
  a.psize = plan->psize; a.p_max = plan->p_max; a.grid = plan->grid;
  a.cap_tokens = int32_t(std::min<int64_t>(int64_t(s.max_blocks) * s.block_size,
                                           int64_t(plan->p_max) * plan->psize));
  a.k_type = s.k_type; a.v_type = s.v_type;
  a.direct = plan->direct;
  a.qscale = float(double(plan->scale) * 1.4426950408889634);   // scale * log2(e)
  a.merge_items = s.B * s.Hq * (s.D / kMergeColsHost);
  a.wait_ticks = 100000000ull;                                   // one second of the 100 MHz clock
  // the LDS-staged kernel's DMA chunks are 16-byte aligned only on aligned
  // pools, and it reads q rows with 16-byte loads
  const bool aligned = ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool) |
                         reinterpret_cast<uintptr_t>(q)) & 15) == 0;
  const bool lds = plan->path == 2 && aligned;
  a.fused = plan->fused && lds ? 1 : 0;
  // a single launch also runs the merge slices: more workgroups, up to the
  // two per CU the units use at most
  if (a.fused) a.grid = int32_t(std::min<int64_t>(int64_t(plan->grid) + a.merge_items, 2ll * plan->num_cus));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = lds ? launch_decode_lds(a, st) : launch_decode_regs(a, st);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  if (plan->fused && !lds) {
    // a fused plan whose pools sent it to the register kernel: merge separately
    MergeArgs m{};
    m.part_o = a.part_o;
    m.part_ml = a.part_ml;
    m.seq_len = seq_len;
    m.out = out;
    m.B = s.B; m.Hq = s.Hq; m.D = s.D; m.psize = plan->psize; m.p_max = plan->p_max;
    m.cap_tokens = a.cap_tokens;
    e = launch_merge(m, st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: merge launch failed: %s", who, hipGetErrorString(e));
  }
  clear_error();
  return PA_OK;
}

extern "C" int32_t paged_attn_merge(const pa_plan* plan, const void* ws, uint64_t ws_bytes,
                                    const int32_t* seq_len, float* out, void* stream) {
  const char* who = "paged_attn_merge";
  int32_t rc = check_plan(plan, who);
  if (rc) return rc;
  if (plan->direct || plan->fused) { clear_error(); return PA_OK; }   // done by the decode
  if (!ws || !seq_len || !out) return fail(PA_ERR_INVALID, "%s: null ws, seq_len or out", who);
  if (ws_bytes < plan->ws_bytes)
    return fail(PA_ERR_INVALID, "%s: workspace of %llu bytes, plan needs %llu", who,
                (unsigned long long)ws_bytes, (unsigned long long)plan->ws_bytes);
  const pa_shape& s = plan->shape;
  MergeArgs a{};
  a.part_o = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(ws) + plan->part_offset);
  a.part_ml = reinterpret_cast<const float*>(a.part_o + uint64_t(s.B) * s.Hq * plan->p_max * s.D);
  a.seq_len = seq_len;
  a.out = out;
  a.B = s.B; a.Hq = s.Hq; a.D = s.D; a.psize = plan->psize; a.p_max = plan->p_max;
  a.cap_tokens = int32_t(std::min<int64_t>(int64_t(s.max_blocks) * s.block_size,
                                           int64_t(plan->p_max) * plan->psize));
  hipError_t e = launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  clear_error();
  return PA_OK;
}

extern "C" int32_t paged_attn_step(const pa_plan* plan, const float* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_table,
                                   const int32_t* seq_len, void* ws, uint64_t ws_bytes, float* out,
                                   void* stream) {
  if (!out) return fail(PA_ERR_INVALID, "paged_attn_step: null out");
  int32_t rc = paged_attn_decode(plan, q, k_pool, v_pool, block_table, seq_len, ws, ws_bytes, out, stream);
  if (rc) return rc;
  return paged_attn_merge(plan, ws, ws_bytes, seq_len, out, stream);
}

extern "C" int32_t paged_attn_step_noalloc(const pa_plan* plan, const float* q, const void* k_pool,
                                           const void* v_pool, const int32_t* block_table,
                                           const int32_t* seq_len, float* out, void* stream) {
  const char* who = "paged_attn_step_noalloc";
  int32_t rc = check_plan(plan, who);
  if (rc) return rc;
  // the single launch needs its counters at zero when it starts; in the
  // shared scratch a two-launch plan of a smaller batch writes partials where
  // a fused plan's counters lie, so no call here can promise that
  if (plan->fused)
    return fail(PA_ERR_INVALID, "%s: a fused plan needs counters that start at zero, which the shared static "
                "scratch does not keep (set fused = 0, or use paged_attn_step with a workspace)", who);
  if (plan->ws_bytes > kNoAllocScratchBytes)
    return fail(PA_ERR_INVALID, "%s: the plan needs %llu bytes of workspace, the static scratch holds %llu",
                who, (unsigned long long)plan->ws_bytes, (unsigned long long)kNoAllocScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = noalloc_scratch(&scratch);
  if (e != hipSuccess)
    return fail(PA_ERR_HIP, "%s: no address for the static scratch: %s", who, hipGetErrorString(e));
  return paged_attn_step(plan, q, k_pool, v_pool, block_table, seq_len, scratch, kNoAllocScratchBytes, out,
                         stream);
}

extern "C" int32_t paged_kv_gather(const pa_plan* plan, const void* pool, int32_t which,
                                   const int32_t* block_table, int32_t b, int32_t t0, int32_t n,
                                   void* dst, void* ws, void* stream) {
  const char* who = "paged_kv_gather";
  int32_t rc = check_plan(plan, who);
  if (rc) return rc;
  const pa_shape& s = plan->shape;
  if (!pool || (n > 0 && !dst)) return fail(PA_ERR_INVALID, "%s: null pool or dst", who);
  if (which != 0 && which != 1) return fail(PA_ERR_INVALID, "%s: which must be 0 (K) or 1 (V)", who);
  if (b < 0 || b >= s.B) return fail(PA_ERR_INVALID, "%s: sequence %d outside [0, B)", who, b);
  if (t0 < 0 || n < 0 || int64_t(t0) + n > int64_t(s.max_blocks) * s.block_size)
    return fail(PA_ERR_INVALID, "%s: tokens [%d, %d+%d) outside the table", who, t0, t0, n);
  GatherArgs a{};
  a.pool = static_cast<const uint8_t*>(pool);
  a.table = block_table;
  a.dst = static_cast<uint8_t*>(dst);
  a.status = static_cast<uint32_t*>(ws);
  a.b = b; a.t0 = t0; a.n = n;
  a.Hkv = s.Hkv;
  a.row_bytes = pa_row_bytes(which == 0 ? s.k_type : s.v_type, s.D);
  a.nblocks = s.nblocks; a.max_blocks = s.max_blocks; a.block_size = s.block_size;
  a.bs_shift = ilog2_exact(s.block_size);
  hipError_t e = launch_gather(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  clear_error();
  return PA_OK;
}

extern "C" int32_t paged_attn_status(void* ws, void* stream, uint32_t* flags) {
  const char* who = "paged_attn_status";
  if (!ws || !flags) return fail(PA_ERR_INVALID, "%s: null ws or flags", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ws, sizeof v, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemsetAsync(ws, 0, sizeof v, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
  *flags = v;
  clear_error();
  return PA_OK;
}

extern "C" int32_t paged_table_update(int32_t* table, int32_t* seq_len, int32_t B, int32_t max_blocks,
                                      const int32_t* updates, int32_t n, void* stream) {
  const char* who = "paged_table_update";
  if (n < 0 || B < 1 || max_blocks < 1)
    return fail(PA_ERR_INVALID, "%s: n < 0, B < 1 or max_blocks < 1", who);
  if (n == 0) { clear_error(); return PA_OK; }
  if (!table || !seq_len || !updates) return fail(PA_ERR_INVALID, "%s: null table, seq_len or updates", who);
  // every entry named once: sort the flat targets (seq_len[b] as -1 - b)
  std::vector<int64_t> targets(static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = updates[3 * i], slot = updates[3 * i + 1];
    if (b < 0 || b >= B || slot < -1 || slot >= max_blocks)
      return fail(PA_ERR_INVALID, "%s: update %d names (b=%d, slot=%d) outside B=%d, max_blocks=%d", who, i,
                  b, slot, B, max_blocks);
    targets[size_t(i)] = slot < 0 ? -1 - int64_t(b) : int64_t(b) * max_blocks + slot;
  }
  std::sort(targets.begin(), targets.end());
  if (std::adjacent_find(targets.begin(), targets.end()) != targets.end())
    return fail(PA_ERR_INVALID, "%s: two updates name the same entry", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t i0 = 0; i0 < n; i0 += kTableUpdates) {
    TableUpdateArgs a;
    a.table = table;
    a.seq_len = seq_len;
    a.max_blocks = max_blocks;
    a.n = std::min(kTableUpdates, n - i0);
    std::memcpy(a.upd, updates + 3 * int64_t(i0), sizeof(int32_t) * 3 * size_t(a.n));
    hipError_t e = launch_table_update(a, st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  }
  clear_error();
  return PA_OK;
}

extern "C" int32_t paged_kv_copy_blocks(void* pool, uint64_t block_bytes, int32_t nblocks,
                                        const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                                        void* stream) {
  const char* who = "paged_kv_copy_blocks";
  if (n < 0 || nblocks < 0) return fail(PA_ERR_INVALID, "%s: n < 0 or nblocks < 0", who);
  if (n == 0) { clear_error(); return PA_OK; }
  if (!pool || !src_ids || !dst_ids) return fail(PA_ERR_INVALID, "%s: null pool, src_ids or dst_ids", who);
  if (block_bytes == 0 || block_bytes % 16 || (reinterpret_cast<uintptr_t>(pool) & 15))
    return fail(PA_ERR_INVALID, "%s: block_bytes must be a positive multiple of 16 and the pool 16-byte aligned",
                who);
  std::vector<int32_t> srcs(src_ids, src_ids + n), dsts(dst_ids, dst_ids + n);
  for (int32_t i = 0; i < n; ++i)
    if (srcs[size_t(i)] < 0 || srcs[size_t(i)] >= nblocks || dsts[size_t(i)] < 0 || dsts[size_t(i)] >= nblocks)
      return fail(PA_ERR_INVALID, "%s: pair %d (%d -> %d) outside [0, %d)", who, i, srcs[size_t(i)],
                  dsts[size_t(i)], nblocks);
  std::sort(srcs.begin(), srcs.end());
  std::vector<int32_t> sorted_dst = dsts;
  std::sort(sorted_dst.begin(), sorted_dst.end());
  if (std::adjacent_find(sorted_dst.begin(), sorted_dst.end()) != sorted_dst.end())
    return fail(PA_ERR_INVALID, "%s: a destination block is named twice", who);
  for (int32_t d : sorted_dst)
    if (std::binary_search(srcs.begin(), srcs.end(), d))
      return fail(PA_ERR_INVALID, "%s: block %d is both a source and a destination", who, d);
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t i0 = 0; i0 < n; i0 += kCopyPairs) {
    CopyBlocksArgs a;
    a.pool = static_cast<uint8_t*>(pool);
    a.block_bytes = block_bytes;
    a.n = std::min(kCopyPairs, n - i0);
    std::memcpy(a.src, src_ids + i0, sizeof(int32_t) * size_t(a.n));
    std::memcpy(a.dst, dst_ids + i0, sizeof(int32_t) * size_t(a.n));
    hipError_t e = launch_copy_blocks(a, st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  }
  clear_error();
  return PA_OK;
}

namespace {
uint64_t chunk_ws_bytes(const pa_shape& s, int tq, int p_max, bool direct) {
  uint64_t bytes = ws_part_offset(s.B, s.Hkv);
  if (!direct) bytes += uint64_t(s.B) * uint64_t(tq) * s.Hq * p_max * (2u * uint64_t(s.D) + 8u);
  return (bytes + 255) & ~uint64_t(255);
}

int32_t check_chunk_plan(const pa_chunk_plan* p, const char* who) {
  if (!p) return fail(PA_ERR_INVALID, "%s: null plan", who);
  int32_t rc = check_shape(&p->shape, who);
  if (rc) return rc;
  if (p->tq < 1 || p->tq > kMaxChunk || p->psize < kTileTokens || p->psize % kTileTokens ||
      p->p_max < 1 || p->grid < 1 || !(p->scale == p->scale) || p->direct != (p->p_max == 1) ||
      p->path < 1 || p->path > 3 || p->part_offset != ws_part_offset(p->shape.B, p->shape.Hkv))
    return fail(PA_ERR_INVALID, "%s: plan was not produced by paged_attn_chunk_plan", who);
  const pa_shape& s = p->shape;
  if (p->path == 2 && !chunk_window_ok(int64_t(p->tq) * (s.Hq / s.Hkv), s.Hkv, s.k_type, s.v_type, s.D))
    return fail(PA_ERR_UNSUPPORTED, "%s: plan path 2 (window kernel) does not take this chunk", who);
  return PA_OK;
}
}  // namespace

extern "C" int32_t paged_attn_chunk_plan(const pa_shape* shape, int32_t tq, int32_t max_seq_len,
                                         int64_t total_tokens, int32_t num_cus, int32_t force_partitions,
                                         int32_t partition_tokens, float scale, pa_chunk_plan* plan) {
  const char* who = "paged_attn_chunk_plan";
  if (!plan) return fail(PA_ERR_INVALID, "%s: null plan", who);
  int32_t rc = check_shape(shape, who);
  if (rc) return rc;
  const pa_shape& s = *shape;
  if (tq < 1 || tq > kMaxChunk) return fail(PA_ERR_INVALID, "%s: tq %d outside [1, %d]", who, tq, kMaxChunk);
  const int64_t cap = int64_t(s.max_blocks) * s.block_size;
  if (max_seq_len < 0 || max_seq_len > cap)
    return fail(PA_ERR_INVALID, "%s: max_seq_len %d outside [0, max_blocks*block_size=%lld]", who,
                max_seq_len, (long long)cap);
  if (total_tokens < 0 || force_partitions < 0 || partition_tokens < 0)
    return fail(PA_ERR_INVALID, "%s: negative total_tokens/force_partitions/partition_tokens", who);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "%s: scale is not finite", who);
  if (num_cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return fail(PA_ERR_HIP, "%s: could not query the device's compute-unit count", who);
  }
  if (num_cus < 1) return fail(PA_ERR_INVALID, "%s: num_cus must be >= 1", who);
  const int64_t L = max_seq_len;
  const int64_t r = s.Hq / s.Hkv;
  const bool window = chunk_window_ok(int64_t(tq) * r, s.Hkv, s.k_type, s.v_type, s.D);
  const int nt = chunk_wave_tiles(int64_t(tq) * r, s.D);
  const int nq = int(ceil_div(int64_t(tq) * r, 16));
  const int64_t tok = total_tokens > 0 ? total_tokens : int64_t(s.B) * L;
  // Partition size for units of qt row blocks of heads_per_unit kv heads,
  // wgs_per_cu workgroups per compute unit.
  auto size_partitions = [&](int64_t qt, int64_t heads_per_unit, int wgs_per_cu) {
    if (partition_tokens > 0) return round_up(partition_tokens, kTileTokens);
    if (force_partitions >= 1) return round_up(std::max<int64_t>(1, ceil_div(L, force_partitions)), kTileTokens);
    // Occupancy-aware partitioning (lucebox PR #555, Summary), counting the
    // workgroups a compute unit holds. Partials cost 2D+8 bytes per query row
    // and partition, written and read once; a partition is never so short
    // that this exceeds a quarter of what it saves, i.e. a quarter of the K/V
    // bytes it streams (memory-bound chunks) or of the HBM time equal to its
    // MFMA work at the machine's flop:byte ratio (compute-bound chunks,
    // 4*D flops per query row and key), whichever floor is lower.
    // Among the sizes above that floor, take the one that finishes soonest:
    // the units run in ceil(units / slots) rounds of psize keys each (a
    // round only partly filled costs as much as a full one).
    const int64_t slots = int64_t(num_cus) * wgs_per_cu;
    const int64_t rbk = pa_row_bytes(s.k_type, s.D), rbv = pa_row_bytes(s.v_type, s.D);
    const double part = double(tq) * s.Hq * (2.0 * s.D + 8.0) * 2.0;
    const double floor_hbm = part / (0.25 * double(s.Hkv) * double(rbk + rbv));
    const double floor_mfma = part * kFlopsPerByte / (0.25 * double(tq) * s.Hq * 4.0 * s.D);
    const int64_t floor_tok = std::max<int64_t>(
        round_up(int64_t(std::ceil(std::min(floor_hbm, floor_mfma))), kTileTokens), 128);
    int64_t ps_best = round_up(std::max<int64_t>(L, 1), kTileTokens);
    int64_t best = -1;
    for (int64_t parts = 1; parts <= 64; ++parts) {
      const int64_t ps = round_up(std::max<int64_t>(1, ceil_div(L, parts)), kTileTokens);
      if (ps < floor_tok && parts > 1) break;
      const int64_t bp = std::min<int64_t>(int64_t(s.B) * ceil_div(std::max<int64_t>(L, 1), ps),
                                           ceil_div(tok, ps) + s.B);
      const int64_t cost = ceil_div(std::max<int64_t>(1, bp * (s.Hkv / heads_per_unit) * qt), slots) * ps;
      if (best < 0 || cost < best) { best = cost; ps_best = ps; }
    }
    return ps_best;
  };
  // The wide-tile kernel takes chunks of more than 64 query rows per kv head:
  // in its paired form always (measured 0.63-0.95x the tile kernel's time
  // over B=8 x 32K chunks of 72-192 rows and 32-512-token chunks over 8K).
  // In its four-wave form (F16 K and V at D = 256, F16 with Q8_0) it does
  // where its units fill at least half the compute units (one workgroup
  // each; F16/F16: 0.86-0.95x over 72-192 rows at B=8 x 32K and 128-512
  // tokens over 8K); with fewer the tile kernel, two per compute unit, was
  // measured faster (a 64-token chunk over 8K in 72 units: 80 against 78 us).
  const int64_t rows = int64_t(tq) * r;
  bool wide = !window && chunk_wide_pick(rows, s.D);
  int64_t psize = 0;
  if (wide) {
    const int64_t qt_w = ceil_div(rows, int64_t(kWideRows));
    psize = size_partitions(qt_w, 1, 1);
    if (!chunk_wide_paired(s.k_type, s.v_type, s.D)) {
      const int64_t units_w =
          int64_t(s.B) * std::max<int64_t>(1, ceil_div(std::max<int64_t>(L, 1), psize)) * s.Hkv * qt_w;
      if (2 * units_w < num_cus) wide = false;
    }
  }
  // the window kernel takes short chunks (a workgroup per kv-head quad, two
  // per CU for at most 16 query rows per kv head, else one; with the head
  // dimension split, a workgroup per kv-head pair, two per CU); the wide-tile
  // kernel long ones (a workgroup per kv head and 128 query rows, one per
  // CU); the tile-conversion kernel the rest (a workgroup per kv head and
  // 64*nt query rows, one or two per CU)
  const int64_t block_rows = wide ? kWideRows : 64 * nt;
  const int64_t qt = window ? 1 : (rows + block_rows - 1) / block_rows;   // row blocks per unit
  const int64_t heads_per_unit = window ? chunk_window_heads(nq, s.D) : 1;
  const int wgs_per_cu = window ? chunk_window_wgs_per_cu(nq, s.D, s.k_type, s.v_type)
                                : (wide ? 1 : chunk_wgs_per_cu(nt, s.k_type, s.v_type, s.D));
  if (!wide) psize = size_partitions(qt, heads_per_unit, wgs_per_cu);
  if (psize >= L) psize = round_up(std::max<int64_t>(L, 1), kTileTokens);
  if (psize > INT32_MAX - kTileTokens) return fail(PA_ERR_INVALID, "%s: partition size overflows", who);
  const int64_t p_max = std::max<int64_t>(1, ceil_div(L, psize));
  const bool direct = p_max == 1;
  const int64_t units = std::max<int64_t>(1, int64_t(s.B) * p_max * (s.Hkv / heads_per_unit) * qt);
  const int64_t grid = std::min<int64_t>(units, int64_t(num_cus) * wgs_per_cu);
  const uint64_t ws = chunk_ws_bytes(s, tq, int(p_max), direct);
  std::memset(plan, 0, sizeof *plan);
  plan->shape = s;
  plan->tq = tq;
  plan->scale = scale == 0.0f ? float(1.0 / std::sqrt(double(s.D))) : scale;
  plan->psize = int32_t(psize);
  plan->p_max = int32_t(p_max);
  plan->max_seq_len = max_seq_len;
  plan->grid = int32_t(grid);
  plan->num_cus = num_cus;
  plan->direct = direct ? 1 : 0;
  plan->path = window ? 2 : (wide ? 3 : 1);
  plan->ws_bytes = ws;
  plan->part_offset = ws_part_offset(s.B, s.Hkv);
  clear_error();
  return PA_OK;
}

extern "C" int32_t paged_attn_chunk(const pa_chunk_plan* plan, const float* q, const void* k_pool,
                                    const void* v_pool, const int32_t* block_table, const int32_t* seq_len,
                                    void* ws, uint64_t ws_bytes, float* out, void* stream) {
  const char* who = "paged_attn_chunk";
  int32_t rc = check_chunk_plan(plan, who);
  if (rc) return rc;
  if (!q || !k_pool || !v_pool || !seq_len || !ws || !out)
    return fail(PA_ERR_INVALID, "%s: null q, k_pool, v_pool, seq_len, ws or out", who);
  if (ws_bytes < plan->ws_bytes)
    return fail(PA_ERR_INVALID, "%s: workspace of %llu bytes, plan needs %llu", who,
                (unsigned long long)ws_bytes, (unsigned long long)plan->ws_bytes);
  const pa_shape& s = plan->shape;
  const uint64_t rows = uint64_t(s.B) * uint64_t(plan->tq) * s.Hq;
  ChunkArgs a{};
  a.q = q;
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.table = block_table;
  a.seq_len = seq_len;
  a.out = out;
  a.status = static_cast<uint32_t*>(ws);
  a.part_o = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + plan->part_offset);
  a.part_ml = reinterpret_cast<float*>(a.part_o + rows * plan->p_max * s.D);
  a.B = s.B; a.Tq = plan->tq; a.Hq = s.Hq; a.Hkv = s.Hkv; a.D = s.D; a.r = s.Hq / s.Hkv;
  a.nblocks = s.nblocks; a.max_blocks = s.max_blocks;
  a.bs_shift = ilog2_exact(s.block_size);
  a.psize = plan->psize; a.p_max = plan->p_max; a.grid = plan->grid;
  a.cap_tokens = int32_t(std::min<int64_t>(int64_t(s.max_blocks) * s.block_size,
                                           int64_t(plan->p_max) * plan->psize));
  a.k_type = s.k_type; a.v_type = s.v_type;
  a.direct = plan->direct;
  a.qscale = float(double(plan->scale) * 1.4426950408889634);
  a.nt = chunk_wave_tiles(int64_t(plan->tq) * a.r, s.D);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the window kernel's DMA chunks are 16-byte aligned only on aligned
  // pools, the window and wide-tile kernels read q rows with 16-byte loads,
  // and the wide-tile kernel writes partial rows with 16-byte stores;
  // otherwise the tile kernel runs
  const bool aligned = ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool) |
                         reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(ws)) & 15) == 0;
  hipError_t e = !aligned || plan->path == 1 ? launch_chunk(a, st)
                 : plan->path == 2         ? launch_chunk_lds(a, st)
                                           : launch_chunk_wide(a, st);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  if (!plan->direct) {
    MergeArgs mg{};
    mg.part_o = a.part_o;
    mg.part_ml = a.part_ml;
    mg.seq_len = seq_len;
    mg.out = out;
    mg.B = s.B; mg.Hq = plan->tq * s.Hq; mg.D = s.D; mg.psize = plan->psize; mg.p_max = plan->p_max;
    mg.cap_tokens = a.cap_tokens;
    mg.min_len = plan->tq;
    e = launch_merge(mg, st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: merge launch failed: %s", who, hipGetErrorString(e));
  }
  clear_error();
  return PA_OK;
}
