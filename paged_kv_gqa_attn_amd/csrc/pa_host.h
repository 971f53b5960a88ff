// Host-side internals shared by the C-ABI translation units: error reporting
// and the launchers each kernel file exports.
#pragma once
#include <cstdint>

#include <hip/hip_runtime.h>

#include "../../include/paged_attn.h"

namespace pa {

// Records a message for pa_last_error() on this thread and returns code.
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Arguments of one decode launch, already validated on the host.
struct DecodeArgs {
  const float* q;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* table;    // nullptr = contiguous layout
  const int32_t* seq_len;
  float* out;              // direct mode
  uint16_t* part_o;        // [B][Hq][p_max][D] binary16 bits
  float* part_ml;          // [B][Hq][p_max][2]
  uint32_t* status;
  int32_t B, Hq, Hkv, D, r;
  int32_t nblocks, max_blocks, block_size, bs_shift;
  int32_t psize, p_max, grid;
  int32_t cap_tokens;      // longest admissible seq_len: min(max_blocks*bs, p_max*psize)
  int32_t k_type, v_type;
  int32_t direct;
  float qscale;            // scale * log2(e)
  int32_t ring_bytes;      // LDS-staged kernel: bytes of the K/V ring (set by its launcher)
  // single-launch merge (LDS-staged kernel, fused == 1): items are claimed from
  // *work (decode units first, then merge_items slices of 64 output columns),
  // done[b*ceil(Hkv/4) + hg] counts finished partitions, *leave the
  // workgroups that have left; the last one to leave zeroes all three
  uint32_t* work;
  uint32_t* leave;
  uint32_t* done;
  int32_t fused;
  int32_t merge_items;
  uint64_t wait_ticks;     // longest wait of a merge slice, 100 MHz constant-clock ticks
};

// Workspace header: status word, then the single-launch counters; done[]
// from byte kWsHeader, one counter every kDoneStride words (4 KB + 64 B, so
// that every counter sits in its own memory line and channel: the waiting
// merge slices poll them, and a line polled by hundreds of workgroups slows
// the K/V stream through its channel), partials from ws_part_offset().
constexpr uint64_t kWsHeader = 256;
constexpr int kDoneStride = 1040;
constexpr uint64_t ws_part_offset(int32_t B, int32_t Hkv) {
  return kWsHeader + ((4ull * kDoneStride * uint64_t(B) * uint64_t((Hkv + 3) / 4) + 255) & ~255ull);
}

// Decode kernels: register streaming (any supported shape) and LDS staged
// (the shapes lds_groups() admits, Hkv % 4 == 0, B <= kLdsMaxB, pools
// 16-byte aligned).
hipError_t launch_decode_regs(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_lds(const DecodeArgs& a, hipStream_t stream);

// Geometry of the LDS-staged kernel, shared by the planner and the kernel.
// One step stages, for the four kv heads of a workgroup, G groups of 16
// token slots of K and of V (one 16-byte DMA chunk per lane, 1 KB per
// instruction) into one slot of a ring of R slots that shares kLdsRingBytes
// of LDS (two workgroups per compute unit); R-1 steps are in flight while one
// is computed.
constexpr int kLdsRingBytes = 73728;
constexpr int kLdsPreferGroups = 2;
constexpr int kLdsMaxSlots = 4;
constexpr int kLdsMaxB = 256;
constexpr int lds_row_bytes(int type, int D) {
  return type == PA_F16 ? 2 * D : (type == PA_Q8_0 ? 34 * (D / 32) : 18 * (D / 32));
}
// 1 KB DMA instructions that stage 16 slots x 4 heads of one side.
constexpr int lds_dma_per_group(int type, int D) { return (16 * 4 * lds_row_bytes(type, D) + 1023) / 1024; }
constexpr int lds_slot_bytes(int kt, int vt, int D, int G) {
  return G * 1024 * (lds_dma_per_group(kt, D) + lds_dma_per_group(vt, D));
}
// 16-slot groups per step (kLdsPreferGroups, else 1), or 0 when not even a
// two-slot ring of one group fits.
constexpr int lds_groups(int kt, int vt, int D) {
  return 2 * lds_slot_bytes(kt, vt, D, kLdsPreferGroups) <= kLdsRingBytes ? kLdsPreferGroups
         : (2 * lds_slot_bytes(kt, vt, D, 1) <= kLdsRingBytes ? 1 : 0);
}
constexpr int lds_ring_slots(int kt, int vt, int D) {
  return lds_groups(kt, vt, D) == 0
             ? 0
             : (kLdsRingBytes / lds_slot_bytes(kt, vt, D, lds_groups(kt, vt, D)) > kLdsMaxSlots
                    ? kLdsMaxSlots
                    : kLdsRingBytes / lds_slot_bytes(kt, vt, D, lds_groups(kt, vt, D)));
}
// The decode kernel also takes rows too large for a 16-slot group (an F16
// side at D = 256: 32 KB of K or V per group of four heads): its steps are
// then one group of 8 slots, still computed as 16-row MFMA tiles whose last
// 8 rows are masked. 1 KB DMA instructions for GS slots x 4 heads of a side:
constexpr int lds_dma_per_slots(int type, int D, int GS, int NH = 4) {
  return (GS * NH * lds_row_bytes(type, D) + 1023) / 1024;
}
// Slots per group of the decode kernel: 16 where lds_groups() admits the
// shape, else 8 when a two-slot ring of 8-slot steps fits, else 0.
constexpr int decode_group_slots(int kt, int vt, int D) {
  return lds_groups(kt, vt, D) > 0 ? 16
         : (2 * 1024 * (lds_dma_per_slots(kt, D, 8) + lds_dma_per_slots(vt, D, 8)) <= kLdsRingBytes ? 8 : 0);
}

// Arguments of one chunk launch (multi-token queries), validated on the host.
struct ChunkArgs {
  const float* q;          // [B][Tq][Hq][D]
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* table;    // nullptr = contiguous layout
  const int32_t* seq_len;
  float* out;              // [B][Tq][Hq][D], direct mode
  uint16_t* part_o;        // [B][Tq*Hq][p_max][D] binary16 bits
  float* part_ml;          // [B][Tq*Hq][p_max][2]
  uint32_t* status;
  int32_t B, Tq, Hq, Hkv, D, r;
  int32_t nblocks, max_blocks, bs_shift;
  int32_t psize, p_max, grid;
  int32_t cap_tokens;
  int32_t k_type, v_type;
  int32_t direct;
  float qscale;            // scale * log2(e)
  int32_t nt;              // 16-row query tiles per wave (chunk_wave_tiles)
};
// Waves per kv head of the window kernel with NQ column groups of 16 query
// rows: 2 (each half of the head dimension) for two or three column groups
// at D = 256, else 1.
constexpr int chunk_window_split(int nq, int D) { return nq >= 2 && D == 256 ? 2 : 1; }
// kv heads per workgroup of the window kernel: a pair with two waves per
// head, else a quad.
constexpr int chunk_window_heads(int nq, int D) { return chunk_window_split(nq, D) == 2 ? 2 : 4; }
// Workgroups per CU of the window kernel: two when one column group fits
// (the decode kernel's register and LDS budget), when the head dimension is
// split, and for two or three groups at D = 128 where K or V is quantised:
// two groups fit the registers twice, three spill 2-53 registers at two per
// CU and still measured 20-45% faster than one, except Q4_0 K with Q8_0 V
// (97 spilled, 16-18% slower), which keeps one; F16/F16, HBM-bound either
// way, keeps the larger ring of one per CU. Else one.
constexpr int chunk_window_wgs_per_cu(int nq, int D, int kt, int vt) {
  const bool d128_twice = D == 128 && (nq == 2 || nq == 3) && !(kt == PA_F16 && vt == PA_F16) &&
                          !(nq == 3 && kt == PA_Q4_0 && vt == PA_Q8_0);
  return nq == 1 || d128_twice || chunk_window_split(nq, D) == 2 ? 2 : 1;
}
// Whether the window kernel takes a chunk with `rows` query rows per kv head
// (pools aside): Hkv % 4 == 0, the shapes lds_groups() admits, and up to 48
// rows (three column groups; at D = 256 over half of the head dimension per
// wave), except that at D = 256 33..48 rows go to the window kernel only for
// Q4_0 K and V, whose pair ring holds steps of two 16-slot groups: with a
// Q8_0 side the steps are single groups and the tile kernel measured as
// fast or faster (B=8 x 32K, Tq=8 at r=6: Q4_0 120 against 140 us, Q8_0 /
// Q4_0 147 against 148, Q4_0 / Q8_0 149 against 146).
constexpr bool chunk_window_ok(int64_t rows, int hkv, int kt, int vt, int D) {
  return (D == 128 || D == 256) && hkv % 4 == 0 && lds_groups(kt, vt, D) > 0 &&
         (rows <= 32 || (rows <= 48 && (D == 128 || (kt == PA_Q4_0 && vt == PA_Q4_0))));
}
hipError_t launch_chunk(const ChunkArgs& a, hipStream_t stream);
// The window kernel (chunk_lds.hip): the decode kernel's LDS ring, each wave
// one kv head with all of its Tq*r query rows (chunk_window_ok); pools
// 16-byte aligned.
hipError_t launch_chunk_lds(const ChunkArgs& a, hipStream_t stream);
// The wide-tile kernel (chunk_wide.hip): 32x32 MFMA tiles, a workgroup per
// kv head and 128 query rows, one per CU (prefill chunks); 16-byte aligned
// pools and q.
hipError_t launch_chunk_wide(const ChunkArgs& a, hipStream_t stream);
constexpr int kWideRows = 128;
// Whether the plan picks the wide-tile kernel for a chunk with `rows` query
// rows per kv head that the window kernel does not take: from 65 rows on,
// where the tile kernel needs a second 64-row block.
constexpr bool chunk_wide_pick(int64_t rows, int D) { return (D == 128 || D == 256) && rows > 64; }
// Query tiles per wave of the chunk kernel for R = Tq*r rows per kv head (a
// workgroup of four waves takes 64*nt rows; two tiles per wave fit the
// registers at D = 128 only), and its workgroups per CU (two waves per SIMD
// at nt = 1, one otherwise).
constexpr int chunk_wave_tiles(int64_t rows, int D) { return rows > 64 && D == 128 ? 2 : 1; }
constexpr int chunk_wgs_per_cu(int nt, int /*kt*/, int /*vt*/, int /*D*/) { return nt == 1 ? 2 : 1; }

// Whole-block copies inside one pool (copy-on-write); up to kCopyPairs pairs
// per launch travel in the kernel arguments.
constexpr int kCopyPairs = 64;
struct CopyBlocksArgs {
  uint8_t* pool;
  uint64_t block_bytes;    // multiple of 16; pool 16-byte aligned
  int32_t n;
  int32_t src[kCopyPairs];
  int32_t dst[kCopyPairs];
};
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

// Block-table / seq_len scatter; up to kTableUpdates (b, slot, value) triples
// per launch travel in the kernel arguments (slot < 0: seq_len[b] = value).
constexpr int kTableUpdates = 256;
struct TableUpdateArgs {
  int32_t* table;
  int32_t* seq_len;
  int32_t max_blocks;
  int32_t n;
  int32_t upd[3 * kTableUpdates];
};
hipError_t launch_table_update(const TableUpdateArgs& a, hipStream_t stream);

struct MergeArgs {
  const uint16_t* part_o;  // binary16 bits
  const float* part_ml;
  const int32_t* seq_len;
  float* out;
  int32_t B, Hq, D, psize, p_max, cap_tokens;
  int32_t min_len;         // 0 < seq_len < min_len counts as empty (chunks: Tq)
};

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
// Output columns of one slice of the wide merge layout (merge_common.h).
constexpr int kMergeColsHost = 64;
// Whether launch_merge takes the row-per-thread layout (many rows of few
// partitions: at most 16 over 1024+ rows or 32 over 512+) rather than the
// wide one (one workgroup per row and 64 columns, merge_common.h).
constexpr bool merge_rows_layout(int64_t rows, int p_max) {
  return (p_max <= 16 && rows >= 1024) || (p_max <= 32 && rows >= 512);
}

// Workspace of paged_attn_step_noalloc: a file-scope device array of this
// many bytes per GPU (step_noalloc.hip). noalloc_scratch returns its device
// address on the current device (looked up once per device).
constexpr uint64_t kNoAllocScratchBytes = 64ull << 20;
hipError_t noalloc_scratch(void** addr);

struct GatherArgs {
  const uint8_t* pool;
  const int32_t* table;    // nullptr = contiguous layout
  uint8_t* dst;
  uint32_t* status;        // may be null
  int32_t b, t0, n;
  int32_t Hkv, row_bytes, nblocks, max_blocks, block_size, bs_shift;
};

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);

}  // namespace pa
