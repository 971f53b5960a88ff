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
  float* part_o;           // [B][Hq][p_max][D]
  float* part_ml;          // [B][Hq][p_max][2]
  uint32_t* status;
  int32_t B, Hq, Hkv, D, r;
  int32_t nblocks, max_blocks, block_size, bs_shift;
  int32_t psize, p_max, grid;
  int32_t cap_tokens;      // longest admissible seq_len: min(max_blocks*bs, p_max*psize)
  int32_t k_type, v_type;
  int32_t direct;
  float qscale;            // scale * log2(e)
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

struct MergeArgs {
  const float* part_o;
  const float* part_ml;
  const int32_t* seq_len;
  float* out;
  int32_t B, Hq, D, psize, p_max, cap_tokens;
};

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

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
