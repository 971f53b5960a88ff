// Host-only build of libpaged_attn for the sanitizer tests.
//
// The C-ABI translation units (api.cpp, kv_pool.cpp) are compiled with the
// host compiler under AddressSanitizer and UndefinedBehaviorSanitizer and
// linked with this file in place of the HIP kernel sources: every launcher
// refuses, so the planner, the argument checks, the error messages and the
// block allocator run instrumented while no device code exists. A call that
// passes every host check therefore fails with PA_ERR_HIP instead of
// launching anything.
#include "../../paged_kv_gqa_attn_amd/csrc/pa_host.h"

namespace pa {

hipError_t launch_decode_regs(const DecodeArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_decode_lds(const DecodeArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_chunk(const ChunkArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_chunk_lds(const ChunkArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_chunk_wide(const ChunkArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_copy_blocks(const CopyBlocksArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_table_update(const TableUpdateArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_merge(const MergeArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_gather(const GatherArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t noalloc_scratch(void**) { return hipErrorNoBinaryForGpu; }

}  // namespace pa

// Marks this build: tests that drive calls all the way to a launch (with
// pointers that are never dereferenced) run only against a library that
// exports it.
extern "C" int32_t pa_host_only_build(void) { return 1; }
