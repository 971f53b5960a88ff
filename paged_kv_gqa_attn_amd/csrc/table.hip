// Paging metadata and block maintenance on the device.
//
//   * copy_blocks_kernel: whole-block copies inside one pool, the device half
//     of copy-on-write (lucebox PR #555, Roadmap item 6: prefix blocks shared
//     under reference counts and copied on write). An allocation that is about
//     to write into a block it shares receives a fresh block id from the
//     allocator; the shared block's bytes are copied there first.
//   * table_update_kernel: scatters a few (sequence, slot, value) entries
//     into the device-resident block table and seq_len (lucebox PR #555,
//     Summary: the table and lengths live on the device beside the pool, so
//     a step sends only the ids of newly allocated blocks).
//
// Both take their short lists by value in the kernel arguments: the host
// validated them, nothing is allocated or copied beforehand, and the call
// can be captured into a graph.
#include "pa_device.h"
#include "pa_host.h"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyChunk = kCopyThreads * 16;   // bytes per workgroup

__global__ void __launch_bounds__(kCopyThreads) copy_blocks_kernel(const CopyBlocksArgs a) {
  const int pair = blockIdx.y;
  const uint64_t off = uint64_t(blockIdx.x) * kCopyChunk + uint64_t(threadIdx.x) * 16u;
  if (pair >= a.n || off >= a.block_bytes) return;
  const uint4* src = reinterpret_cast<const uint4*>(a.pool + uint64_t(a.src[pair]) * a.block_bytes + off);
  uint4* dst = reinterpret_cast<uint4*>(a.pool + uint64_t(a.dst[pair]) * a.block_bytes + off);
  *dst = *src;
}

__global__ void __launch_bounds__(kTableUpdates) table_update_kernel(const TableUpdateArgs a) {
  const int i = threadIdx.x;
  if (i >= a.n) return;
  const int32_t b = a.upd[3 * i], slot = a.upd[3 * i + 1], v = a.upd[3 * i + 2];
  if (slot < 0)
    a.seq_len[b] = v;
  else
    a.table[int64_t(b) * a.max_blocks + slot] = v;
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.n < 1 || a.n > kCopyPairs || a.block_bytes % 16) return hipErrorInvalidValue;
  const uint64_t chunks = (a.block_bytes + kCopyChunk - 1) / kCopyChunk;
  if (chunks > 0x7fffffffull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(chunks), unsigned(a.n)), dim3(kCopyThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_table_update(const TableUpdateArgs& a, hipStream_t stream) {
  if (a.n < 1 || a.n > kTableUpdates) return hipErrorInvalidValue;
  hipLaunchKernelGGL(table_update_kernel, dim3(1), dim3(kTableUpdates), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
