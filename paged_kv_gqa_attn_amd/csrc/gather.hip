// Raw row gather through the block table: the indexing probe of the decode
// path. It resolves block ids and forms the 64-bit row address with the same
// helpers as the decode kernel (pa_device.h) and copies the encoded bytes, so
// a bit-exact comparison against a host gather checks the addressing alone,
// including rows past 2^32 elements (mlxcel issue #2153, Acceptance
// Criteria: a pool past 2^32 elements must match the gather path).
#include "pa_device.h"
#include "pa_host.h"

namespace pa {
namespace {

// One workgroup per token; threads copy the token's Hkv rows dword by dword.
__global__ void __launch_bounds__(256) gather_kernel(const GatherArgs a) {
  const int tok = a.t0 + blockIdx.x;
  const int jb = tok >> a.bs_shift;
  int32_t id = block_of(a.table, a.b, a.max_blocks, jb);
  if (uint32_t(id) >= uint32_t(a.nblocks)) {
    if (threadIdx.x == 0 && a.status) atomicOr(a.status, 1u);
    return;
  }
  const int slot = tok & ((1 << a.bs_shift) - 1);
  const uint8_t* src = a.pool + row_offset(id, slot, a.bs_shift, a.Hkv, 0, a.row_bytes);
  uint8_t* dst = a.dst + int64_t(blockIdx.x) * a.Hkv * a.row_bytes;
  const int ndw = a.Hkv * a.row_bytes / 4;
  for (int i = threadIdx.x; i < ndw; i += blockDim.x)
    reinterpret_cast<uint32_t*>(dst)[i] = ld_u32(src + 4 * i);
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
