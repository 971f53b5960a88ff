// Workspace of the no-allocation decode step (paged_attn_step_noalloc).
//
// Some callers cannot allocate device memory while they run (code under HIP
// graph capture, tight serving loops). For them the decode step's workspace
// - the status word and the partition partials that paged_attn_step keeps in
// the caller's `ws` - lives in a file-scope device array of fixed size,
// `scratch`, which every GPU the library runs on holds from the moment the
// library's code object is loaded on it until the process ends. The host
// never uses the array's name as an address: on its first use on a device
// the entry point looks the array up with hipGetSymbolAddress (with that
// device current) and keeps the device address per device.
//
// Nothing in the scratch has to start at zero: the decode kernels write every
// partial the merge reads before it reads it, and only OR bits into the
// status word, which this entry point never reads. Every call on a GPU shares
// that GPU's array, so two calls that overlap on one GPU (different streams,
// or different host threads) race on it.
#include <mutex>

#include "pa_host.h"

namespace pa {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *addr = g_addr[dev];
  return hipSuccess;
}

}  // namespace pa
