// Scratch of the allocation-free forward entry point: a file-scope device
// array instead of a caller workspace, for callers that cannot allocate
// (code under graph capture, tight serving loops). Each GPU holds its own
// copy from module load until the process ends.
//
// In host code the array's name is a host-side stand-in, not a device
// address: its device address is taken with hipGetSymbolAddress, once per
// device with that device current, and only that address is ever handed to
// kernels. The array is zero at load; its first QLORA_LINEAR_SYNC_BYTES are
// the linear path's synchronization words, which every call leaves zero, so
// they need no clearing between calls. The rest keeps the last call's
// contents; no kernel reads scratch it has not written in the same call.
#include <mutex>

#include "internal.h"

namespace qnf4 {
namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace qnf4
