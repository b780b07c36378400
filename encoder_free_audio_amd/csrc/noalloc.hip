// Scratch memory of the allocation-free forward (dmel_forward_noalloc): the
// intermediates of one call (levels, RMSNorm scales, and for small batches the
// RMSNorm partial sums) live in a fixed-size device array of this library
// instead of a caller's workspace, for callers that cannot allocate.
//
// In host code the array's name is only a host-side stand-in; its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current, from dmel_create) and that address is what the kernels get.  Each
// GPU holds its own copy of the array until the process ends.  Every call on
// a GPU uses the same array, so calls that overlap on one GPU race.
#include <mutex>

#include "internal.h"

namespace dmel {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[device] != nullptr) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch[device] = p;
  return hipSuccess;
}

void* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_scratch[device];
}

}  // namespace dmel
