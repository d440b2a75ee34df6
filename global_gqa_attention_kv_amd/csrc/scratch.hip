// scratch.hip -- device-resident scratch for gqa_attn_decode_noalloc, the
// decode entry point for callers that cannot allocate (code under HIP graph
// capture, tight serving loops): its split partials go to a file-scope
// device array instead of a caller workspace.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Host code never uses the array's name as an address (on the
// host it names a stand-in, not device memory): its device address is looked
// up once per device with hipGetSymbolAddress, with that device current, and
// remembered.
#include <atomic>

#include "internal.h"

namespace gqa {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::atomic<uintptr_t> addr[kMaxDevices];  // 0 = not looked up yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return nullptr;
  uintptr_t a = addr[dev].load(std::memory_order_acquire);
  if (a) return reinterpret_cast<void*>(a);
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
    return nullptr;
  addr[dev].store(reinterpret_cast<uintptr_t>(ptr), std::memory_order_release);
  return ptr;
}

}  // namespace gqa
