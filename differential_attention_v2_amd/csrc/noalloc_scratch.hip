// Fixed device scratch for the decode entry point that allocates nothing
// (diffattn_decode_fwd_noalloc): the split kernel's partial-state records live
// in this array instead of a caller workspace.  Each device that loads the
// library holds its own copy, from module load until the process ends.
#include <mutex>

#include "diffattn.h"
#include "internal.h"

namespace diffattn {

static __device__ __align__(256) unsigned char scratch[DIFFATTN_NOALLOC_SCRATCH_BYTES];

hipError_t decode_scratch(void** ptr) {
  // In host code `scratch` names a host-side stand-in, not device memory: the
  // device copy's address is looked up once per device (with that device
  // current) and only that address is handed to kernels.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace diffattn
