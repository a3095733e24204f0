// Static device scratch of attn_bwd_noalloc: the backward's workspace for
// callers that cannot allocate device memory.  One file-scope array, of
// which every GPU the library runs on holds its own copy from the moment
// this code object is loaded there until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_internal.h"

namespace eta {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU

// In host code `scratch` names a host-side stand-in, not device memory: only
// the address hipGetSymbolAddress returns (per device) reaches the kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_dev[kMaxDevices];  // device address of each GPU's copy, once resolved
std::mutex g_scratch_mu;
}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return (int)e;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return 0;
}

}  // namespace eta
