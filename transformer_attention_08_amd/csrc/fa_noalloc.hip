// The fixed scratch array behind fa_forward_splitkv_noalloc: the split-KV
// partials (per key block: O_g and LSE_g of every row) of callers that
// cannot allocate device memory. One copy per GPU, held by the loaded code
// object until the process ends; every call on a GPU reuses its contents.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fa_kernels.h"

namespace {

static __device__ __align__(256) uint8_t scratch[fa::kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device

}  // namespace

namespace fa {

// Device address of this GPU's scratch array, looked up once per device with
// that device current (the array's name is only a host-side stand-in; its
// device address differs per GPU).
hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace fa
