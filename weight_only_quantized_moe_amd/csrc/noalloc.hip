// hybrid_moe_forward_static: the layer forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). The scratch the forward needs comes from a file-scope device array of
// fixed size instead of a caller buffer; the library never allocates.
#include <mutex>
#include <string>

#include "hmoe_internal.h"

namespace {

constexpr size_t kStaticScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

// One copy per GPU, at its own device address, held until the process ends. In host
// code this name stands for the symbol only; its device address comes from
// hipGetSymbolAddress.
__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

thread_local std::string g_error;

}  // namespace

namespace hmoe {

// The device address of this device's static scratch array (looked up once per device,
// with that device current).
hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

size_t static_scratch_bytes() { return kStaticScratchBytes; }

}  // namespace hmoe
