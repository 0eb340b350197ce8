// The workspace of wide_ffn_forward_noalloc, for callers that cannot
// allocate: one static device array per GPU, placed by the code-object loader
// when the library is loaded on that GPU and held until the process ends.
//
// Host code never uses the array's name as an address: on the host it names
// a stand-in, not device memory, and a kernel handed it would fault. The
// device address comes from hipGetSymbolAddress, called once per device with
// that device current, and is kept in a per-device table.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"
#include "wide.h"

namespace wide {

namespace {

__device__ __attribute__((aligned(256))) uint8_t scratch[WIDE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipSuccess;
  if (stream != nullptr) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(stream, &sd);
    dev = (int)sd;
  } else {
    e = hipGetDevice(&dev);
  }
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t restore = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (restore != hipSuccess) return restore;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace wide
