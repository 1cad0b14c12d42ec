// Device scratch of ra_block_attn_fwd_noalloc: a fixed-size array in the
// library's code object, so callers that cannot allocate device memory
// (stream capture into a graph, tight serving loops, harnesses that forbid
// hipMalloc) still have room for the transposed V block.
//
// In host code `scratch` names a host-side stand-in, not a device address;
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and kept in a per-device table. Every call on a
// device shares that device's array: calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ra_internal.h"

namespace ra {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace ra
