// gdn_noalloc.hip -- the fixed device array behind gdn_prefill_noalloc, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU that loads this code object
// holds its own copy, at its own address, until the process ends. In host code the name
// `scratch` is only a host-side handle of the symbol, not a device address, so it is never
// passed to a kernel or a copy: the first call on a device resolves the device address with
// hipGetSymbolAddress, with that device current, and keeps it per device; every later use
// goes through that address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __align__(256) unsigned char scratch[GDN_PREFILL_NOALLOC_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once resolved

}  // namespace

// The device address of `scratch` on `device`, resolved on the first call for that device
// (with the device made current for the lookup, then the caller's device restored).
hipError_t noalloc_scratch(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[device]) {
    int current = 0;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t restore = current != device ? hipSetDevice(current) : hipSuccess;
    if (e != hipSuccess) return e;
    if (restore != hipSuccess) return restore;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[device] = ptr;
  }
  *out = g_scratch[device];
  return hipSuccess;
}

}  // namespace gdn
