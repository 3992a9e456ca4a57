// Scratch memory of the allocation-free selection call, for callers that
// cannot allocate device memory (code under HIP graph capture, serving
// loops that forbid allocation).
//
// The scratch is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a host-side stand-in, so its device address
// is looked up once per device, with that device current, and kept; the
// kernels only ever get that address.
#include <mutex>

#include "kernels.hpp"

namespace cskv {

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  try {                                    // no exception may leave a C entry point
    std::call_once(g_once[dev], [dev] {
      void* p = nullptr;
      g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
  } catch (...) {
    return hipErrorUnknown;
  }
  *ptr = g_ptr[dev];
  return g_err[dev];
}

}  // namespace cskv
