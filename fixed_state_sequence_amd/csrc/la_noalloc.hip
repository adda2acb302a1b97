// Static scratch memory for la_prefill_noalloc, the prefill entry point for
// callers that cannot allocate device memory.
//
// The chunked prefill keeps one state slot per stage-1 sub-segment (and the
// slots' log-decays and stabilisers) between its three stages.  la_prefill
// takes that workspace from the caller; la_prefill_noalloc takes it from the
// file-scope array below instead, which every GPU the library runs on holds
// (LA_NOALLOC_SCRATCH_BYTES) from the loading of this code object until the
// process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.  Every
// call on one device shares that device's array: calls that overlap on one
// GPU (two streams, two threads) race on it.  Nothing in it has to start at
// zero: stage 1 writes every slot the scan and stage 3 read in the same call.
#include <mutex>

#include "la_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

namespace la {

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace la
