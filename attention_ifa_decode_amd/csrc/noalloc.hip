// ifa_decode without a caller-supplied workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The split partials go to one fixed device array, `scratch`, of
// IFA_NOALLOC_SCRATCH_BYTES, which every device the library runs on holds
// until the process ends.  Its device address is taken once per device, at
// the first call made with that device current, through hipGetSymbolAddress;
// host code uses only that address, never the array's name (which in host
// code names a host-side stand-in).  Nothing here allocates: no hipMalloc,
// hipFree or allocating library routine.
//
// No part of the array needs to start at zero: the combine uses only the
// partial slots that the split-KV kernel of the same call writes (the
// per-sequence layout reads stale slots of empty splits but gives them no
// weight; the balanced layout reads the (first slot, count) pair of a
// sequence with tokens, which that call's kernel writes).  All calls on one
// device share the array, so calls that overlap on one device (on different
// streams, or from different threads without ordering) race.
#include <mutex>

#include "../../include/ifa_decode.h"
#include "kernels.hpp"

namespace ifa {
// Records the calling thread's error message (what ifa_last_error returns)
// and returns st; printf-style.  Defined with the rest of the C ABI.
ifa_status set_last_error(ifa_status st, const char* fmt, ...);
}  // namespace ifa

namespace {

constexpr size_t kScratchBytes = IFA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

}  // namespace

// the fixed partials array; in host code this name is a host-side stand-in
static __device__ __align__(256) char scratch[kScratchBytes];

extern "C" ifa_status ifa_decode_noalloc(const ifa_decode_args* args, hipStream_t stream) {
  size_t bytes = 0;
  ifa_status st = ifa_decode_workspace_size(args, &bytes);
  if (st != IFA_OK) return st;
  if (bytes > kScratchBytes)
    return ifa::set_last_error(IFA_ERR_PLAN,
                               "ifa_decode_noalloc: this call needs %zu bytes of partials, more than the %zu of the "
                               "library's fixed scratch array; use ifa_decode with a workspace",
                               bytes, kScratchBytes);
  if (args->batch == 0) return ifa_decode(args, nullptr, 0, stream);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ifa::set_last_error(IFA_ERR_RUNTIME, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return ifa::set_last_error(IFA_ERR_RUNTIME, "device %d outside the %d this library tracks", dev, kMaxDevices);
  // once per device, with that device current: the device address of this
  // device's copy of the array
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr)
    return ifa::set_last_error(IFA_ERR_RUNTIME, "hipGetSymbolAddress(scratch): %s",
                               hipGetErrorString(g_scratch_err[dev]));
  return ifa_decode(args, g_scratch_ptr[dev], kScratchBytes, stream);
}
