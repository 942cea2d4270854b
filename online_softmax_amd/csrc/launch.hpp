// Launch-status check and device queries shared by the entry points.
#pragma once
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/sa_attn.h"
#include "host_logic.hpp"

namespace sa {

// SA_OK, or SA_ERR_HIP with the launch error recorded.
inline int launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return SA_OK;
}

constexpr int kMaxDevices = 64;

// Compute-unit count per device, queried once.
inline int num_cus(int* out) {
  static std::once_flag flags[kMaxDevices];
  static int cus[kMaxDevices];
  static hipError_t errs[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_HIP, "device index %d out of range", dev);
  std::call_once(flags[dev], [dev] {
    errs[dev] = hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
  });
  if (errs[dev] != hipSuccess)
    return fail(SA_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(errs[dev]));
  *out = cus[dev];
  return SA_OK;
}

// Split and merge launches of a validated decode (sa_attn.hip) over `splits`
// splits with its partial results in `workspace`, which holds at least
// decode_layout(B, H_q, splits, D).bytes.
int launch_decode(const DecodeShape& s, int splits, void* workspace, sa_stream_t stream);

}  // namespace sa
