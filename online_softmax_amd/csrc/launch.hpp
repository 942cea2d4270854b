// Launch-status check shared by the entry points.
#pragma once
#include <hip/hip_runtime.h>

#include "host_logic.hpp"

namespace sa {

// SA_OK, or SA_ERR_HIP with the launch error recorded.
inline int launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return SA_OK;
}

}  // namespace sa
