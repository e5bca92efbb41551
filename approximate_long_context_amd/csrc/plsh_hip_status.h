// plsh_hip_status.h -- HIP error checks of the device-side translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "plsh_internal.h"

namespace plsh {

// PLSH_ERR_HIP with the runtime's message when the last launch failed.
inline plsh_status launch_check(const char *who) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PLSH_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PLSH_OK;
}

// PLSH_ERR_HIP when no HIP device is usable from this thread.
inline plsh_status have_device(const char *who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PLSH_ERR_HIP, "%s: no HIP device: %s", who, hipGetErrorString(e));
  }
  return PLSH_OK;
}

}  // namespace plsh
