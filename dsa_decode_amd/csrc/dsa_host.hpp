// Host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

// After a kernel launch: map a launch error to DSA_ERR_HIP.
inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int ceil_div(long a, long b) { return int((a + b - 1) / b); }

}  // namespace dsa
