// Status strings and ABI version of libdsa.so.
#include "dsa_host.hpp"

extern "C" const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a dimension is non-positive or inconsistent";
    case DSA_ERR_UNSUPPORTED: return "a dimension is outside what the kernels implement";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP launch error";
    case DSA_ERR_TOO_LARGE: return "the call needs more scratch than the fixed-size buffer holds";
    default: return "unknown status";
  }
}

extern "C" int dsa_abi_version(void) { return DSA_ABI_VERSION; }
