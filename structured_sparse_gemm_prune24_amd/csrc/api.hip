// Library-level C ABI entry points (version, error strings).
#include "p24_api_internal.hpp"

extern "C" P24_API int32_t prune24_abi_version(void) { return PRUNE24_ABI_VERSION; }

extern "C" P24_API const char* prune24_strerror(p24_status s) {
  switch (s) {
    case P24_OK: return "ok";
    case P24_ERR_NULL: return "a required pointer is NULL";
    case P24_ERR_SHAPE: return "invalid shape, leading dimension, tile or keep count";
    case P24_ERR_ALIGN: return "pointer or leading dimension not aligned as required";
    case P24_ERR_DTYPE: return "unknown or unsupported dtype";
    case P24_ERR_UNSUPPORTED: return "request not supported by the library (see the shape rules)";
    case P24_ERR_HIP: return "HIP runtime error at kernel launch";
    case P24_ERR_WORKSPACE: return "workspace missing or too small";
    case P24_ERR_LAYOUT: return "unknown layout, or layout not accepted by this entry point";
    case P24_ERR_SCRATCH: return "problem larger than the fixed scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}
