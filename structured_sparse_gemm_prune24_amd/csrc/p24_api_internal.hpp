// Host-side helpers shared by the C ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/prune24.h"

static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Status of the launch just enqueued.
static inline p24_status launch_status() {
  return hipGetLastError() == hipSuccess ? P24_OK : P24_ERR_HIP;
}
