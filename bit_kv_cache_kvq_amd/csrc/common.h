// Shared host/device helpers of libkvq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host.h"
#include "kvq.h"

namespace kvq {

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
