// Shared host/device helpers of libkvq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kTokenBlock = 64;  // padding granularity of a chunk and size of a value block

__host__ __device__ inline int chunk_pad(int chunk_len) {
  return (chunk_len + kTokenBlock - 1) / kTokenBlock * kTokenBlock;
}

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
