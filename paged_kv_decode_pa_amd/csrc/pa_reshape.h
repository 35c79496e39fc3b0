// The KV-cache scatter used by pa_reshape_and_cache.
#pragma once

#include "pa_device.h"

namespace pa {

// One workgroup per new token: copy its K and V rows (all KV heads) into
// slot slot_mapping[i] with 16-byte moves.
__global__ __launch_bounds__(256) void reshape_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const int64_t* __restrict__ slot_mapping, int64_t num_slots, int row16) {
  const int i = blockIdx.x;
  const int64_t s = slot_mapping[i];
  if (s < 0 || s >= num_slots) return;
  const uint4* ks = key + (int64_t)i * row16;
  const uint4* vs = value + (int64_t)i * row16;
  uint4* kd = k_cache + s * row16;
  uint4* vd = v_cache + s * row16;
  for (int j = threadIdx.x; j < row16; j += blockDim.x) {
    kd[j] = ks[j];
    vd[j] = vs[j];
  }
}

}  // namespace pa
