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

// One workgroup per (src, dst) pair: 16-byte copies of a whole block of K
// and of V.
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const int64_t* __restrict__ block_mapping, int64_t num_blocks, int64_t block16) {
  const int64_t src = block_mapping[2 * (int64_t)blockIdx.x];
  const int64_t dst = block_mapping[2 * (int64_t)blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint4* ks = k_cache + src * block16;
  const uint4* vs = v_cache + src * block16;
  uint4* kd = k_cache + dst * block16;
  uint4* vd = v_cache + dst * block16;
  for (int64_t j = threadIdx.x; j < block16; j += blockDim.x) {
    kd[j] = ks[j];
    vd[j] = vs[j];
  }
}

}  // namespace pa
