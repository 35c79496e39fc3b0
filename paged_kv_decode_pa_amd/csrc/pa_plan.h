// Work ordering for pa_decode.
#pragma once

#include "pa_device.h"

namespace pa {

// One workgroup: order the sequences by attended length, longest first
// (counting sort over 256 length buckets; order within a bucket is
// arbitrary, which no result depends on).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ context_lens,
                                                    int num_seqs, int max_context_len, int window,
                                                    int32_t* __restrict__ order) {
  constexpr int NBK = 256;
  __shared__ int hist[NBK];
  __shared__ int offs[NBK];
  const int t = threadIdx.x;
  if (t < NBK) hist[t] = 0;
  __syncthreads();
  const int span = max(max_context_len, 1);
  auto bucket = [&](int b) {
    int n = min(max(context_lens[b], 0), max_context_len);
    if (window > 0) n = min(n, window);
    // descending: the longest sequences land in bucket 0
    return NBK - 1 - (int)(((long long)n * (NBK - 1)) / span);
  };
  for (int b = t; b < num_seqs; b += blockDim.x) atomicAdd(&hist[bucket(b)], 1);
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int k = 0; k < NBK; ++k) {
      offs[k] = run;
      run += hist[k];
    }
  }
  __syncthreads();
  for (int b = t; b < num_seqs; b += blockDim.x) order[atomicAdd(&offs[bucket(b)], 1)] = b;
}

}  // namespace pa
