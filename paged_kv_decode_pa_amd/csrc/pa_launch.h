// Host-side launchers, one translation unit per storage type.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_kernels.h"

namespace pa {

// Each returns false when (head_dim, group) has no instantiation.
bool launch_decode_f32(int D, int G, dim3 grid, dim3 block, hipStream_t s, const DecodeParams& p);
bool launch_decode_f16(int D, int G, dim3 grid, dim3 block, hipStream_t s, const DecodeParams& p);
bool launch_decode_bf16(int D, int G, dim3 grid, dim3 block, hipStream_t s, const DecodeParams& p);

}  // namespace pa

// Expands to the body of a launcher for storage type DT.
#define PA_DEFINE_DECODE_LAUNCHER(NAME, DT)                                          \
  bool NAME(int D, int G, dim3 grid, dim3 block, hipStream_t s, const DecodeParams& p) { \
    switch (D * 16 + G) {                                                           \
      case 64 * 16 + 1: decode_kernel<DT, 64, 1><<<grid, block, 0, s>>>(p); return true;   \
      case 64 * 16 + 2: decode_kernel<DT, 64, 2><<<grid, block, 0, s>>>(p); return true;   \
      case 64 * 16 + 4: decode_kernel<DT, 64, 4><<<grid, block, 0, s>>>(p); return true;   \
      case 64 * 16 + 8: decode_kernel<DT, 64, 8><<<grid, block, 0, s>>>(p); return true;   \
      case 128 * 16 + 1: decode_kernel<DT, 128, 1><<<grid, block, 0, s>>>(p); return true; \
      case 128 * 16 + 2: decode_kernel<DT, 128, 2><<<grid, block, 0, s>>>(p); return true; \
      case 128 * 16 + 4: decode_kernel<DT, 128, 4><<<grid, block, 0, s>>>(p); return true; \
      case 128 * 16 + 8: decode_kernel<DT, 128, 8><<<grid, block, 0, s>>>(p); return true; \
      case 256 * 16 + 1: decode_kernel<DT, 256, 1><<<grid, block, 0, s>>>(p); return true; \
      case 256 * 16 + 2: decode_kernel<DT, 256, 2><<<grid, block, 0, s>>>(p); return true; \
      case 256 * 16 + 4: decode_kernel<DT, 256, 4><<<grid, block, 0, s>>>(p); return true; \
      case 256 * 16 + 8: decode_kernel<DT, 256, 8><<<grid, block, 0, s>>>(p); return true; \
      default: return false;                                                        \
    }                                                                               \
  }
