// Host-side launchers, one translation unit per storage type.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_kernels.h"

namespace pa {

// Each returns false when (head_dim, group) has no instantiation.
bool launch_decode_f32(int D, int G, bool paged, dim3 grid, dim3 block, hipStream_t s, const DecodeParams& p);
bool launch_decode_f16(int D, int G, bool paged, dim3 grid, dim3 block, hipStream_t s, const DecodeParams& p);
bool launch_decode_bf16(int D, int G, bool paged, dim3 grid, dim3 block, hipStream_t s, const DecodeParams& p);

}  // namespace pa

// Expands to the body of a launcher for storage type DT.
#define PA_DECODE_CASE(DT, DV, GV)                                                  \
  case DV * 16 + GV:                                                                \
    if (paged) decode_kernel<DT, DV, GV, true><<<grid, block, 0, s>>>(p);           \
    else decode_kernel<DT, DV, GV, false><<<grid, block, 0, s>>>(p);                \
    return true;

#define PA_DEFINE_DECODE_LAUNCHER(NAME, DT)                                         \
  bool NAME(int D, int G, bool paged, dim3 grid, dim3 block, hipStream_t s,         \
            const DecodeParams& p) {                                                \
    switch (D * 16 + G) {                                                           \
      PA_DECODE_CASE(DT, 64, 1) PA_DECODE_CASE(DT, 64, 2)                           \
      PA_DECODE_CASE(DT, 64, 4) PA_DECODE_CASE(DT, 64, 8)                           \
      PA_DECODE_CASE(DT, 128, 1) PA_DECODE_CASE(DT, 128, 2)                         \
      PA_DECODE_CASE(DT, 128, 4) PA_DECODE_CASE(DT, 128, 8)                         \
      PA_DECODE_CASE(DT, 256, 1) PA_DECODE_CASE(DT, 256, 2)                         \
      PA_DECODE_CASE(DT, 256, 4) PA_DECODE_CASE(DT, 256, 8)                         \
      default: return false;                                                        \
    }                                                                               \
  }
