// Host-side launchers, one translation unit per storage type.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_kernels.h"
#include "pa_mfma.h"
#include "pa_mq.h"

namespace pa {

// Each returns false when (head_dim, group) has no instantiation.  With
// blocks_per_cu set, nothing is launched: it receives how many such
// workgroups one CU holds at once.
bool launch_decode_f32(int D, int G, bool paged, bool loop, dim3 grid, dim3 block, hipStream_t s,
                       const DecodeParams& p, int* blocks_per_cu = nullptr);
bool launch_decode_f16(int D, int G, bool paged, bool loop, dim3 grid, dim3 block, hipStream_t s,
                       const DecodeParams& p, int* blocks_per_cu = nullptr);
bool launch_decode_bf16(int D, int G, bool paged, bool loop, dim3 grid, dim3 block, hipStream_t s,
                        const DecodeParams& p, int* blocks_per_cu = nullptr);

// Matrix-core path (f16/bf16, G in {8, 16}, block_size >= 16); returns
// false when not built for the shape.
// heads: one wavefront per KV head (nw = num_kv_heads).
bool launch_decode_mfma_f16(int D, int G, int tiles, bool loop, bool heads, int nw, dim3 grid,
                            hipStream_t s, const DecodeParams& p);
bool launch_decode_mfma_bf16(int D, int G, int tiles, bool loop, bool heads, int nw, dim3 grid,
                             hipStream_t s, const DecodeParams& p);
size_t decode_mfma_lds_bytes(int D, int G, int tiles);

// Tiled multi-query path (f16/bf16, block_size >= 16 * tiles); nr 16-row
// blocks per wavefront.  Returns false when not built for the shape.
// heads: one wavefront per KV head (nw = num_kv_heads).  With blocks_per_cu
// set, nothing is launched: it receives how many such workgroups one CU
// holds at once.
bool launch_mq_mfma_f16(int D, int nr, int tiles, bool heads, int nw, dim3 grid, hipStream_t s,
                        const MQParams& p, int* blocks_per_cu = nullptr);
bool launch_mq_mfma_bf16(int D, int nr, int tiles, bool heads, int nw, dim3 grid, hipStream_t s,
                         const MQParams& p, int* blocks_per_cu = nullptr);
size_t mq_mfma_lds_bytes(int D, int nr, int tiles, bool heads);

// Workgroup-shared multi-query path (four wavefronts of 16 * nr rows each).
bool launch_mq_wg_f16(int D, int nr, int tiles, int nbuf, dim3 grid, hipStream_t s,
                      const MQParams& p);
bool launch_mq_wg_bf16(int D, int nr, int tiles, int nbuf, dim3 grid, hipStream_t s,
                       const MQParams& p);

}  // namespace pa

// Expands to the body of a launcher for storage type DT.
#define PA_DECODE_CASE(DT, DV, GV)                                                  \
  case DV * 16 + GV:                                                                \
  {                                                                                 \
    const size_t lds = (block.x / 64) * sizeof(float) *                             \
                       DecodeShape<DT, DV, GV>::LDS_FLOATS;                          \
    if (blocks_per_cu)                                                              \
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(                          \
                 blocks_per_cu,                                                     \
                 paged ? (loop ? decode_kernel<DT, DV, GV, true, true>              \
                               : decode_kernel<DT, DV, GV, true, false>)            \
                       : (loop ? decode_kernel<DT, DV, GV, false, true>             \
                               : decode_kernel<DT, DV, GV, false, false>),          \
                 block.x, lds) == hipSuccess;                                       \
    if (p.tail_slots && !loop)                                                      \
      paged ? decode_kernel<DT, DV, GV, true, false, true><<<grid, block, lds, s>>>(p) \
            : decode_kernel<DT, DV, GV, false, false, true><<<grid, block, lds, s>>>(p); \
    else if (paged && loop) decode_kernel<DT, DV, GV, true, true><<<grid, block, lds, s>>>(p); \
    else if (paged) decode_kernel<DT, DV, GV, true, false><<<grid, block, lds, s>>>(p);     \
    else if (loop) decode_kernel<DT, DV, GV, false, true><<<grid, block, lds, s>>>(p);      \
    else decode_kernel<DT, DV, GV, false, false><<<grid, block, lds, s>>>(p);               \
    return true;                                                                    \
  }

#define PA_DEFINE_DECODE_LAUNCHER(NAME, DT)                                         \
  bool NAME(int D, int G, bool paged, bool loop, dim3 grid, dim3 block, hipStream_t s, \
            const DecodeParams& p, int* blocks_per_cu) {                            \
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

#define PA_MFMA_CASE(DT, DV, GV, TV)                                                \
  case (DV * 32 + GV) * 4 + TV: {                                                   \
    const size_t lds = (size_t)nw * sizeof(float) *                                 \
                       MfmaShape<DT, DV, GV, TV>::LDS_FLOATS;                       \
    if (heads && loop) decode_mfma_kernel<DT, DV, GV, TV, true, true><<<grid, dim3(64 * nw), lds, s>>>(p); \
    else if (heads) decode_mfma_kernel<DT, DV, GV, TV, false, true><<<grid, dim3(64 * nw), lds, s>>>(p); \
    else if (loop) decode_mfma_kernel<DT, DV, GV, TV, true><<<grid, dim3(64 * nw), lds, s>>>(p); \
    else decode_mfma_kernel<DT, DV, GV, TV, false><<<grid, dim3(64 * nw), lds, s>>>(p);     \
    return true;                                                                    \
  }

// two-tile chunks only up to head_dim 128 (the launcher's choice; at 256 the
// K fragments of both tiles do not fit in registers)
#define PA_DEFINE_MFMA_LAUNCHER(NAME, DT)                                           \
  bool NAME(int D, int G, int tiles, bool loop, bool heads, int nw, dim3 grid,      \
            hipStream_t s, const DecodeParams& p) {                                 \
    switch ((D * 32 + G) * 4 + tiles) {                                             \
      PA_MFMA_CASE(DT, 64, 8, 1) PA_MFMA_CASE(DT, 64, 8, 2)                         \
      PA_MFMA_CASE(DT, 128, 8, 1) PA_MFMA_CASE(DT, 128, 8, 2)                       \
      PA_MFMA_CASE(DT, 256, 8, 1)                                                   \
      PA_MFMA_CASE(DT, 64, 16, 1) PA_MFMA_CASE(DT, 64, 16, 2)                       \
      PA_MFMA_CASE(DT, 128, 16, 1) PA_MFMA_CASE(DT, 128, 16, 2)                     \
      PA_MFMA_CASE(DT, 256, 16, 1)                                                  \
      default: return false;                                                        \
    }                                                                               \
  }

#define PA_MQ_CASE(DT, DV, NRV, TV)                                                 \
  case (DV * 8 + NRV) * 4 + TV: {                                                   \
    if (heads) {                                                                    \
      const size_t lds = (size_t)nw * sizeof(float) * MQShape<DT, DV, NRV, TV, true>::LDS_FLOATS; \
      if (blocks_per_cu)                                                            \
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(                        \
                   blocks_per_cu, mq_mfma_kernel<DT, DV, NRV, TV, true>, 64 * nw, lds) == \
               hipSuccess;                                                          \
      mq_mfma_kernel<DT, DV, NRV, TV, true><<<grid, dim3(64 * nw), lds, s>>>(p);     \
    } else {                                                                        \
      const size_t lds = (size_t)nw * sizeof(float) * MQShape<DT, DV, NRV, TV>::LDS_FLOATS; \
      if (blocks_per_cu)                                                            \
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(                        \
                   blocks_per_cu, mq_mfma_kernel<DT, DV, NRV, TV, false>, 64 * nw, lds) == \
               hipSuccess;                                                          \
      mq_mfma_kernel<DT, DV, NRV, TV><<<grid, dim3(64 * nw), lds, s>>>(p);           \
    }                                                                               \
    return true;                                                                    \
  }

// head_dim 64 takes up to 4 row blocks, 128 up to 2, 256 one, and two-tile
// chunks only while nr * head_dim <= 128 (the accumulators, query and K
// fragments stay in registers)
#define PA_DEFINE_MQ_LAUNCHER(NAME, DT)                                             \
  bool NAME(int D, int nr, int tiles, bool heads, int nw, dim3 grid, hipStream_t s,  \
            const MQParams& p, int* blocks_per_cu) {                                \
    switch ((D * 8 + nr) * 4 + tiles) {                                             \
      PA_MQ_CASE(DT, 64, 1, 1) PA_MQ_CASE(DT, 64, 1, 2)                             \
      PA_MQ_CASE(DT, 64, 2, 1) PA_MQ_CASE(DT, 64, 2, 2)                             \
      PA_MQ_CASE(DT, 64, 4, 1)                                                      \
      PA_MQ_CASE(DT, 128, 1, 1) PA_MQ_CASE(DT, 128, 1, 2)                           \
      PA_MQ_CASE(DT, 128, 2, 1)                                                     \
      PA_MQ_CASE(DT, 256, 1, 1)                                                     \
      default: return false;                                                        \
    }                                                                               \
  }

#define PA_MQ_WG_CASE(DT, DV, NRV, TV, BV)                                          \
  case ((DV * 8 + NRV) * 8 + TV) * 8 + BV:                                          \
    mq_wg_kernel<DT, DV, NRV, TV, BV><<<grid, dim3(256), 0, s>>>(p); /* static LDS */ \
    return true;

#define PA_DEFINE_MQ_WG_LAUNCHER(NAME, DT)                                          \
  bool NAME(int D, int nr, int tiles, int nbuf, dim3 grid, hipStream_t s, const MQParams& p) { \
    switch (((D * 8 + nr) * 8 + tiles) * 8 + nbuf) {                               \
      PA_MQ_WG_CASE(DT, 64, 1, 1, 3) PA_MQ_WG_CASE(DT, 64, 1, 2, 3)                 \
      PA_MQ_WG_CASE(DT, 64, 1, 4, 3) PA_MQ_WG_CASE(DT, 64, 2, 4, 3)                 \
      PA_MQ_WG_CASE(DT, 64, 2, 1, 3) PA_MQ_WG_CASE(DT, 64, 2, 2, 3)                 \
      PA_MQ_WG_CASE(DT, 64, 4, 1, 3) PA_MQ_WG_CASE(DT, 64, 4, 2, 3)                 \
      PA_MQ_WG_CASE(DT, 64, 2, 2, 4) PA_MQ_WG_CASE(DT, 64, 4, 2, 4)                 \
      PA_MQ_WG_CASE(DT, 128, 1, 1, 3) PA_MQ_WG_CASE(DT, 128, 1, 2, 3)               \
      PA_MQ_WG_CASE(DT, 128, 2, 1, 3) PA_MQ_WG_CASE(DT, 128, 2, 2, 3)               \
      PA_MQ_WG_CASE(DT, 256, 1, 1, 3) PA_MQ_WG_CASE(DT, 256, 2, 1, 3)               \
      PA_MQ_WG_CASE(DT, 256, 1, 1, 4)                                               \
      default: return false;                                                        \
    }                                                                               \
  }
