// Read-bandwidth probe: one plain streaming pass over a device buffer, the
// practical ceiling the memory-bound attention kernels are measured against
// (the data sheet's HBM peak is not reachable by any kernel).
#include <hip/hip_runtime.h>

#include "../../include/pa.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One pass of 16-byte non-temporal loads in which each workgroup step reads
// one contiguous block of UNROLL * 4 KB (lane l of load u at word
// 256 u + l of the block), the blocks dealt to the workgroups in turn; the
// words are folded into one value that is stored only when it matches a
// pattern the caller never fills in, so the loads stay and nothing is
// written.  (Measured on MI355X over 4 GiB: contiguous 32 KB blocks read
// 7.1-7.2 TB/s where a grid-stride pass of the same loads, consecutive
// lanes of a workgroup 4 KB apart from the next workgroup's, read
// 6.3-7.0 TB/s.)
template <int UNROLL>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p, size_t n16,
                                                         unsigned int* sink) {
  constexpr size_t kBlock = (size_t)256 * UNROLL;  // 16-byte words per block
  unsigned int acc = 0;
  const size_t nblocks = n16 / kBlock;
  for (size_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    const u32x4* q = p + blk * kBlock + threadIdx.x;
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(q + u * 256);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // the words past the last whole block
  for (size_t i = nblocks * kBlock + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

}  // namespace

extern "C" int pa_read_bandwidth_probe(const void* buf, size_t bytes, int grid, void* sink,
                                       void* stream) {
  if (!buf || !sink || grid < 1 || bytes < 16 || bytes % 16 ||
      reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(sink) % 4)
    return PA_EINVAL;
  read_probe_kernel<8><<<dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(buf), bytes / 16, static_cast<unsigned int*>(sink));
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
}
