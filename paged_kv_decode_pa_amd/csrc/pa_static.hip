// pa_step_static: the layer step with its scratch in a file-scope device
// array instead of a caller-provided workspace, for callers that cannot
// allocate device memory.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/pa.h"

// One copy per GPU, alive until the process ends.  Host code never uses this
// name as an address: on the host it is only a stand-in for the symbol.
static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The device address of the current device's copy of `scratch`, looked up
// once per device with that device current; null on failure.
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int pa_step_static(const pa_step_args* a, void* stream) {
  if (!a) return PA_EINVAL;
  const size_t need = pa_decode_workspace_size(a->num_seqs, a->num_heads, a->head_dim,
                                               a->max_context_len, a->partition_size);
  if (need > (size_t)PA_STATIC_SCRATCH_BYTES) return PA_ESCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ELAUNCH;
  void* p = scratch_ptr(dev);
  if (!p) return PA_ELAUNCH;
  pa_step_args b = *a;
  b.workspace = p;
  b.workspace_bytes = (size_t)PA_STATIC_SCRATCH_BYTES;
  return pa_step(&b, stream);
}

}  // extern "C"
