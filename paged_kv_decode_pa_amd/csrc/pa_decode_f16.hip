// Decode-kernel instantiations for f16 storage.
#include "pa_launch.h"

namespace pa {
PA_DEFINE_DECODE_LAUNCHER(launch_decode_f16, DT_F16)
PA_DEFINE_MFMA_LAUNCHER(launch_decode_mfma_f16, DT_F16)
size_t decode_mfma_lds_bytes(int D, int G, int tiles) {
  // identical for f16 and bf16: every element is 2 bytes
  const int vf = PA_MFMA_DEPTH * (16 * tiles * D * 2 / 4);  // the V chunks in flight
  return sizeof(float) * (size_t)(vf + 64 + 2 * G + G * (D + 4));
}
}  // namespace pa
