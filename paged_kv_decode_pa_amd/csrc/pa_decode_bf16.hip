// Decode-kernel instantiations for bf16 storage.
#include "pa_launch.h"

namespace pa {
PA_DEFINE_DECODE_LAUNCHER(launch_decode_bf16, DT_BF16)
PA_DEFINE_MFMA_LAUNCHER(launch_decode_mfma_bf16, DT_BF16)
}  // namespace pa
