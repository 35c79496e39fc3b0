// Decode-kernel instantiations for f16 storage.
#include "pa_launch.h"

namespace pa {
PA_DEFINE_DECODE_LAUNCHER(launch_decode_f16, DT_F16)
}  // namespace pa
