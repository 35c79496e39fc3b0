// Decode-kernel instantiations for f32 storage.
#include "pa_launch.h"

namespace pa {
PA_DEFINE_DECODE_LAUNCHER(launch_decode_f32, DT_F32)
}  // namespace pa
