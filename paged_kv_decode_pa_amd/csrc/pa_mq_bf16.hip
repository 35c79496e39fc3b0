// Multi-query (tiled) kernel instantiations for bf16 storage.
#include "pa_launch.h"

namespace pa {
PA_DEFINE_MQ_LAUNCHER(launch_mq_mfma_bf16, DT_BF16)
PA_DEFINE_MQ_WG_LAUNCHER(launch_mq_wg_bf16, DT_BF16)
}  // namespace pa
