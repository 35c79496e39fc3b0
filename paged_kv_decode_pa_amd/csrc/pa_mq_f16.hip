// Multi-query (tiled) kernel instantiations for f16 storage.
#include "pa_launch.h"

namespace pa {
PA_DEFINE_MQ_LAUNCHER(launch_mq_mfma_f16, DT_F16)
PA_DEFINE_MQ_WG_LAUNCHER(launch_mq_wg_f16, DT_F16)
size_t mq_mfma_lds_bytes(int D, int nr, int tiles, bool heads) {
  // identical for f16 and bf16 (MQShape::LDS_FLOATS)
  const int vf = 2 * (16 * tiles * D * 2) / 4;
  const int rd = heads ? 0 : 16 * nr * (D + 4);
  return sizeof(float) * (size_t)((vf > rd ? vf : rd) + 64 + 2 * 16 * nr);
}
}  // namespace pa
