// attn_mfma_tiled.hip -- placeholder until the LDS-tiled MFMA kernel lands.
#include "kvq_internal.h"
namespace kvq {
hipError_t launch_attn_mfma_tiled(const AttnArgs&, const AttnPlan&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kvq
