// attn_mfma_stream.hip -- placeholder until the streaming MFMA kernel lands.
#include "kvq_internal.h"
namespace kvq {
hipError_t launch_attn_mfma_stream(const AttnArgs&, const AttnPlan&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kvq
