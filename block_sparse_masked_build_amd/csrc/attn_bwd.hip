// Block-sparse masked attention, backward pass (placeholder launcher).
#include "attn_common.hpp"

namespace bsm {
hipError_t launch_attn_bwd(const AttnParams &, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace bsm
