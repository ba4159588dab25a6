// What the stand-in launchers record (see stub_launchers.cpp).
#pragma once
#include "../../block_sparse_masked_build_amd/csrc/bsm_internal.hpp"

namespace stub {
extern int calls;
extern bsm::AttnParams last_attn;
extern bsm::MaskBuildParams last_build;
extern bsm::DecodeLaunch last_decode;
extern bsm::GatherLaunch last_gather;
extern float *last_decode_part;
}  // namespace stub
