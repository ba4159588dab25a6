// Stand-ins for the kernel launchers, for the host-sanitizer build of the C
// ABI shim: they launch nothing, record the parameter blocks the shim built,
// and return success, so that every host path of bsm_api.cpp runs without a
// GPU under AddressSanitizer and UndefinedBehaviorSanitizer.
#include "stub_launchers.hpp"

namespace stub {
int calls = 0;
bsm::AttnParams last_attn{};
bsm::MaskBuildParams last_build{};
bsm::DecodeLaunch last_decode{};
bsm::GatherLaunch last_gather{};
float *last_decode_part = nullptr;
}  // namespace stub

namespace bsm {

static hipError_t record(const AttnParams &p) {
    ++stub::calls;
    stub::last_attn = p;
    return hipSuccess;
}

hipError_t launch_gather_pages(const GatherLaunch &g, hipStream_t) {
    ++stub::calls;
    stub::last_gather = g;
    return hipSuccess;
}
hipError_t launch_build_block_mask(const MaskBuildParams &p, hipStream_t) {
    ++stub::calls;
    stub::last_build = p;
    return hipSuccess;
}
hipError_t launch_attn_fwd_d64_bf16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_fwd_d128_bf16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_bwd_d64_bf16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_bwd_d128_bf16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_fwd_d64_f16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_fwd_d128_f16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_fwd_d256_bf16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_fwd_d256_f16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_bwd_d256_bf16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_bwd_d256_f16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_bwd_d64_f16(const AttnParams &p, hipStream_t) { return record(p); }
hipError_t launch_attn_bwd_d128_f16(const AttnParams &p, hipStream_t) { return record(p); }

static hipError_t record_decode(const DecodeLaunch &d, float *part) {
    ++stub::calls;
    stub::last_decode = d;
    stub::last_decode_part = part;
    return hipSuccess;
}
hipError_t launch_attn_decode_bf16(const DecodeLaunch &d, float *part, hipStream_t) { return record_decode(d, part); }
hipError_t launch_attn_decode_f16(const DecodeLaunch &d, float *part, hipStream_t) { return record_decode(d, part); }

}  // namespace bsm
