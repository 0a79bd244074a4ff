// Stand-ins for the kernel launchers of libwanattn, for a host-only build of
// the C ABI layer (attention_wan_qk_amd/csrc/wan_api.cpp) under the address
// and undefined-behaviour sanitizers. Reaching one means every host check
// passed: it launches nothing and returns an error, which the ABI reports as
// WAN_ERROR_LAUNCH, so a rejection test whose check regressed fails on the
// status code instead of touching device memory.
#include "../../attention_wan_qk_amd/csrc/wan_internal.h"

namespace wan {

hipError_t launch_norm_rope(const NormRopeArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_adaln(const AdaLNArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_fwd(const AttnArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_linear(const LinearArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_quant8(const Quant8Args&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn8_fwd(const Attn8Args&, hipStream_t) { return hipErrorNotSupported; }
// no device: the allocation-free call cannot look up its scratch array
hipError_t device_scratch(void**, uint64_t*) { return hipErrorNotSupported; }
// a 256-unit device, so that workspace sizes are those of the real one
hipError_t device_cu_count(int* n) {
  *n = 256;
  return hipSuccess;
}

}  // namespace wan
