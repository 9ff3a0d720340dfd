// Launcher stubs for the sanitizer build of the C ABI's host code
// (kda_api.hip): argument checks, size functions and buffer layouts run for
// real; any call that passes the checks reaches one of these and fails with
// hipErrorNotSupported, so no device code is needed.
#include "../../gated_delta_rule_41_amd/csrc/kda_internal.h"

namespace kda {
hipError_t launch_fwd(const FwdParams&, int, int, int, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd(const BwdParams&, int, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode(const DecodeParams&, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_segments(const SegParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_maps(const FwdParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_carry(const CarryParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_staged(const StagedParams&, int, int, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kda
