// Test-only launchers for a host-only build of the C-ABI layer (gdn_api.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer: every launcher reports that no device is present, so the
// validation paths and the error reporting run without any GPU code.
#include "gdn_launch.h"
#include "gdn_prefill_launch.h"
#include "gdn_lowrank_launch.h"
namespace gdn {
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_verify(const VerifyArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_conv_gate_decode(const FusedArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_lowrank(const LowrankArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t prefill_scratch_address(float**) { return hipErrorNoDevice; }
}
