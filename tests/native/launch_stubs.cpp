// Stand-ins for the kernel launchers, linked only into the sanitizer build of
// the host runtime (tests/test_abi_sanitize.py), which runs on a machine
// without a GPU.  Every check that program makes returns before a launch;
// should one be reached, it fails with an error instead of running anything.
#include "fb_internal.h"

namespace fbk {
hipError_t launch_attn(int, int, int, const AttnParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_combine(int, const CombineParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decide(const DecideParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_reset(const ResetParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_complement(const ComplementParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_fin(const AttnParams&, const FinParams&, hipStream_t) { return hipErrorNoDevice; }
bool fin_supported(int, int, const AttnParams&) { return false; }
}  // namespace fbk
