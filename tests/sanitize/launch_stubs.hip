// Launcher stubs for the host-sanitizer build of the C ABI layer: the ABI's
// validation runs in full, and a call that passes it reaches one of these
// instead of a kernel, which reports that the launch is not available.  No
// device code is built.
#include "launch.hpp"

namespace fa {

hipError_t launch_fwd_mfma(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_mfma(const AttnArgs&, hipStream_t, int) { return hipErrorNotSupported; }
hipError_t launch_fwd_f32(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_f32(const AttnArgs&, hipStream_t, int) { return hipErrorNotSupported; }
hipError_t launch_kvcache(const KvArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_preprocess(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa
