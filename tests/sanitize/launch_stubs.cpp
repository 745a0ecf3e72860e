// Host-only stand-ins for the kernel launchers, so that the C ABI's host code
// (argument validation, kernel choice) can be built with the address and
// undefined-behaviour sanitizers and run without a GPU.  Nothing here touches
// memory; a "launch" succeeds.
#include "kernels.hpp"

namespace alnp {

hipError_t launch_adaln_fp8(const Fp8Args&, int, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_fp4(const Fp4Args&, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_modulation6(const Mod6Args&, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_gated_residual(const GateArgs&, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_quant_fp8(const float*, const float*, int64_t, uint8_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_mxfp8(const Fp8Args&, int, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_rms_modulate(const RmsArgs&, bool, hipStream_t) { return hipSuccess; }

}  // namespace alnp
