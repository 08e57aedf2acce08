// fp8 (e4m3) path: placeholder until the kernels land.
#include "common.h"
#include "launch.h"

namespace attn127 {
hipError_t launch_fp8_prepare(const Fp8PrepArgs&) { return hipErrorNotSupported; }
hipError_t launch_fp8_fwd(const Fp8Args&) { return hipErrorNotSupported; }
}  // namespace attn127
