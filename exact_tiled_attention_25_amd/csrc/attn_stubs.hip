// Entry points whose kernels are not built yet report ATTN_ELAUNCH through an invalid launch code.
#include "attn_launch.h"
namespace attn {
hipError_t launch_fp8_quantize(bool, int, const Fp8QuantParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_fp8(bool, int, bool, const Fp8FwdParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
