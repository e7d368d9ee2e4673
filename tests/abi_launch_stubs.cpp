// Host-only stand-ins for the kernel launchers of libmiattn, for building the
// C-ABI validation layer (fa_api.cpp) with the host sanitizers and no GPU
// code.  Every launcher reports a failed launch, so a call that passes
// validation returns FA_ERR_LAUNCH and nothing is computed.
#include <hip/hip_runtime.h>

#include "../tiled_attention_fa_amd/csrc/fa_launch.h"

namespace miattn {

template <int D, bool F32>
hipError_t launch_fwd_dt(const FwdArgs&, int, int, hipStream_t) {
  return hipErrorLaunchFailure;
}
template hipError_t launch_fwd_dt<64, false>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd_dt<128, false>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd_dt<64, true>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd_dt<128, true>(const FwdArgs&, int, int, hipStream_t);

template <int D>
hipError_t launch_bwd_d(const BwdArgs&, int, int, int, hipStream_t) {
  return hipErrorLaunchFailure;
}
template hipError_t launch_bwd_d<64>(const BwdArgs&, int, int, int, hipStream_t);
template hipError_t launch_bwd_d<128>(const BwdArgs&, int, int, int, hipStream_t);

hipError_t launch_block_mask(int, int, const int32_t*, int, int, const BlockMaskArgs&, hipStream_t) {
  return hipErrorLaunchFailure;
}
hipError_t launch_fp8_fwd(const Fp8FwdArgs&, int, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_fp8_quantize(const void*, void*, uint8_t*, int, int, int, const float*, hipStream_t) {
  return hipErrorLaunchFailure;
}
hipError_t scratch_address(void**) { return hipErrorNotSupported; }
hipError_t device_cu_count(int*) { return hipErrorNotSupported; }

}  // namespace miattn
