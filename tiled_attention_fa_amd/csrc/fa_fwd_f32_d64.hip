// Forward kernels: f32 inputs, head dim 64.
#include "fa_fwd.inl"
#include "fa_launch.h"

namespace miattn {
template hipError_t launch_fwd_dt<64, true>(const FwdArgs&, int, int, hipStream_t);
}  // namespace miattn
