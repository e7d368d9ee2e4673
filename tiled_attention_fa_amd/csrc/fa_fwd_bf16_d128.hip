// Forward kernels: bf16 inputs, head dim 128.
#include "fa_fwd.inl"
#include "fa_launch.h"

namespace miattn {
template hipError_t launch_fwd_dt<128, false>(const FwdArgs&, int, int, hipStream_t);
}  // namespace miattn
