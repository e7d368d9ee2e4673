// Backward kernels: bf16 inputs, head dim 64.
#include "fa_bwd.inl"
#include "fa_launch.h"

namespace miattn {
template hipError_t launch_bwd_d<64>(const BwdArgs&, int, int, int, hipStream_t);
}  // namespace miattn
