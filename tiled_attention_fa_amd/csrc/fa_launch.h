// Host-side launchers implemented in the .hip translation units.
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/libmiattn.h"
#include "fa_args.h"

namespace miattn {

template <int D, bool F32>
hipError_t launch_fwd_dt(const FwdArgs& a, int mask, int mod, hipStream_t st);

// phases: bit 1 delta, bit 2 dK/dV, bit 4 dQ.
template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, int mask, int mod, int phases, hipStream_t st);

hipError_t launch_block_mask(int mask_kind, int window, const int32_t* doc_ids, int Sq, int Skv,
                             const BlockMaskArgs& m, hipStream_t st);

hipError_t launch_fp8_fwd(const Fp8FwdArgs& a, int mask, hipStream_t st);
hipError_t launch_fp8_quantize(const void* x, void* x8, uint8_t* scales, int rows, int S, int D, const float* signs,
                               hipStream_t st);

// Size of the library's fixed device scratch (fa_scratch.hip): the backward
// workspace of fa_bwd_noalloc, two [B][Hq][Sq] float arrays, i.e. up to
// 2^21 query rows (B * Hq * Sq).
constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;

// Device address of the current device's copy of the scratch array, looked
// up once per device (the first call with that device current) and cached.
hipError_t scratch_address(void** ptr);

// Compute units of the current device (the size of persistent grids),
// looked up once per device and cached.
hipError_t device_cu_count(int* n);

// Keys per forward step for each instantiation.
constexpr int fwd_kv_step(bool f32) { return f32 ? 32 : 64; }

}  // namespace miattn
