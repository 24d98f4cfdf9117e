// Kernel launchers (defined in the .hip files, called by the C ABI layer).
#pragma once

#include <hip/hip_runtime.h>

#include "kernel_common.hpp"
#include "plan.hpp"

namespace mqa {

// Split-K kernel on matrix cores (any group size; 16 heads per tile).
hipError_t launch_decode_mfma(const Plan& p, const DecodeArgs& a, hipStream_t stream);
// Split-K kernel on the vector ALU (groups of up to 8 heads per workgroup).
hipError_t launch_decode_valu(const Plan& p, const DecodeArgs& a, hipStream_t stream);
// Log-sum-exp merge of the per-chunk partials of split sequences.
hipError_t launch_combine(const Plan& p, const CombineArgs& a, hipStream_t stream);

}  // namespace mqa
