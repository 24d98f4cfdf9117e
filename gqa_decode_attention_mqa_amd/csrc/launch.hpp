// Kernel launchers (defined in the .hip files, called by the C ABI layer).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kernel_common.hpp"
#include "plan.hpp"

namespace mqa {

// Split-K kernel on matrix cores: one wave per 16 query heads, K/V streamed
// through an LDS ring.  When ev0/ev1 are non-null the dispatch itself records
// them around the kernel.
hipError_t launch_decode_mfma(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1);
// Split-K kernel on the vector ALU (groups of up to 8 heads per workgroup).
hipError_t launch_decode_valu(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1);
// Log-sum-exp merge of the per-chunk partials of split sequences; ev0/ev1 as
// above, recorded around the merge kernel.
hipError_t launch_combine(const Plan& p, const CombineArgs& a, hipStream_t stream, hipEvent_t ev0 = nullptr,
                          hipEvent_t ev1 = nullptr);
// Causal prefill on matrix cores: prefill_rows(D) query rows of one (sequence,
// kv head) per workgroup, the causal prefix streamed through an LDS ring.
hipError_t launch_prefill_mfma(const Plan& p, const PrefillArgs& a, hipStream_t stream);
// Streaming-read calibration: `workgroups` workgroups each read one
// contiguous slice of `bytes` bytes (a multiple of 16) and write one word to
// sink[workgroup].
hipError_t launch_stream_read(const void* buf, long long bytes, int workgroups, uint32_t* sink, hipStream_t stream,
                              hipEvent_t ev0, hipEvent_t ev1);

}  // namespace mqa
