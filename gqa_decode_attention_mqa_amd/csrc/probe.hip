// Streaming-read calibration kernel: the read rate HBM delivers to a pure
// 16-byte-load stream on this device, against which the decode kernels'
// achieved rate is read (decode attention is bound by reading the cache:
// "How To Scale Your Model", Part 7 "Transformer Inference", the passage on
// the arithmetic intensity of attention).
//
// Workgroup w reads bytes [w * slice, (w + 1) * slice) of the buffer with
// 16-byte non-temporal buffer loads (the cache policy of the K/V tiles), 256
// threads, UNROLL loads in flight per thread, and folds them with XOR into one
// word per workgroup so that no load can be dropped.
#include <hip/hip_ext.h>

#include "kernel_common.hpp"

namespace mqa {

template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_kernel(const unsigned char* buf, long long bytes, long long slice,
                                                          uint32_t* sink) {
    const long long first = (long long)blockIdx.x * slice;
    const long long n = bytes - first < slice ? bytes - first : slice;  // bytes of this workgroup (> 0)
    const __amdgpu_buffer_rsrc_t r = make_rsrc(buf + first, (int)n);
    const int step = 256 * 16;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (int off = threadIdx.x * 16; off < (int)n; off += UNROLL * step) {
        u32x4_t v[UNROLL];
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) v[j] = buffer_load_u32x4(r, off + j * step);  // past n: zeros
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) acc ^= v[j];
    }
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_stream_read(const void* buf, long long bytes, int workgroups, uint32_t* sink, hipStream_t stream,
                              hipEvent_t ev0, hipEvent_t ev1) {
    const long long slice = ((bytes + workgroups - 1) / workgroups + 15) / 16 * 16;
    const unsigned grid = (unsigned)((bytes + slice - 1) / slice);
    const auto* p = static_cast<const unsigned char*>(buf);
    if (ev0 || ev1)
        hipExtLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(256), 0, stream, ev0, ev1, 0, p, bytes, slice,
                              sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(256), 0, stream, p, bytes, slice, sink);
    return hipGetLastError();
}

}  // namespace mqa
