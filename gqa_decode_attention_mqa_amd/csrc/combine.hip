// Log-sum-exp merge of split-K partials.
//
// A sequence whose positions were cut into n chunks has, per query head, n
// normalised partial outputs O_s = (sum_{j in s} w_j v_j) / l_s and base-2
// log-sum-exps lse_s = m_s + log2(l_s).  With M = max_s lse_s the full result is
//     out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M),
// an exact identity of softmax over a partition of the positions.  The chunks
// are visited in ascending order, so the result is bitwise reproducible for a
// given plan.  One workgroup per (row, query head); threads run along d.
#include "kernel_common.hpp"
#include "launch.hpp"

namespace mqa {

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const long long rh = blockIdx.x;
    const int h = (int)(rh % a.Hq);
    const long long row = rh / a.Hq;
    int b, len;
    row_extent(a.seq_lens, row, a.Lmax, a.causal, &b, &len);
    const int nsplit = len > 0 ? (len + a.chunk - 1) / a.chunk : 1;
    if (nsplit <= 1) return;  // written directly by the split kernel

    const int kvh = h / a.G, g = h % a.G;
    const size_t first = ((size_t)(row * a.Hkv + kvh) * a.max_splits) * a.G + g;  // split 0
    const float* lse = a.part_lse + first;
    const float* po = a.part_o + first * a.D;
    const size_t step = (size_t)a.G;  // partials of consecutive splits are G heads apart

    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, lse[s * step]);

    float* dst = a.out + ((size_t)row * a.Hq + h) * a.D;
    for (int d = threadIdx.x; d < a.D; d += blockDim.x) {
        float acc = 0.f, wsum = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            const float wgt = __builtin_amdgcn_exp2f(lse[s * step] - M);
            acc += wgt * po[s * step * a.D + d];
            wsum += wgt;
        }
        dst[d] = acc / wsum;
    }
}

hipError_t launch_combine(const Plan& p, const CombineArgs& a, hipStream_t stream) {
    if (p.grid_combine <= 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)p.grid_combine), dim3(a.D), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mqa
