// Log-sum-exp merge of split-K partials (separate kernels).
//
// A sequence whose positions were cut into n chunks has, per query head, n
// normalised partial outputs O_s = (sum_{j in s} w_j v_j) / l_s (stored as
// fp16 scaled by 2^-e_s, see kernel_common.hpp) and base-2 log-sum-exps
// lse_s = m_s + log2(l_s).  With M = max_s lse_s the full result is
//     out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M),
// an exact identity of softmax over a partition of the positions.
//
// A row with T query tokens has T * Hq query rows (token i, head h); their
// partials sit at query row i * G + h % G of unit (row, h / G).
//
// Many chunks: dsplit workgroups per (row, token, query head), each merging a
// slice of D/dsplit columns with 256 threads (dsplit > 1 only while the grid
// would not cover the CUs).  With S = D/(4 dsplit) four-column slots, thread t
// owns slot t mod S and the chunks s = t div S, step 256/S, so several chunks
// are read in parallel; the per-thread sums are then added in a fixed order
// through LDS, so the result is bitwise reproducible for a plan.
#include "kernel_common.hpp"
#include "launch.hpp"

namespace mqa {

// Output row of query row g (token g / G, head g % G of kv head kvh) of row `row`.
__device__ __forceinline__ long long out_row(const CombineArgs& a, long long row, int kvh, int g) {
    const int tok = g / a.G;
    return (row * a.T + tok) * a.Hq + (long long)kvh * a.G + (g - tok * a.G);
}

// Merged rows leave as 16-byte device-scope stores (sc1) through a descriptor
// over the workgroup's rows; with the split kernel's partials stored the same
// way this measured faster than plain stores on MI355X (PaLM-shaped MQA,
// merge 4.0 against 4.3 us).
__device__ __forceinline__ void store_out16(__amdgpu_buffer_rsrc_t r, int byte_off, const f32x4_t& v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, byte_off, 0, kCachePolicyCoherent);
}

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    __shared__ float s_max[4];
    __shared__ __attribute__((aligned(16))) f32x4_t s_acc[256];
    __shared__ float s_w[256];

    const int tid = threadIdx.x;
    const long long rh = blockIdx.x / a.dsplit;  // (row * T + token) * Hq + h
    const int ds = (int)(blockIdx.x % a.dsplit);  // this workgroup's slice of d
    const int h = (int)(rh % a.Hq);
    const long long rt = rh / a.Hq;
    const long long row = rt / a.T;
    const int tok = (int)(rt % a.T);
    int b, len;
    row_extent(a.seq_lens, row, a.Lmax, &b, &len);
    const int nsplit = chunk_span(a.window, a.chunk, a.max_splits, len, 0).nsplit;
    if (nsplit <= 1) return;  // written directly by the split kernel

    const int kvh = h / a.G, g = tok * a.G + h % a.G;
    const size_t first = ((size_t)(row * a.Hkv + kvh) * a.max_splits) * a.GT + g;  // split 0
    const f32x2_t* ml = a.part_ml + first;
    const uint16_t* po = a.part_o + first * a.D;
    const size_t step = (size_t)a.GT;  // partials of consecutive splits are T * G query rows apart

    // M = max over chunks (threads stride over the chunks, then a block max)
    float m = -INFINITY;
    for (int s = tid; s < nsplit; s += 256) m = fmaxf(m, ml[s * step].x);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((tid & 63) == 0) s_max[tid >> 6] = m;
    __syncthreads();
    // A query row that sees no position in any chunk (a later token of a
    // multi-token call whose limit lies before the sequence start) has lse =
    // -inf everywhere: every weight is then 0 and the row is written as zeros.
    float M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    M = M == -INFINITY ? 0.f : M;

    const int slots = a.D / 4 / a.dsplit;  // 16-byte column slots of this workgroup's slice
    const int lanes_per_slot = 256 / slots;
    const int slot = tid % slots, sl = tid / slots;
    const int col = ds * slots + slot;     // slot in the row
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
#pragma unroll 8
    for (int s = sl; s < nsplit; s += lanes_per_slot) {
        const f32x2_t mle = ml[s * step];
        const float wgt = __builtin_amdgcn_exp2f(mle.x - M);
        const u32x2_t hv = *reinterpret_cast<const u32x2_t*>(po + s * step * a.D + 4 * col);
        acc += wgt * unpack_partial4(hv, (int)mle.y);
        wsum += wgt;
    }
    s_acc[tid] = acc;
    s_w[tid] = wsum;
    __syncthreads();
    if (sl == 0) {
        for (int j = 1; j < lanes_per_slot; ++j) {
            acc += s_acc[j * slots + slot];
            wsum += s_w[j * slots + slot];
        }
        const __amdgpu_buffer_rsrc_t ors = make_rsrc(a.out + (size_t)rh * a.D, a.D * 4);
        store_out16(ors, 16 * col, acc * (wsum > 0.f ? 1.f / wsum : 0.f));
    }
}

// Few chunks per sequence (at most S, the plan's chunk bound rounded up to
// 2, 4 or 8): one thread per (query row, 8-value column slot), 2048/D query
// rows per workgroup, all of one unit (row, kv head).  Workgroup b runs on XCD
// b mod 8; when the number of units is a multiple of 8 it takes a unit of the
// same residue, the XCD on which the split kernel ran that unit's chunks
// (map_block), so the partials it reads were written through that XCD's L2.
// Each thread issues the loads of all S chunks' {lse, e} and slot at once
// (indices clamped to the sequence's chunks, so every load is in bounds) and
// merges them in ascending chunk order, so the result is bitwise
// reproducible for a plan.
template <int D, int S>
__global__ __launch_bounds__(256) void combine_few_kernel(CombineArgs a, long long units, int blocks_per_unit) {
    constexpr int SLOTS = D / 8;
    constexpr int HPB = 256 / SLOTS;
    static_assert(S >= 2 && S <= kCombineFewMaxSplits, "chunk bound of the few-chunk combine");
    const int tid = threadIdx.x;
    const long long bx = blockIdx.x;
    long long unit;
    int j;
    if ((units & 7) == 0) {
        const long long y = bx >> 3;
        unit = (y / blocks_per_unit) * 8 + (bx & 7);
        j = (int)(y % blocks_per_unit);
    } else {
        unit = bx / blocks_per_unit;
        j = (int)(bx % blocks_per_unit);
    }
    const int g = j * HPB + tid / SLOTS;  // query row of the unit: token g / G, head kvh * G + g % G
    if (unit >= units || g >= a.GT) return;
    const int slot = tid % SLOTS;
    const long long row = unit / a.Hkv;
    const int kvh = (int)(unit % a.Hkv);
    const long long gh = out_row(a, row, kvh, g);
    int b, len;
    row_extent(a.seq_lens, row, a.Lmax, &b, &len);
    const int nsplit = chunk_span(a.window, a.chunk, a.max_splits, len, 0).nsplit;
    if (nsplit <= 1) return;  // written directly by the split kernel

    const size_t first = ((size_t)unit * a.max_splits) * a.GT + g;  // split 0
    const size_t step = (size_t)a.GT;  // partials of consecutive splits are T * G query rows apart
    f32x2_t ml[S];
    u32x4_t o[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int sc = s < nsplit ? s : nsplit - 1;
        ml[s] = a.part_ml[first + sc * step];
        o[s] = *reinterpret_cast<const u32x4_t*>(a.part_o + (first + sc * step) * D + 8 * slot);
    }
    f32x4_t r0, r1;
    merge_slot<S>(ml, o, nsplit, r0, r1);
    // the block's rows j HPB .. (up to HPB of them) are increasing output rows
    const long long gh0 = out_row(a, row, kvh, j * HPB);
    const long long ghl = out_row(a, row, kvh, min(j * HPB + HPB, a.GT) - 1);
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(a.out + (size_t)gh0 * D, (int)((ghl - gh0 + 1) * D * 4));
    const int off = (int)((gh - gh0) * D * 4) + 32 * slot;
    store_out16(ors, off, r0);
    store_out16(ors, off + 16, r1);
}

// Launch through hipExtLaunchKernelGGL when the caller asked for events
// recorded by the merge's own dispatch.
#define MQA_LAUNCH(kernel, grid, ...)                                                               \
    do {                                                                                            \
        if (ev0 || ev1)                                                                             \
            hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, stream, ev0, ev1, 0, __VA_ARGS__); \
        else                                                                                        \
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, stream, __VA_ARGS__);                \
    } while (0)

template <int D>
static void launch_few(int max_splits, const CombineArgs& a, long long units, hipStream_t stream, hipEvent_t ev0,
                       hipEvent_t ev1) {
    const int bpu = (a.GT + combine_heads_per_block(D) - 1) / combine_heads_per_block(D);
    const unsigned grid = (unsigned)(units * bpu);
    if (max_splits <= 2)
        MQA_LAUNCH((combine_few_kernel<D, 2>), grid, a, units, bpu);
    else if (max_splits <= 4)
        MQA_LAUNCH((combine_few_kernel<D, 4>), grid, a, units, bpu);
    else
        MQA_LAUNCH((combine_few_kernel<D, kCombineFewMaxSplits>), grid, a, units, bpu);
}

hipError_t launch_combine(const Plan& p, const CombineArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (p.grid_combine <= 0) return hipSuccess;
    if (p.max_splits <= kCombineFewMaxSplits) {
        const long long units = p.rows * a.Hkv;
        switch (a.D) {
            case 64: launch_few<64>(p.max_splits, a, units, stream, ev0, ev1); break;
            case 128: launch_few<128>(p.max_splits, a, units, stream, ev0, ev1); break;
            case 256: launch_few<256>(p.max_splits, a, units, stream, ev0, ev1); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        MQA_LAUNCH(combine_kernel, (unsigned)p.grid_combine, a);
    }
    return hipGetLastError();
}
#undef MQA_LAUNCH

}  // namespace mqa
