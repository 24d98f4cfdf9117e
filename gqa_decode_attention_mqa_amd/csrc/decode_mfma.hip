// Split-K decode attention on bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// For groups of at least 16 query heads per key/value head the two products
// of a decode step are dense enough for matrix tiles: one workgroup owns
// (query row, kv head, chunk of positions, block of up to 64 heads) and reads
// each K/V row of its chunk exactly once for all of its heads.  This is the
// single-device form of the batch-sharded multiquery layout of "Efficiently
// Scaling Transformer Inference", section 3.4, "Attention Layer
// Partitioning": attention for a sequence is computed where its cache lives,
// and the shared key/value head is never replicated or re-read per query head.
//
// Per tile of TILE positions (4 waves, 256 threads):
//   * S^T = K q^T: each wave takes 16 (or 32) positions as the M dimension;
//     its K rows load straight from HBM into the A-operand layout (row = lane
//     mod 16, 8 contiguous d per lane = one 128-bit load); q^T is the B operand,
//     read from LDS.  The accumulator puts head g = lane mod 16 in every lane
//     group, so each lane holds 4 positions of one head.
//   * online softmax in base 2 (log2(e) folded into the logit scale): the tile
//     maximum per head is combined across waves through LDS, P = exp2(S - m)
//     is rounded to bf16 and written to LDS transposed ([head][position]).
//   * O^T += V^T P^T: each wave owns 64 columns of d (and, for D < 256, a slice
//     of the tile's positions).  V rows are loaded as 8-byte pieces and
//     transposed in registers with v_perm_b32 into the A operand (row = d,
//     8 consecutive positions per lane); P^T is the B operand from LDS.  The
//     accumulator's column is again the head, so the rescale by
//     exp2(m_old - m_new) happens in-lane.
// The chunk ends by normalising; a sequence that fits in one chunk writes its
// output directly, otherwise the chunk writes O/l and its base-2 log-sum-exp
// for the combine kernel.
#include <atomic>
#include <type_traits>

#include "kernel_common.hpp"
#include "launch.hpp"

namespace mqa {

template <int D, int NG>
struct MfmaCfg {
    static constexpr int NW = 4;             // waves per workgroup, each independent in the main loop
    // 16-row S^T tiles per step: two (P.V on 16x16x32, 8 k-slots) while the
    // registers allow, one (P.V on 16x16x16, 4 k-slots) for D = 256.
    static constexpr int MQ = (D >= 256) ? 1 : 2;
    static constexpr int STEP = 16 * MQ;     // positions a wave takes per step
    static constexpr int KSL = 4 * MQ;       // k-slots of the P.V tile per lane group
    static constexpr int KS = D / 32;        // k-steps over d in q.K
    static constexpr int DPL = D / 16;       // V columns per lane = M tiles of O^T
    static constexpr int GP = 16 * NG;       // heads per workgroup (padded)
    static constexpr int QLD = D + 8;        // LDS row pitch of q (bf16)
    static constexpr int ACC = DPL * NG;     // O^T accumulator tiles per lane (4 floats each)
    static constexpr int Q_BYTES = GP * QLD * 2;
    static constexpr int OLD = D + 4;                        // LDS row pitch of an O exchange region (fp32)
    static constexpr int REGION_BYTES = GP * OLD * 4;        // one wave's O, row-major [head][d]
    static constexpr int ML_BYTES = 2 * NW * GP * 4;        // running max and row sum per wave
    static constexpr int BODY_BYTES = (2 * REGION_BYTES > Q_BYTES) ? 2 * REGION_BYTES : Q_BYTES;
    static constexpr int LDS_BYTES = ML_BYTES + BODY_BYTES;
    static_assert(D % 64 == 0, "head size");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
    static_assert(BODY_BYTES >= (kFusedMaxSplits + 2) * GP * 4, "fused-combine weights fit in the body");
};

template <int D, int NG>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
    using C = MfmaCfg<D, NG>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float* m_lds = reinterpret_cast<float*>(smem);           // [NW][GP]
    float* l_lds = m_lds + C::NW * C::GP;                    // [NW][GP]
    unsigned char* body = smem + C::ML_BYTES;
    uint16_t* qs = reinterpret_cast<uint16_t*>(body);        // q, during the main loop
    float* region0 = reinterpret_cast<float*>(body);         // O^T exchange, after it
    float* region1 = reinterpret_cast<float*>(body + C::REGION_BYTES);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (wave-uniform)
    const int li = lane & 15, kg = lane >> 4;

    long long unit;
    int s;
    map_block(blockIdx.x, a.units, a.max_splits, &unit, &s);
    const int kvh = (int)(unit % a.Hkv);
    const long long row = unit / a.Hkv;
    const int g0 = blockIdx.y * C::GP;
    const int gcnt = min(C::GP, a.G - g0);

    int b, len;
    row_extent(a.seq_lens, row, a.Lmax, a.causal, &b, &len);
    // Workgroup-uniform; stated so the compiler keeps them (and the buffer
    // descriptors built from them) in scalar registers.
    b = __builtin_amdgcn_readfirstlane(b);
    len = __builtin_amdgcn_readfirstlane(len);
    const int p0 = s * a.chunk;
    if (s > 0 && p0 >= len) return;  // whole workgroup: this chunk is past the end
    const int p1 = min(p0 + a.chunk, len);
    const int nsplit = len > 0 ? (len + a.chunk - 1) / a.chunk : 1;

    const size_t pos_stride = (size_t)a.Hkv * D;  // elements between consecutive positions
    const int rowbytes = (int)(pos_stride * 2);
    const uint16_t* kseq = a.k + ((size_t)b * a.Lmax * a.Hkv + kvh) * D;  // position 0 of this head
    const uint16_t* vseq = a.v + ((size_t)b * a.Lmax * a.Hkv + kvh) * D;
    const float qk = a.qk_log2;

    // Lane offsets inside a step (loop invariant).  The S^T accumulator of M
    // tile mq gives lane group kg the positions 16*mq + 4*kg + r, r < 4; these
    // positions are the k-slots (element e = 4*mq + r) of the P^T operand of
    // P.V, so V rows are loaded in the same order.
    constexpr int MQ = C::MQ, KSL = C::KSL;
    using pv_t = typename std::conditional<MQ == 2, u32x4_t, u32x2_t>::type;
    const int koff0 = li * rowbytes + kg * 16;                 // + 16*mq*rowbytes, + 64*ks
    int voff[KSL];
#pragma unroll
    for (int e = 0; e < KSL; ++e) voff[e] = (16 * (e / 4) + 4 * kg + (e % 4)) * rowbytes + li * (C::DPL * 2);

    // K rows of one step: [mq][ks] -> 16 bytes of row 16*mq + li, d = 32*ks + 8*kg ...
    u32x4_t kr[MQ][C::KS];
    // V rows of one step: KSL rows (k-slots) x DPL columns d = DPL*li + c.
    constexpr int VW = C::DPL / 2;  // dwords of V per row per lane
    uint32_t vr[KSL][VW];

    auto load_k = [&](int st) {
        const int rows = max(0, min(C::STEP, p1 - st));
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(kseq + (size_t)st * pos_stride, rows * rowbytes);
#pragma unroll
        for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) kr[mq][ks] = buffer_load_u32x4(rs, koff0 + 16 * mq * rowbytes + 64 * ks);
    };
    auto load_v = [&](int st) {
        const int rows = max(0, min(C::STEP, p1 - st));
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(vseq + (size_t)st * pos_stride, rows * rowbytes);
#pragma unroll
        for (int e = 0; e < KSL; ++e) {
            if constexpr (VW >= 4) {
#pragma unroll
                for (int j = 0; j < VW / 4; ++j) {
                    const u32x4_t t4 = buffer_load_u32x4(rs, voff[e] + 16 * j);
                    vr[e][4 * j] = t4.x;
                    vr[e][4 * j + 1] = t4.y;
                    vr[e][4 * j + 2] = t4.z;
                    vr[e][4 * j + 3] = t4.w;
                }
            } else {
                const u32x2_t t2 = buffer_load_u32x2(rs, voff[e]);
                vr[e][0] = t2.x;
                vr[e][1] = t2.y;
            }
        }
    };

    // q is fetched first and the first K/V step right behind it: the q staging
    // below then waits only for q (loads complete in order), while K/V stream in.
    constexpr int QV = (C::GP * (D / 8) + 255) / 256;  // 16-byte pieces of q per thread
    const uint16_t* qrow = a.q + ((size_t)row * a.Hq + (size_t)kvh * a.G + g0) * D;
    u32x4_t qv[QV];
#pragma unroll
    for (int i = 0; i < QV; ++i) {
        const int c = tid + 256 * i;
        const int g = c / (D / 8), dc = c % (D / 8);
        qv[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (c < C::GP * (D / 8) && g < gcnt) qv[i] = load_u32x4(qrow + (size_t)g * D + dc * 8);
    }
    int st = p0 + C::STEP * w;
    load_k(st);
    load_v(st);
#pragma unroll
    for (int i = 0; i < QV; ++i) {
        const int c = tid + 256 * i;
        if (c < C::GP * (D / 8))
            *reinterpret_cast<u32x4_t*>(qs + (c / (D / 8)) * C::QLD + (c % (D / 8)) * 8) = qv[i];
    }
    __syncthreads();

    float m_run[NG], l_run[NG];
    f32x4_t oacc[C::DPL][NG];
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        m_run[n] = -INFINITY;
        l_run[n] = 0.f;
#pragma unroll
        for (int j = 0; j < C::DPL; ++j) oacc[j][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // ---- main loop: this wave's steps st, st + 4*STEP, ...; no cross-wave sync
    while (st < p1) {
        // Keeps the q^T reads below inside the loop: hoisted, they would pin
        // KS * NG * 4 registers for the whole loop (96 for 48 heads of 256).
        asm volatile("" ::: "memory");
        const int nxt = st + C::NW * C::STEP;
        // S^T = K q^T
        f32x4_t sacc[MQ][NG];
#pragma unroll
        for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
            for (int n = 0; n < NG; ++n) sacc[mq][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
            for (int n = 0; n < NG; ++n) {
                const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(qs + (16 * n + li) * C::QLD + ks * 32 + kg * 8);
#pragma unroll
                for (int mq = 0; mq < MQ; ++mq) sacc[mq][n] = mfma_16x16x32_bf16(kr[mq][ks], bq, sacc[mq][n]);
            }
        }
        load_k(nxt);  // the next step's K streams in under softmax and P.V

        // scale to base-2 units; mask past the end (last step only)
#pragma unroll
        for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
            for (int n = 0; n < NG; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[mq][n][r] *= qk;
        if (st + C::STEP > p1) {
#pragma unroll
            for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool ok = st + 16 * mq + 4 * kg + r < p1;
#pragma unroll
                    for (int n = 0; n < NG; ++n) sacc[mq][n][r] = ok ? sacc[mq][n][r] : -INFINITY;
                }
        }
        // online softmax with lazy rescaling; P^T operand built in registers
        pv_t pb[NG];
        float alpha[NG];
        bool any_rescale = false;
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            float mx = fmaxf(fmaxf(sacc[0][n][0], sacc[0][n][1]), fmaxf(sacc[0][n][2], sacc[0][n][3]));
#pragma unroll
            for (int mq = 1; mq < MQ; ++mq)
                mx = fmaxf(mx, fmaxf(fmaxf(sacc[mq][n][0], sacc[mq][n][1]), fmaxf(sacc[mq][n][2], sacc[mq][n][3])));
            mx = max_xor32(max_xor16(mx));
            const bool moved = mx > m_run[n] + kRescaleSlack;
            alpha[n] = moved ? __builtin_amdgcn_exp2f(m_run[n] - mx) : 1.f;
            m_run[n] = moved ? mx : m_run[n];
            any_rescale |= moved;
            float lsum = 0.f;
#pragma unroll
            for (int mq = 0; mq < MQ; ++mq) {
                const uint32_t lo = pack2_bf16_rne(__builtin_amdgcn_exp2f(sacc[mq][n][0] - m_run[n]),
                                                   __builtin_amdgcn_exp2f(sacc[mq][n][1] - m_run[n]));
                const uint32_t hi = pack2_bf16_rne(__builtin_amdgcn_exp2f(sacc[mq][n][2] - m_run[n]),
                                                   __builtin_amdgcn_exp2f(sacc[mq][n][3] - m_run[n]));
                pb[n][2 * mq] = lo;
                pb[n][2 * mq + 1] = hi;
                lsum += (bf16_lo_f32(lo) + bf16_hi_f32(lo)) + (bf16_lo_f32(hi) + bf16_hi_f32(hi));
            }
            l_run[n] = l_run[n] * alpha[n] + lsum;
        }
        if (__any(any_rescale)) {
#pragma unroll
            for (int j = 0; j < C::DPL; ++j)
#pragma unroll
                for (int n = 0; n < NG; ++n) oacc[j][n] = oacc[j][n] * alpha[n];
        }
        // O^T += V^T P^T: column c of this lane's V rows is M tile c (row li <-> d = DPL*li + c)
#pragma unroll
        for (int wd = 0; wd < VW; ++wd) {
            pv_t va_even, va_odd;
#pragma unroll
            for (int m = 0; m < KSL / 2; ++m) {
                va_even[m] = perm_b32(vr[2 * m + 1][wd], vr[2 * m][wd], kPermLoHalves);
                va_odd[m] = perm_b32(vr[2 * m + 1][wd], vr[2 * m][wd], kPermHiHalves);
            }
#pragma unroll
            for (int n = 0; n < NG; ++n) {
                oacc[2 * wd][n] = mfma_pv(va_even, pb[n], oacc[2 * wd][n]);
                oacc[2 * wd + 1][n] = mfma_pv(va_odd, pb[n], oacc[2 * wd + 1][n]);
            }
        }
        load_v(nxt);
        st = nxt;
    }

    // ---- merge the four waves' (m, l, O) by log-sum-exp, through LDS
#pragma unroll
    for (int n = 0; n < NG; ++n) l_run[n] = sum_xor32(sum_xor16(l_run[n]));  // whole wave, head li
    if (kg == 0) {
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            m_lds[w * C::GP + 16 * n + li] = m_run[n];
            l_lds[w * C::GP + 16 * n + li] = l_run[n];
        }
    }
    // Row-major exchange: accumulator (c, n, r) of lane (li, kg) is head
    // 16*n + li, columns DPL*(4*kg + r) + c, so each (n, r) is DPL consecutive
    // floats written or read as 16-byte pieces.
    auto region_ptr = [&](float* reg, int n, int r, int q4) {
        return reinterpret_cast<f32x4_t*>(reg + (16 * n + li) * C::OLD + C::DPL * (4 * kg + r) + 4 * q4);
    };
    auto store_region = [&](float* reg, const float* scale) {
#pragma unroll
        for (int n = 0; n < NG; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int q4 = 0; q4 < C::DPL / 4; ++q4)
                    *region_ptr(reg, n, r, q4) = f32x4_t{oacc[4 * q4][n][r], oacc[4 * q4 + 1][n][r],
                                                         oacc[4 * q4 + 2][n][r], oacc[4 * q4 + 3][n][r]} * scale[n];
    };
    __syncthreads();  // all waves left the main loop: q is dead, regions may overwrite it
    if (w >= 2) {
        float ones[NG];
#pragma unroll
        for (int n = 0; n < NG; ++n) ones[n] = 1.f;
        store_region(w == 2 ? region0 : region1, ones);
    }
    __syncthreads();
    if (w < 2) {
        // wave w absorbs wave w + 2
        const float* reg = w == 0 ? region0 : region1;
        float sa[NG], sb[NG];
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            const float mo = m_lds[(w + 2) * C::GP + 16 * n + li];
            const float lo = l_lds[(w + 2) * C::GP + 16 * n + li];
            const float M = fmaxf(m_run[n], mo);
            sa[n] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[n] - M);
            sb[n] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - M);
            l_run[n] = sa[n] * l_run[n] + sb[n] * lo;
            m_run[n] = M;
        }
#pragma unroll
        for (int n = 0; n < NG; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int q4 = 0; q4 < C::DPL / 4; ++q4) {
                    const f32x4_t o = *region_ptr(const_cast<float*>(reg), n, r, q4);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        oacc[4 * q4 + c][n][r] = sa[n] * oacc[4 * q4 + c][n][r] + sb[n] * o[c];
                }
        if (kg == 0) {
#pragma unroll
            for (int n = 0; n < NG; ++n) {
                m_lds[w * C::GP + 16 * n + li] = m_run[n];
                l_lds[w * C::GP + 16 * n + li] = l_run[n];
            }
        }
    }
    __syncthreads();
    // Waves 0 and 1 hold the pairs (0,2) and (1,3): each writes its share of
    // the normalised result, 2^(m_w - M) / L * O_w, to its own region.
    float lse2[NG], scale[NG];
    if (w < 2) {
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            const int g = 16 * n + li;
            const float m0 = m_lds[g], m1 = m_lds[C::GP + g];
            const float M = fmaxf(m0, m1);
            const float s0 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - M);
            const float s1 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
            const float L = s0 * l_lds[g] + s1 * l_lds[C::GP + g];
            const float inv = L > 0.f ? 1.f / L : 0.f;
            scale[n] = (w == 0 ? s0 : s1) * inv;
            lse2[n] = M + __log2f(L);
        }
    }
    __syncthreads();  // m_lds / l_lds have been read; regions 0 and 1 are free
    if (w < 2) {
        store_region(w == 0 ? region0 : region1, scale);
        if (w == 0 && kg == 0) {
#pragma unroll
            for (int n = 0; n < NG; ++n) m_lds[16 * n + li] = lse2[n];
        }
    }
    __syncthreads();

    // ---- store: every thread, contiguous rows (region0 + region1)
    const bool direct = nsplit == 1;
    for (int idx = tid; idx < gcnt * (D / 4); idx += 256) {
        const int g = idx / (D / 4), d = 4 * (idx % (D / 4));
        const f32x4_t o4 = *reinterpret_cast<const f32x4_t*>(region0 + g * C::OLD + d) +
                           *reinterpret_cast<const f32x4_t*>(region1 + g * C::OLD + d);
        const int gh = g0 + g;
        if (direct) {
            *reinterpret_cast<f32x4_t*>(a.out + ((size_t)row * a.Hq + (size_t)kvh * a.G + gh) * D + d) = o4;
        } else {
            const size_t part = ((size_t)unit * a.max_splits + s) * a.G + gh;
            *reinterpret_cast<f32x4_t*>(a.part_o + part * D + d) = o4;
            if (d == 0) a.part_lse[part] = m_lds[g];
        }
    }
    if (direct || !a.fused) return;
    // ---- fused combine: the last chunk of this (row, kv head, head block) merges all partials
    int* flag = reinterpret_cast<int*>(m_lds);
    __syncthreads();  // m_lds is reused as the arrival flag
    if (!arrive_last(a.counters + unit * gridDim.y + blockIdx.y, nsplit, flag)) return;
    float* wts = reinterpret_cast<float*>(body);
    fused_combine(a, unit, nsplit, g0, gcnt, a.out + ((size_t)row * a.Hq + (size_t)kvh * a.G + g0) * D,
                  wts, C::GP);
}

template <int D, int NG>
static hipError_t launch_one(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                             hipEvent_t ev1) {
    constexpr int lds = MfmaCfg<D, NG>::LDS_BYTES;
    if (lds > 64 * 1024) {
        // More than 64 KB of LDS must be opted into, once per device.
        static std::atomic<uint64_t> done_mask{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = 1ull << (dev & 63);
        if (!(done_mask.load() & bit)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_mfma_kernel<D, NG>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
            done_mask.fetch_or(bit);
        }
    }
    const dim3 grid((unsigned)p.grid_main, (unsigned)p.head_blocks);
    const dim3 block(256);
    if (ev0 || ev1) {
        // The dispatch packet itself records the two events, so their interval is
        // the kernel's execution time (no launch or queueing overhead).
        hipExtLaunchKernelGGL((decode_mfma_kernel<D, NG>), grid, block, lds, stream, ev0, ev1, 0, a);
    } else {
        hipLaunchKernelGGL((decode_mfma_kernel<D, NG>), grid, block, lds, stream, a);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_mfma_d(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                                hipEvent_t ev1) {
    // Groups of more than 16 heads go to the one-wave-per-16-heads kernel.
    if (p.heads_per_block != 16) return hipErrorInvalidValue;
    return launch_one<D, 1>(p, a, stream, ev0, ev1);
}

hipError_t launch_decode_mfma(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1) {
    switch (a.D) {
        case 64: return launch_mfma_d<64>(p, a, stream, ev0, ev1);
        case 128: return launch_mfma_d<128>(p, a, stream, ev0, ev1);
        case 256: return launch_mfma_d<256>(p, a, stream, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mqa
