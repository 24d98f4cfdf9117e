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
#include "kernel_common.hpp"
#include "launch.hpp"

namespace mqa {

template <int D, int NG>
struct MfmaCfg {
    static constexpr int NW = 4;                         // waves per workgroup
    static constexpr int WD = D / 64;                    // waves along d in P.V
    static constexpr int WT = NW / WD;                   // waves along positions in P.V
    static constexpr int TILE = (32 * WT > 64) ? 32 * WT : 64;
    static constexpr int QKM = TILE / (16 * NW);         // 16-position M tiles per wave in q.K
    static constexpr int PVK = TILE / WT / 32;           // 32-position k-steps per wave in P.V
    static constexpr int KS = D / 32;                    // k-steps over d in q.K
    static constexpr int GP = 16 * NG;                   // heads per workgroup (padded)
    static constexpr int QLD = D + 8;                    // LDS row pitch of q (bf16)
    static constexpr int PLD = TILE + 8;                 // LDS row pitch of P^T (bf16)
    static constexpr int RED_BYTES = NW * GP * 4;
    static constexpr int Q_BYTES = GP * QLD * 2;
    static constexpr int P_BYTES = GP * PLD * 2;
    static constexpr int MERGE_BYTES = (WT - 1) * WD * 4 * NG * 4 * 64 * 4;
    static constexpr int BODY_BYTES = (Q_BYTES + P_BYTES) > MERGE_BYTES ? (Q_BYTES + P_BYTES) : MERGE_BYTES;
    static constexpr int LDS_BYTES = RED_BYTES + BODY_BYTES;
    static_assert(TILE % (16 * NW) == 0, "q.K tiles must cover the tile");
    static_assert(PVK >= 1, "each P.V wave needs a whole 32-position k-step");
    static_assert(LDS_BYTES <= 65536, "static LDS budget");
    static_assert(BODY_BYTES >= (kFusedMaxSplits + 2) * GP * 4, "fused-combine weights fit in the body");
};

template <int D, int NG>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
    using C = MfmaCfg<D, NG>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_BYTES];
    float* red = reinterpret_cast<float*>(smem);
    uint16_t* qs = reinterpret_cast<uint16_t*>(smem + C::RED_BYTES);
    uint16_t* ps = qs + C::GP * C::QLD;
    float* merge = reinterpret_cast<float*>(smem + C::RED_BYTES);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
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
    const int p0 = s * a.chunk;
    if (s > 0 && p0 >= len) return;  // whole workgroup: this chunk is past the end
    const int p1 = min(p0 + a.chunk, len);
    const int nsplit = len > 0 ? (len + a.chunk - 1) / a.chunk : 1;

    // Stage this block's query heads (bf16, zero rows past the group) in LDS.
    const uint16_t* qrow = a.q + ((size_t)row * a.Hq + (size_t)kvh * a.G + g0) * D;
    for (int c = tid; c < C::GP * (D / 8); c += 256) {
        const int g = c / (D / 8), dc = c % (D / 8);
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (g < gcnt) val = load_u32x4(qrow + (size_t)g * D + dc * 8);
        *reinterpret_cast<u32x4_t*>(qs + g * C::QLD + dc * 8) = val;
    }

    const size_t pos_stride = (size_t)a.Hkv * D;  // elements between consecutive positions
    const uint16_t* kbase = a.k + ((size_t)b * a.Lmax * a.Hkv + kvh) * D;
    const uint16_t* vbase = a.v + ((size_t)b * a.Lmax * a.Hkv + kvh) * D;
    const int ds = w % C::WD, ts = w / C::WD;
    const int vcol = 64 * ds + 4 * li;        // this lane's 4 V columns in P.V
    const float qk = a.qk_log2;
    const int last = p1 - 1;                  // loads past the end re-read this row

    float m_run[NG], l_run[NG];
    f32x4_t oacc[4][NG];
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        m_run[n] = -INFINITY;
        l_run[n] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) oacc[j][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Loads are unconditional: a position at or past p1 is clamped to the last
    // valid row.  Its logit is masked to -inf (so its weight is exactly 0 and the
    // clamped V row adds nothing); padding is never read.
    auto load_tile = [&](int tile0, u32x4_t (&kr)[C::QKM][C::KS], u32x2_t (&vr)[C::PVK][8]) {
#pragma unroll
        for (int mq = 0; mq < C::QKM; ++mq) {
            const int t = min(tile0 + 16 * (w * C::QKM + mq) + li, last);
            const uint16_t* src = kbase + (size_t)t * pos_stride + kg * 8;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) kr[mq][ks] = load_nt_u32x4(src + ks * 32);
        }
#pragma unroll
        for (int kk = 0; kk < C::PVK; ++kk) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = min(tile0 + ts * (C::TILE / C::WT) + 32 * kk + 8 * kg + e, last);
                vr[kk][e] = load_nt_u32x2(vbase + (size_t)t * pos_stride + vcol);
            }
        }
    };

    auto compute_tile = [&](int tile0, const u32x4_t (&kr)[C::QKM][C::KS], const u32x2_t (&vr)[C::PVK][8]) {
        // ---- S^T = K q^T
        f32x4_t sacc[C::QKM][NG];
#pragma unroll
        for (int mq = 0; mq < C::QKM; ++mq)
#pragma unroll
            for (int n = 0; n < NG; ++n) sacc[mq][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
            for (int n = 0; n < NG; ++n) {
                const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(qs + (16 * n + li) * C::QLD + ks * 32 + kg * 8);
#pragma unroll
                for (int mq = 0; mq < C::QKM; ++mq) sacc[mq][n] = mfma_16x16x32_bf16(kr[mq][ks], bq, sacc[mq][n]);
            }
        }
        // ---- scale, mask the ragged tail, per-wave maximum per head
        float wmax[NG];
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            float mx = -INFINITY;
#pragma unroll
            for (int mq = 0; mq < C::QKM; ++mq)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = tile0 + 16 * (w * C::QKM + mq) + 4 * kg + r;
                    const float val = (t < p1) ? sacc[mq][n][r] * qk : -INFINITY;
                    sacc[mq][n][r] = val;
                    mx = fmaxf(mx, val);
                }
            mx = fmaxf(mx, shfl_xor_f32(mx, 16));
            mx = fmaxf(mx, shfl_xor_f32(mx, 32));
            wmax[n] = mx;
        }
        if (kg == 0) {
#pragma unroll
            for (int n = 0; n < NG; ++n) red[w * C::GP + 16 * n + li] = wmax[n];
        }
        __syncthreads();
        float alpha[NG];
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            float tmax = red[16 * n + li];
#pragma unroll
            for (int ww = 1; ww < C::NW; ++ww) tmax = fmaxf(tmax, red[ww * C::GP + 16 * n + li]);
            const float m_new = fmaxf(m_run[n], tmax);
            alpha[n] = __builtin_amdgcn_exp2f(m_run[n] - m_new);
            m_run[n] = m_new;
        }
        // ---- P = exp2(S - m), bf16, transposed into LDS; row sums of the rounded values
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            float lsum = 0.f;
#pragma unroll
            for (int mq = 0; mq < C::QKM; ++mq) {
                uint32_t pb[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pb[r] = f32_to_bf16_bits(__builtin_amdgcn_exp2f(sacc[mq][n][r] - m_run[n]));
                    lsum += bf16_bits_to_f32(pb[r]);
                }
                u32x2_t packed = {pack_bf16x2(pb[0], pb[1]), pack_bf16x2(pb[2], pb[3])};
                *reinterpret_cast<u32x2_t*>(ps + (16 * n + li) * C::PLD + 16 * (w * C::QKM + mq) + 4 * kg) = packed;
            }
            l_run[n] = l_run[n] * alpha[n] + lsum;
        }
        __syncthreads();
        // ---- O^T = alpha * O^T + V^T P^T
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int n = 0; n < NG; ++n) oacc[j][n] = oacc[j][n] * alpha[n];
#pragma unroll
        for (int kk = 0; kk < C::PVK; ++kk) {
            u32x4_t va[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x2_t r0 = vr[kk][2 * c], r1 = vr[kk][2 * c + 1];
                va[0][c] = perm_b32(r1.x, r0.x, kPermLoHalves);
                va[1][c] = perm_b32(r1.x, r0.x, kPermHiHalves);
                va[2][c] = perm_b32(r1.y, r0.y, kPermLoHalves);
                va[3][c] = perm_b32(r1.y, r0.y, kPermHiHalves);
            }
#pragma unroll
            for (int n = 0; n < NG; ++n) {
                const u32x4_t pbv = *reinterpret_cast<const u32x4_t*>(
                    ps + (16 * n + li) * C::PLD + ts * (C::TILE / C::WT) + 32 * kk + 8 * kg);
#pragma unroll
                for (int j = 0; j < 4; ++j) oacc[j][n] = mfma_16x16x32_bf16(va[j], pbv, oacc[j][n]);
            }
        }
    };

    // Two register stages: while a tile is computed, the next one is in flight.
    if (p0 < p1) {
        u32x4_t kA[C::QKM][C::KS], kB[C::QKM][C::KS];
        u32x2_t vA[C::PVK][8], vB[C::PVK][8];
        load_tile(p0, kA, vA);
        __syncthreads();  // q staged
        int tile0 = p0;
        while (true) {
            load_tile(tile0 + C::TILE, kB, vB);
            compute_tile(tile0, kA, vA);
            tile0 += C::TILE;
            if (tile0 >= p1) break;
            load_tile(tile0 + C::TILE, kA, vA);
            compute_tile(tile0, kB, vB);
            tile0 += C::TILE;
            if (tile0 >= p1) break;
        }
    }

    // ---- epilogue: row sums across lane groups and waves, merge P.V position slices
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        float l = l_run[n];
        l += shfl_xor_f32(l, 16);
        l += shfl_xor_f32(l, 32);
        l_run[n] = l;
    }
    __syncthreads();  // every wave is done with q, P and the maxima
    if (kg == 0) {
#pragma unroll
        for (int n = 0; n < NG; ++n) red[w * C::GP + 16 * n + li] = l_run[n];
    }
    if (C::WT > 1 && ts > 0) {
        float* dst = merge + (size_t)((ts - 1) * C::WD + ds) * (4 * NG * 4 * 64);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int n = 0; n < NG; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[((j * NG + n) * 4 + r) * 64 + lane] = oacc[j][n][r];
    }
    __syncthreads();

    const bool direct = nsplit == 1;
    if (ts == 0) {
        float inv_l[NG], lse2[NG];
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            float L = 0.f;
#pragma unroll
            for (int ww = 0; ww < C::NW; ++ww) L += red[ww * C::GP + 16 * n + li];
            inv_l[n] = L > 0.f ? 1.f / L : 0.f;
            lse2[n] = m_run[n] + __log2f(L);
        }
        if (C::WT > 1) {
#pragma unroll
            for (int tt = 1; tt < C::WT; ++tt) {
                const float* src = merge + (size_t)((tt - 1) * C::WD + ds) * (4 * NG * 4 * 64);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int n = 0; n < NG; ++n)
#pragma unroll
                        for (int r = 0; r < 4; ++r) oacc[j][n][r] += src[((j * NG + n) * 4 + r) * 64 + lane];
            }
        }
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            const int g = 16 * n + li;
            if (g >= gcnt) continue;
            const int gh = g0 + g;  // head index inside the group
            float* dst;
            if (direct)
                dst = a.out + ((size_t)row * a.Hq + (size_t)kvh * a.G + gh) * D;
            else
                dst = a.part_o + (((size_t)unit * a.max_splits + s) * a.G + gh) * D;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 64 * ds + 16 * kg + 4 * r;
                f32x4_t o4 = {oacc[0][n][r] * inv_l[n], oacc[1][n][r] * inv_l[n],
                              oacc[2][n][r] * inv_l[n], oacc[3][n][r] * inv_l[n]};
                *reinterpret_cast<f32x4_t*>(dst + d) = o4;
            }
            if (!direct && ds == 0 && kg == 0)
                a.part_lse[((size_t)unit * a.max_splits + s) * a.G + gh] = lse2[n];
        }
    }
    if (direct || !a.fused) return;
    // ---- fused combine: the last chunk of this (row, kv head, head block) merges all partials
    int* flag = reinterpret_cast<int*>(red);
    if (!arrive_last(a.counters + unit * gridDim.y + blockIdx.y, nsplit, flag)) return;
    float* wts = reinterpret_cast<float*>(smem + C::RED_BYTES);
    fused_combine(a, unit, nsplit, g0, gcnt, a.out + ((size_t)row * a.Hq + (size_t)kvh * a.G + g0) * D,
                  wts, C::GP);
}

template <int D>
static hipError_t launch_mfma_d(const Plan& p, const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)p.grid_main, (unsigned)p.head_blocks);
    const dim3 block(256);
    switch (p.heads_per_block / 16) {
        case 1: hipLaunchKernelGGL((decode_mfma_kernel<D, 1>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((decode_mfma_kernel<D, 2>), grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL((decode_mfma_kernel<D, 3>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((decode_mfma_kernel<D, 4>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_mfma(const Plan& p, const DecodeArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 64: return launch_mfma_d<64>(p, a, stream);
        case 128: return launch_mfma_d<128>(p, a, stream);
        case 256: return launch_mfma_d<256>(p, a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mqa
