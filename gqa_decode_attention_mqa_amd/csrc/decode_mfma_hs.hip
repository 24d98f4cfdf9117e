// Split-K decode attention on bf16 matrix cores, one wave per 16 query heads.
//
// For large groups (more than 16 query heads per key/value head, e.g. the
// 48-head multiquery attention of PaLM 540B in "Efficiently Scaling
// Transformer Inference", section 3.4, "Attention Layer Partitioning") a
// workgroup of NG waves owns (query row, kv head, chunk of positions, block of
// 16*NG heads).  Wave w owns heads 16w .. 16w+15 for every position of the
// chunk, so no two waves ever need to merge softmax state.  The chunk's K and
// V rows are read from HBM exactly once per workgroup into an LDS ring of
// STAGES tiles of 32 positions, with direct buffer-to-LDS loads (no registers
// hold data in flight); every wave then reads the whole tile from LDS.
//
// Per tile, in each wave:
//   * S^T = K q^T on 16x16x32 bf16 tiles: A = two 16-row K tiles (read from
//     LDS), B = this wave's q^T (registers).  Head g = lane mod 16.
//   * base-2 online softmax with lazy rescaling; the two S^T accumulators are
//     exactly the 8 k-slots per lane of the P^T operand of P.V.
//   * O^T += V^T P^T on 16x16x32 tiles: V rows read from LDS and transposed
//     in registers with v_perm_b32 (row = d, 8 positions per lane).
// LDS layout of a tile: row t of D bf16 = D/8 chunks of 16 bytes; chunk c of
// row t sits in slot c ^ (t mod 8).  The direct loads realise the swizzle by
// choosing, for each lane's 16-byte LDS slot, the global chunk that belongs
// there.  Rows at or past the end of the chunk are out of the buffer range and
// arrive as zeros; their logits are masked, so padding is never read.
#include <atomic>

#include "kernel_common.hpp"
#include "launch.hpp"

namespace mqa {

template <int D, int NG>
struct HsCfg {
    static constexpr int NW = NG;                    // waves = 16-head tiles
    static constexpr int THREADS = 64 * NW;
    static constexpr int STEP = 32;                  // positions per tile
    static constexpr int STAGES = 4;                 // tiles in the LDS ring
    static constexpr int KS = D / 32;                // k-steps over d in q.K
    static constexpr int DPL = D / 16;               // V columns per lane = M tiles of O^T
    static constexpr int CPR = D / 8;                // 16-byte chunks per row
    static constexpr int TILE_BYTES = STEP * D * 2;  // K (or V) bytes of one tile
    static constexpr int LOADS = TILE_BYTES / 1024;  // wave-wide 16-byte loads per tile (K or V)
    static constexpr int KPW = (LOADS + NW - 1) / NW;  // K loads (and V loads) each wave issues per tile
    static constexpr int PER_WAVE = 2 * KPW;           // every wave issues exactly this many
    static constexpr bool SPARE = LOADS % NW != 0;     // some waves issue out-of-range fillers
    static constexpr int RING_BYTES = STAGES * 2 * TILE_BYTES;
    static constexpr int LDS_BYTES = RING_BYTES + (SPARE ? 1024 : 0);
    static_assert(D >= 64 && D % 64 == 0, "head size");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
    static_assert(LDS_BYTES >= (kFusedMaxSplits + 2) * 16 * NG * 4, "fused-combine weights fit");
};

// LDS byte offset of chunk c of row t inside a tile.
template <int CPR>
__device__ __forceinline__ int swz(int t, int c) {
    return (t * CPR + (c ^ (t & 7))) * 16;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int D, int NG>
__global__ __launch_bounds__(256) void decode_mfma_hs_kernel(DecodeArgs a) {
    using C = HsCfg<D, NG>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, kg = lane >> 4;

    long long unit;
    int s;
    map_block(blockIdx.x, a.units, a.max_splits, &unit, &s);
    const int kvh = (int)(unit % a.Hkv);
    const long long row = unit / a.Hkv;
    const int g0 = blockIdx.y * 16 * NG;
    const int gcnt = min(16 * NG, a.G - g0);

    int b, len;
    row_extent(a.seq_lens, row, a.Lmax, a.causal, &b, &len);
    b = __builtin_amdgcn_readfirstlane(b);
    len = __builtin_amdgcn_readfirstlane(len);
    const int p0 = s * a.chunk;
    if (s > 0 && p0 >= len) return;  // whole workgroup: this chunk is past the end
    const int p1 = min(p0 + a.chunk, len);
    const int nsplit = len > 0 ? (len + a.chunk - 1) / a.chunk : 1;
    const int ntiles = p1 > p0 ? (p1 - p0 + C::STEP - 1) / C::STEP : 0;

    const size_t pos_stride = (size_t)a.Hkv * D;
    const int rowbytes = (int)(pos_stride * 2);
    const uint16_t* kseq = a.k + ((size_t)b * a.Lmax * a.Hkv + kvh) * D;
    const uint16_t* vseq = a.v + ((size_t)b * a.Lmax * a.Hkv + kvh) * D;

    // This wave's q^T operand (B of q.K): lane (li, kg), k-step ks holds
    // q[head 16w + li][32 ks + 8 kg .. +8]; heads past the group read as zero.
    u32x4_t qb[C::KS];
    {
        const uint16_t* qblk = a.q + ((size_t)row * a.Hq + (size_t)kvh * a.G + g0) * D;
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(qblk, gcnt * D * 2);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            qb[ks] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                      qr, (16 * w + li) * D * 2 + ks * 64 + kg * 16, 0, 0));
    }

    // Issue this wave's share of the loads of tile `tile` into ring slot tile % STAGES.
    // Load jj (0 .. LOADS-1) covers 1 KB of the K tile and, with a second
    // load, the same 1 KB of the V tile; wave w issues jj = w, w + NW, ...
    // Every wave issues KPW of each, so all waves keep the same count of loads
    // in flight: a jj past the tile is a filler whose offset is out of range
    // (it reads nothing and writes zeros to a spare 1 KB past the ring).
    constexpr unsigned kOutOfRange = 0x7FFFFFF0u;  // the planner bounds 128 rows of K to 2^31 bytes
    auto issue_tile = [&](int tile) {
        const int t0 = p0 + tile * C::STEP;
        const int rows = max(0, min(C::STEP, p1 - t0));
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kseq + (size_t)t0 * pos_stride, rows * rowbytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vseq + (size_t)t0 * pos_stride, rows * rowbytes);
        unsigned char* slot = smem + (tile % C::STAGES) * 2 * C::TILE_BYTES;
#pragma unroll
        for (int i = 0; i < C::KPW; ++i) {
            const int jj = w + C::NW * i;
            const bool real = !C::SPARE || jj < C::LOADS;
            const int p = jj * 64 + lane;  // 16-byte LDS slot in the tile
            const int t = p / C::CPR, cs = p % C::CPR;
            const unsigned voff = real ? (unsigned)(t * rowbytes + ((cs ^ (t & 7)) * 16)) : kOutOfRange;
            unsigned char* dst = real ? slot + jj * 1024 : smem + C::RING_BYTES;
            unsigned char* vdst = real ? dst + C::TILE_BYTES : dst;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)dst, 16, voff, 0, 0, kCachePolicyNT);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)vdst, 16, voff, 0, 0, kCachePolicyNT);
        }
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t oacc[C::DPL];
#pragma unroll
    for (int j = 0; j < C::DPL; ++j) oacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float qk = a.qk_log2;

    // Prologue: STAGES - 1 tiles in flight (tiles past the end read nothing).
    // q was issued first, so waiting until only the prologue's loads remain
    // guarantees q without waiting for any tile.
#pragma unroll
    for (int t = 0; t < C::STAGES - 1; ++t) issue_tile(t);
    __builtin_amdgcn_s_waitcnt(kVmcntStages<C::STAGES - 1, C::PER_WAVE>());

    for (int tile = 0; tile < ntiles; ++tile) {
        // Tile `tile` has landed once at most (STAGES - 2) later tiles of this
        // wave are still outstanding, and this wave's reads of the previous
        // tile are done once no LDS read is pending.  The barrier then
        // publishes every wave's part and frees the slot refilled below.  A
        // plain s_barrier, not __syncthreads: the latter's release fence also
        // waits for the loads still in flight to the ring.
        __builtin_amdgcn_s_waitcnt(kVmcntStages<C::STAGES - 2, C::PER_WAVE>() & ~(0xF << 8));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_tile(tile + C::STAGES - 1);

        const unsigned char* kt = smem + (tile % C::STAGES) * 2 * C::TILE_BYTES;
        const unsigned char* vt = kt + C::TILE_BYTES;
        const int st = p0 + tile * C::STEP;

        // ---- S^T = K q^T (two 16-row tiles)
        f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) {
                const int t = 16 * mq + li;
                const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(kt + swz<C::CPR>(t, 4 * ks + kg));
                sacc[mq] = mfma_16x16x32_bf16(ka, qb[ks], sacc[mq]);
            }
        }
        // ---- scale, mask the tail, lazy online softmax, P^T in registers
#pragma unroll
        for (int mq = 0; mq < 2; ++mq)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[mq][r] *= qk;
        if (st + C::STEP > p1) {
#pragma unroll
            for (int mq = 0; mq < 2; ++mq)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sacc[mq][r] = (st + 16 * mq + 4 * kg + r < p1) ? sacc[mq][r] : -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                         fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
        mx = max_xor32(max_xor16(mx));
        const bool moved = mx > m_run + kRescaleSlack;
        const float alpha = moved ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
        m_run = moved ? mx : m_run;
        u32x4_t pb;
        float lsum = 0.f;
#pragma unroll
        for (int mq = 0; mq < 2; ++mq) {
            const uint32_t lo = pack2_bf16_rne(__builtin_amdgcn_exp2f(sacc[mq][0] - m_run),
                                               __builtin_amdgcn_exp2f(sacc[mq][1] - m_run));
            const uint32_t hi = pack2_bf16_rne(__builtin_amdgcn_exp2f(sacc[mq][2] - m_run),
                                               __builtin_amdgcn_exp2f(sacc[mq][3] - m_run));
            pb[2 * mq] = lo;
            pb[2 * mq + 1] = hi;
            lsum += (bf16_lo_f32(lo) + bf16_hi_f32(lo)) + (bf16_lo_f32(hi) + bf16_hi_f32(hi));
        }
        l_run = l_run * alpha + lsum;
        if (__any(moved)) {
#pragma unroll
            for (int j = 0; j < C::DPL; ++j) oacc[j] = oacc[j] * alpha;
        }

        // ---- O^T += V^T P^T.  Element e of lane group kg is position
        // 16*(e/4) + 4*kg + e%4; lane li holds columns DPL*li .. DPL*li + DPL-1.
        constexpr int VW = C::DPL / 2;  // dwords per row per lane
        uint32_t vr[8][VW];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = 16 * (e / 4) + 4 * kg + (e % 4);
            if constexpr (VW >= 4) {
#pragma unroll
                for (int h = 0; h < VW / 4; ++h) {
                    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(vt + swz<C::CPR>(t, (VW / 4) * li + h));
                    vr[e][4 * h] = x.x;
                    vr[e][4 * h + 1] = x.y;
                    vr[e][4 * h + 2] = x.z;
                    vr[e][4 * h + 3] = x.w;
                }
            } else {
                // D = 64: 8 bytes per lane, half of chunk li/2
                const u32x2_t x = *reinterpret_cast<const u32x2_t*>(vt + swz<C::CPR>(t, li >> 1) + 8 * (li & 1));
                vr[e][0] = x.x;
                vr[e][1] = x.y;
            }
        }
#pragma unroll
        for (int wd = 0; wd < VW; ++wd) {
            u32x4_t va_even, va_odd;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                va_even[m] = perm_b32(vr[2 * m + 1][wd], vr[2 * m][wd], kPermLoHalves);
                va_odd[m] = perm_b32(vr[2 * m + 1][wd], vr[2 * m][wd], kPermHiHalves);
            }
            oacc[2 * wd] = mfma_16x16x32_bf16(va_even, pb, oacc[2 * wd]);
            oacc[2 * wd + 1] = mfma_16x16x32_bf16(va_odd, pb, oacc[2 * wd + 1]);
        }
    }

    // No buffer->LDS load of this workgroup may still be landing when its LDS
    // is released (the ring's tail loads read nothing, so this is quick).
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue: this wave's 16 heads, no merge with other waves
    l_run = sum_xor32(sum_xor16(l_run));
    const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
    const bool direct = nsplit == 1;
    const int g = 16 * w + li;  // head inside the block
    if (g < gcnt) {
        const int gh = g0 + g;
        float* dst;
        if (direct)
            dst = a.out + ((size_t)row * a.Hq + (size_t)kvh * a.G + gh) * D;
        else
            dst = a.part_o + (((size_t)unit * a.max_splits + s) * a.G + gh) * D;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int q4 = 0; q4 < C::DPL / 4; ++q4) {
                const int d = C::DPL * (4 * kg + r) + 4 * q4;
                *reinterpret_cast<f32x4_t*>(dst + d) =
                    f32x4_t{oacc[4 * q4][r], oacc[4 * q4 + 1][r], oacc[4 * q4 + 2][r], oacc[4 * q4 + 3][r]} * inv_l;
            }
        if (!direct && kg == 0)
            a.part_lse[((size_t)unit * a.max_splits + s) * a.G + gh] = m_run + __log2f(l_run);
    }
    if (direct || !a.fused) return;
    // ---- fused combine: the last chunk of this (row, kv head, head block) merges all partials
    __syncthreads();
    int* flag = reinterpret_cast<int*>(smem);
    if (!arrive_last(a.counters + unit * gridDim.y + blockIdx.y, nsplit, flag)) return;
    float* wts = reinterpret_cast<float*>(smem + 16);
    fused_combine(a, unit, nsplit, g0, gcnt, a.out + ((size_t)row * a.Hq + (size_t)kvh * a.G + g0) * D,
                  wts, 16 * NG);
}

template <int D, int NG>
static hipError_t launch_hs(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1) {
    using C = HsCfg<D, NG>;
    constexpr int lds = C::LDS_BYTES;
    if (lds > 64 * 1024) {
        static std::atomic<uint64_t> done_mask{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = 1ull << (dev & 63);
        if (!(done_mask.load() & bit)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_mfma_hs_kernel<D, NG>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
            done_mask.fetch_or(bit);
        }
    }
    const dim3 grid((unsigned)p.grid_main, (unsigned)p.head_blocks);
    const dim3 block(C::THREADS);
    if (ev0 || ev1)
        hipExtLaunchKernelGGL((decode_mfma_hs_kernel<D, NG>), grid, block, lds, stream, ev0, ev1, 0, a);
    else
        hipLaunchKernelGGL((decode_mfma_hs_kernel<D, NG>), grid, block, lds, stream, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_hs_d(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1) {
    switch (p.heads_per_block / 16) {
        case 2: return launch_hs<D, 2>(p, a, stream, ev0, ev1);
        case 3: return launch_hs<D, 3>(p, a, stream, ev0, ev1);
        case 4: return launch_hs<D, 4>(p, a, stream, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_mfma_heads(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                                    hipEvent_t ev1) {
    switch (a.D) {
        case 64: return launch_hs_d<64>(p, a, stream, ev0, ev1);
        case 128: return launch_hs_d<128>(p, a, stream, ev0, ev1);
        case 256: return launch_hs_d<256>(p, a, stream, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mqa
