// Causal prefill on the matrix cores (gfx950): every position t of a prompt
// attends positions 0 .. t of its own sequence, with no cache ("How To Scale
// Your Model", Part 7, the passage on prefill versus generation: prefill is
// the compute-bound pass over a whole prompt; "Efficiently Scaling Transformer
// Inference", section 3.4, "Attention Layer Partitioning": the K/V read is
// amortised over the query tokens).
//
// The query rows of one (sequence b, kv head) are the (position t, head g in
// the group) pairs in token-major order, r = t * G + g; row r attends
// positions 0 .. r / G.  A workgroup owns ROWS consecutive rows and
// ROWS / (16 RT) compute waves, each with RT 16-row tiles of the matrix
// products (the configuration per head size is prefill_rows, _row_tiles,
// _step and _stages).  The workgroup's causal prefix is streamed through an
// LDS ring of STAGES slots of STEP-position K and V tiles, loaded by all
// waves with direct buffer-to-LDS loads, STAGES - 1 tiles ahead of the one
// in use.  Per tile and wave:
//   * S^T = K q^T on 16x16x32 bf16 products: every K read (16 positions x 32
//     of d) feeds the wave's RT row tiles;
//   * a base-2 online softmax with lazy rescaling, the row maximum reduced
//     over the four lane groups that hold a row;
//   * O^T += V^T P^T with the V^T operand from gfx950's transposing LDS
//     reads; every V^T read feeds the RT row tiles.
// Tiles that lie wholly below the wave's first row skip the causal mask.
// Rows at or past the sequence length are written as zeros.
#include <atomic>

#include "kernel_common.hpp"
#include "launch.hpp"
#include "lds_tile.hpp"

namespace mqa {

template <int D>
struct PrefillCfg {
    static constexpr int ROWS = prefill_rows(D);       // query rows per workgroup
    static constexpr int RT = prefill_row_tiles(D);    // 16-row tiles per compute wave
    static constexpr int WAVES = ROWS / (16 * RT);     // compute waves
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int STEP = prefill_step(D);       // positions per K/V tile
    static constexpr int STAGES = prefill_stages(D);   // LDS ring slots
    static constexpr int NQ = STEP / 16;               // 16-position blocks of a tile (q.K products)
    static constexpr int NKB = STEP / 32;              // 32-position blocks of a tile (P.V products)
    static constexpr int ROWB = D * 2;                 // bytes of one cached row
    static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
    static constexpr int TILE_BYTES = STEP * ROWB;     // K (or V) bytes of a tile
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int LOADS = TILE_BYTES / 1024;    // wave-wide 16-byte loads per K (or V) tile
    static constexpr int LPW = LOADS / WAVES;          // of them, per wave
    static constexpr int KS = D / 32;                  // k-steps of q.K
    static constexpr int MT = D / 16;                  // 16-row tiles of O^T (along d)
    static_assert(RT == 1 || RT == 2, "one or two 16-row tiles per wave");
    static_assert(ROWS % (16 * RT) == 0 && THREADS <= 1024, "whole waves of row tiles");
    static_assert(STEP == 32 || STEP == 64, "tiles of 32 or 64 positions");
    static_assert(STAGES >= 2, "a tile in use and one landing");
    static_assert(LOADS % WAVES == 0 && LPW > 0, "every wave issues the same number of loads");
    static_assert(2 * LPW * (STAGES - 1) <= 63, "the ring's loads in flight fit a wave's counter");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// Launch bound 512 threads even for smaller workgroups: the register budget
// of two waves per SIMD, so that two smaller workgroups share a CU.
template <int D>
__global__ __launch_bounds__(PrefillCfg<D>::THREADS > 512 ? PrefillCfg<D>::THREADS : 512) void prefill_mfma_kernel(
    PrefillArgs a) {
    using C = PrefillCfg<D>;
    constexpr int RT = C::RT;
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, kg = lane >> 4;

    // workgroup -> (sequence b, kv head, block of rows).  Workgroup x runs on
    // XCD x mod 8; with a multiple of 8 (sequence, kv head) units, unit u's
    // row blocks all run on XCD u mod 8, one after another, longest prefix
    // first, so the XCD's CUs stream the same prefix at the same time and
    // its L2 serves most of the re-reads (a unit's K and V are at most a few
    // MB).  Otherwise the units take turns, longest prefixes first.
    const long long units = (long long)a.B * a.Hkv;
    const long long x = blockIdx.x;
    long long unit;
    int blk;
    if ((units & 7) == 0) {
        const long long r = x >> 3;
        unit = (r / a.row_blocks) * 8 + (x & 7);
        blk = a.row_blocks - 1 - (int)(r % a.row_blocks);
    } else {
        unit = x % units;
        blk = a.row_blocks - 1 - (int)(x / units);
    }
    const int b = (int)(unit / a.Hkv), kvh = (int)(unit % a.Hkv);
    const int nrows = a.Lmax * a.G;  // query rows of (b, kvh)
    int len = a.seq_lens[b];
    len = __builtin_amdgcn_readfirstlane(len < 0 ? 0 : (len > a.Lmax ? a.Lmax : len));
    const int r0 = blk * C::ROWS;
    const int rlast = min(r0 + C::ROWS, nrows) - 1;
    const int kv_end = min(rlast / a.G + 1, len);  // positions any row of the block attends
    const int ntiles = kv_end > 0 ? (kv_end + C::STEP - 1) / C::STEP : 0;

    // This lane's rows r = r0 + 16 (RT w + rt) + li: token t = r / G
    // attends positions below lim = min(t + 1, len); rows with t >= len are
    // computed like the others and written as zeros.  orow indexes the row in
    // q and out ([B, Lmax, Hq, D]), -1 past the last row.
    int lim[RT];
    bool valid[RT];
    long long orow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = r0 + 16 * RT * w + 16 * rt + li;
        const int t = r / a.G;
        lim[rt] = min(t + 1, len);
        valid[rt] = r < nrows && t < len;
        orow[rt] = r < nrows ? ((long long)b * a.Lmax + t) * a.Hq + (long long)kvh * a.G + (r - t * a.G) : -1;
    }
    // the wave's first row has the smallest limit: a tile ending at or below
    // it needs no causal mask in this wave
    const int wr = r0 + 16 * RT * w;
    const int lim_wave = wr < nrows ? min(wr / a.G + 1, len) : 0;

    // q^T operand (B of q.K) of each row tile: lane (li, kg), k-step ks holds
    // q[row li][32 ks + 8 kg .. +8]; rows past the last read as zero
    u32x4_t qb[RT][C::KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const uint16_t* qp = a.q + (orow[rt] < 0 ? 0 : orow[rt]) * D + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            qb[rt][ks] = orow[rt] < 0 ? u32x4_t{0u, 0u, 0u, 0u} : *reinterpret_cast<const u32x4_t*>(qp + 32 * ks);
    }

    // Loads of tile `tile` into stage tile % STAGES: load jj (0 .. LOADS-1)
    // covers 1 KB of the K tile and, with a second load, the same 1 KB of the
    // V tile; wave w issues jj = w, w + WAVES, ....  Rows at or past kv_end
    // are outside the buffer range and arrive as zeros, so a tile past the
    // last is loaded too (as zeros): every wave has the same loads in flight.
    const int rowbytes = a.Hkv * C::ROWB;  // bytes between consecutive positions
    const size_t kv0 = ((size_t)b * a.Lmax * a.Hkv + kvh) * D;
    auto issue_tile = [&](int tile) {
        const int t0 = tile * C::STEP;
        const int rows = max(0, min(C::STEP, kv_end - t0));
        const size_t off = kv0 + (size_t)t0 * a.Hkv * D;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + off, rows * rowbytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + off, rows * rowbytes);
        unsigned char* stage = smem + (tile % C::STAGES) * C::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < C::LPW; ++i) {
            const int jj = w + C::WAVES * i;
            const int p = jj * 64 + lane;  // 16-byte LDS slot in the tile
            const int t = p / C::CPR, cs = p % C::CPR;
            const int voff = t * rowbytes + ((cs ^ swz_key<D>(t)) * 16);
            unsigned char* dst = stage + jj * 1024;
            // default cache policy: the prefix is re-read by the unit's other
            // row blocks, which run beside this one on the same XCD (the
            // non-temporal loads of the decode kernels measured 7 % slower)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)dst, 16, voff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(dst + C::TILE_BYTES), 16, voff, 0, 0, 0);
        }
    };

    float m_run[RT], l_run[RT];
    f32x4_t oacc[RT][C::MT];  // O^T of row tile rt, 16-row tile m of d: rows d = 16m .. 16m+15
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) m_run[rt] = -INFINITY, l_run[rt] = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int m = 0; m < C::MT; ++m) oacc[rt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float qk = a.qk_log2;

    // Transposing V^T reads, as in the decode kernel: in each 16-lane group,
    // lane 4j + c points at the 8 bytes d = 16m + 4c .. +3 of position row j
    // of its group of four rows; element e of lane group kg is position
    // 16 (e / 4) + 4 kg + e % 4 of a 32-position block (the P^T order).
    constexpr int NR = kSwzRegs<D>;
    const int tr_j = li >> 2, tr_b = li & 3;
    const int tr_lo = swz<D>(4 * kg + tr_j, tr_b >> 1) + (tr_b & 1) * 8;
    const int tr_hi = swz<D>(16 + 4 * kg + tr_j, tr_b >> 1) + (tr_b & 1) * 8;

    // O^T += V^T P^T of the tile in stage `stage`, in steps of MS 16-row
    // tiles of d for each 32-position block.  The V^T reads of step s + 1 are
    // issued before the wait for those of step s, which therefore leaves the
    // 2 MS reads of step s + 1 in flight (LDS reads complete in order; any
    // other LDS or scalar-memory operation in flight only makes the wait
    // longer).  Measured on MI355X against a wait for every read of each half
    // of d: PaLM-shaped prefill 8.49 against 8.68 ms, gqa70b-shaped equal.
    constexpr int MS = 4, SPB = C::MT / MS, NS = C::NKB * SPB;
    static_assert(C::MT % MS == 0 && 2 * MS <= 15, "whole steps; the wait count fits lgkmcnt");
    auto pv_tile = [&](int stage, const u32x4_t (&pb)[RT][C::NKB]) {
        const uint32_t vbase = lds_addr(smem + stage * C::STAGE_BYTES + C::TILE_BYTES);
        u32x2_t lo[2][MS], hi[2][MS];
        auto issue = [&](auto sc) {
            constexpr int s = decltype(sc)::value, kb = s / SPB, M0 = (s % SPB) * MS;
            const uint32_t vb = vbase + kb * 32 * C::ROWB;
            issue_vt_tile<M0, MS, NR>(vb + tr_lo, vb + tr_hi, lo[s & 1], hi[s & 1]);
        };
        issue(std::integral_constant<int, 0>{});
        static_for<0, NS>([&](auto sc) {
            constexpr int s = decltype(sc)::value, kb = s / SPB, M0 = (s % SPB) * MS;
            if constexpr (s + 1 < NS) {
                issue(std::integral_constant<int, s + 1>{});
                asm volatile("s_waitcnt lgkmcnt(%0)" :: "i"(2 * MS) : "memory");
            } else {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
#pragma unroll
            for (int m = 0; m < MS; ++m) asm volatile("" : "+v"(lo[s & 1][m]), "+v"(hi[s & 1][m]));
#pragma unroll
            for (int j = 0; j < MS; ++j) {
                const u32x4_t va = u32x4_t{lo[s & 1][j].x, lo[s & 1][j].y, hi[s & 1][j].x, hi[s & 1][j].y};
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    oacc[rt][M0 + j] = mfma_16x16x32_bf16(va, pb[rt][kb], oacc[rt][M0 + j]);
            }
        });
    };

    // The tile loop keeps the accumulators untouched by vector instructions:
    // when a row maximum moves past the lazy-rescale slack (rare after the
    // first tiles) the inner loop stops before that tile's P.V, the
    // accumulators are rescaled outside it, and the tile is finished there.
    // (A rescale inside the loop, however rarely taken, makes the compiler
    // copy all accumulators between AGPRs and VGPRs on every tile.)
    u32x4_t pb[RT][C::NKB];
    float alpha[RT];
    int tile = 0;
    if (ntiles > 0) {
#pragma unroll
        for (int t = 0; t < C::STAGES - 1; ++t) issue_tile(t);
    }
    while (tile < ntiles) {
        bool rescale = false;
        for (; tile < ntiles; ++tile) {
            // this wave's loads of the tile have landed (those of the
            // STAGES - 2 tiles after it may still be in flight) and its LDS
            // reads of the previous tile have returned; after the barrier
            // every wave's have, so tile + STAGES - 1 may land in the previous
            // tile's stage
            __builtin_amdgcn_s_waitcnt(kVmcntStages<C::STAGES - 2, 2 * C::LPW>() & ~(0xF << 8));
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            issue_tile(tile + C::STAGES - 1);
            const unsigned char* kt = smem + (tile % C::STAGES) * C::STAGE_BYTES;

            // S^T = K q^T: accumulator (mq, rt), lane (li, kg), element e
            // holds row li of tile rt at position 16 mq + 4 kg + e
            f32x4_t sacc[C::NQ][RT];
#pragma unroll
            for (int mq = 0; mq < C::NQ; ++mq)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) sacc[mq][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
                for (int mq = 0; mq < C::NQ; ++mq) {
                    const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(kt + swz<D>(16 * mq + li, 4 * ks + kg));
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) sacc[mq][rt] = mfma_16x16x32_bf16(ka, qb[rt][ks], sacc[mq][rt]);
                }

            // scaled logits; the causal mask only on tiles reaching past the
            // wave's first row (a real branch: most tiles skip it)
            const int st = tile * C::STEP;
            float s[RT][C::NQ][4];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int mq = 0; mq < C::NQ; ++mq)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[rt][mq][e] = sacc[mq][rt][e] * qk;
            if (st + C::STEP > lim_wave) {
                asm volatile("" ::: "memory");
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int mq = 0; mq < C::NQ; ++mq)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            s[rt][mq][e] = st + 16 * mq + 4 * kg + e < lim[rt] ? s[rt][mq][e] : -INFINITY;
            }

            // online softmax of each row tile; P^T operands pb[rt][kb] of the
            // 32-position blocks kb
            bool moved_any = false;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                float mx = -INFINITY;
#pragma unroll
                for (int mq = 0; mq < C::NQ; ++mq)
#pragma unroll
                    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[rt][mq][e]);
                mx = max_xor32(max_xor16(mx));
                const bool moved = mx > m_run[rt] + kRescaleSlack;
                alpha[rt] = moved ? __builtin_amdgcn_exp2f(m_run[rt] - mx) : 1.f;
                m_run[rt] = moved ? mx : m_run[rt];
                moved_any |= moved;
                // a row with no visible position yet keeps m = -inf; its weights are 0
                const float m_use = m_run[rt] == -INFINITY ? 0.f : m_run[rt];
                float lsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb) {
                    uint32_t pk[4];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int x = 0; x < 2; ++x) {
                            const int mq = 2 * kb + h;
                            const float p0 = __builtin_amdgcn_exp2f(s[rt][mq][2 * x] - m_use);
                            const float p1 = __builtin_amdgcn_exp2f(s[rt][mq][2 * x + 1] - m_use);
                            pk[2 * h + x] = pack2_bf16_rne(p0, p1);
                            lsum += p0 + p1;
                        }
                    pb[rt][kb] = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
                }
                l_run[rt] = l_run[rt] * alpha[rt] + lsum;
            }
            if (__any(moved_any)) {
                rescale = true;
                break;  // P.V of this tile after the rescale, outside the loop
            }
            pv_tile(tile % C::STAGES, pb);
        }
        if (!rescale) break;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int m = 0; m < C::MT; ++m) oacc[rt][m] = oacc[rt][m] * alpha[rt];
        pv_tile(tile % C::STAGES, pb);
        ++tile;
    }
    // No buffer->LDS load of this workgroup (the ring's tail loads read
    // nothing) may still be landing when its LDS is released.
    __builtin_amdgcn_s_waitcnt(0);

    // Epilogue: O / l of each row, rows at or past the length as zeros; lane
    // (li, kg) writes d = 16m + 4kg .. +3 of row li (16 bytes, every m)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float l = sum_xor32(sum_xor16(l_run[rt]));
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (orow[rt] >= 0) {
            float* op = a.out + orow[rt] * D + 4 * kg;
#pragma unroll
            for (int m = 0; m < C::MT; ++m) {
                const f32x4_t o = valid[rt] ? oacc[rt][m] * inv : f32x4_t{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<f32x4_t*>(op + 16 * m) = o;
            }
        }
    }
}

template <int D>
static hipError_t launch_prefill_d(const Plan& p, const PrefillArgs& a, hipStream_t stream) {
    using C = PrefillCfg<D>;
    constexpr int lds = C::LDS_BYTES;
    if (lds > 64 * 1024) {
        static std::atomic<uint64_t> done_mask{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = 1ull << (dev & 63);
        if (!(done_mask.load() & bit)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_mfma_kernel<D>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
            done_mask.fetch_or(bit);
        }
    }
    if (p.block_main != C::THREADS || a.row_blocks * (long long)C::ROWS < (long long)a.Lmax * a.G)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_mfma_kernel<D>), dim3((unsigned)p.grid_main), dim3(C::THREADS), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill_mfma(const Plan& p, const PrefillArgs& a, hipStream_t stream) {
    if (p.grid_main <= 0) return hipSuccess;
    switch (a.D) {
        case 64: return launch_prefill_d<64>(p, a, stream);
        case 128: return launch_prefill_d<128>(p, a, stream);
        case 256: return launch_prefill_d<256>(p, a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mqa
