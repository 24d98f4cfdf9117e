// Split-K decode attention on the vector ALU, for small head groups.
//
// When only a few query heads share a key/value head (grouped-query attention
// with a small group, "How To Scale Your Model", Part 7 "Transformer
// Inference", passage on shrinking the KV cache), the q.K and P.V products are
// too thin for a 16-wide matrix tile, so they run as bf16 dot products
// (v_dot2_f32_bf16) with fp32 accumulation.
//
// Layout: a cache row of D bf16 is spread over RL = D/8 lanes, each holding 8
// consecutive elements (one 128-bit load), so a wave covers RS = 64/RL
// positions per load instruction and every load is fully coalesced.  The q.K
// dot product of a position is summed across its RL lanes with DPP row
// permutations (the sum lands in every lane of the row, which is where P.V
// needs the weight).  Each wave keeps its own online softmax (base 2) over the
// positions it visits; the four waves merge by log-sum-exp through LDS at the
// end of the chunk.  P.V pairs two positions of the same column into one
// v_dot2 after a v_perm_b32, with P rounded to bf16 (the row sum uses the same
// rounded weights).
#include "kernel_common.hpp"
#include "launch.hpp"

namespace mqa {

template <int RL>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    if constexpr (RL >= 8) x += dpp_f32<kDppRowHalfMirror>(x);
    if constexpr (RL >= 16) x += dpp_f32<kDppRowMirror>(x);
    if constexpr (RL >= 32) x = sum_xor16(x);
    return x;
}

// Reduction over the lanes that share a column slot but sit in different rows
// (lane i meets lanes i^RL, ..., i^32): DPP inside a 16-lane row, permlane
// swaps across rows.
template <int RL, bool MAX>
__device__ __forceinline__ float across_rows(float x) {
    if constexpr (RL <= 4) {
        const float y = dpp_f32<kDppRowRor4>(x);
        x = MAX ? fmaxf(x, y) : x + y;
    }
    if constexpr (RL <= 8) {
        const float y = dpp_f32<kDppRowRor8>(x);
        x = MAX ? fmaxf(x, y) : x + y;
    }
    if constexpr (RL <= 16) x = MAX ? max_xor16(x) : sum_xor16(x);
    x = MAX ? max_xor32(x) : sum_xor32(x);
    return x;
}

// Value of lane `src` (0..63) of x, in every lane.  Must run with every lane
// of the wave active: ds_bpermute reads zero from an inactive source lane.
__device__ __forceinline__ float lane_value(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

// FUSED: the fused-combine form, a separate instantiation (as for the
// matrix-core kernel) so that its tail leaves the plain form's code alone.
template <int D, int GB, int FMT, bool FUSED>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
    constexpr bool Q8 = FMT != kKvBf16;  // 8-bit codes with one scale per cached row
    constexpr int NW = 4;
    constexpr int EPL = Q8 ? 16 : 8;     // cached elements per lane of one 16-byte load
    constexpr int NP = EPL / 2;          // bf16 pairs per lane
    constexpr int RL = D / EPL;          // lanes per cache row
    constexpr int RS = 64 / RL;          // rows per load instruction
    constexpr int NB = RS * 4 <= 32 ? 4 : 2;  // load instructions per block (even: P.V pairs them)
    constexpr int WB = NB * RS;          // positions per wave block
    static_assert(WB <= 32 && 32 % WB == 0, "a block never straddles a page");
    __shared__ float mrg_m[NW][GB];
    __shared__ float mrg_l[NW][GB];
    __shared__ __attribute__((aligned(16))) float mrg_o[NW][GB][D];
    __shared__ int s_flag;
    __shared__ unsigned s_amax[GB];  // per head: largest |output| (fp32 bits) of a partial row
    static_assert(D % 64 == 0, "a wave of the merge covers one head row");

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (wave-uniform)
    const int rl = lane % RL, rr = lane / RL;

    long long unit;
    int s;
    map_block(blockIdx.x, a.units, a.max_splits, &unit, &s);
    const int kvh = (int)(unit % a.Hkv);
    const long long row = unit / a.Hkv;
    const int g0 = blockIdx.y * GB;
    const int gcnt = min(GB, a.GT - g0);  // query rows (token, head) of this block

    int b, len;
    row_extent(a.seq_lens, row, a.Lmax, &b, &len);
    // Workgroup-uniform; stated so the compiler keeps them (and the buffer
    // descriptors built from them) in scalar registers.
    b = __builtin_amdgcn_readfirstlane(b);
    len = __builtin_amdgcn_readfirstlane(len);
    const ChunkSpan span = chunk_span(a.window, a.chunk, a.max_splits, len, s);
    if (s > 0 && span.p0 >= len) return;
    // Blocks start at the block holding the first attended position (a
    // multiple of WB, which divides 32), so every block has a valid row.
    const int lo = span.lo;
    const int p0 = max(span.p0, lo & ~(WB - 1));
    const int p1 = span.p1;
    const int nsplit = span.nsplit;

    // q for this lane's EPL columns of every query row in the block, as bf16
    // pairs; and the positions each row may attend (token i of the row's T:
    // len - T + 1 + i).
    uint32_t qv[GB][NP];
    int lim[GB];
#pragma unroll
    for (int gg = 0; gg < GB; ++gg) {
        const uint16_t* qrow = a.q + qrow_offset(a, row, kvh, min(g0 + gg, a.GT - 1)) + EPL * rl;
        lim[gg] = len - a.T + 1 + (g0 + gg) / a.G;
#pragma unroll
        for (int h = 0; h < NP / 4; ++h) {
            u32x4_t t = {0u, 0u, 0u, 0u};
            if (gg < gcnt) t = load_u32x4(qrow + 8 * h);
#pragma unroll
            for (int c = 0; c < 4; ++c) qv[gg][4 * h + c] = t[c];
        }
    }
    const int tmask = p1 - a.T + 1;  // blocks reaching past it hold a position some row must not see

    const int rowbytes = a.Hkv * D * (Q8 ? 1 : 2);  // bytes between consecutive positions of a cache
    const float qk = a.qk_log2;
    // Byte offset of this lane's 16 bytes in row st*RS + rr of a block.
    int off[NB];
#pragma unroll
    for (int st = 0; st < NB; ++st) off[st] = (st * RS + rr) * rowbytes + rl * 16;

    float m[GB], l[GB], o[GB][EPL];
#pragma unroll
    for (int gg = 0; gg < GB; ++gg) {
        m[gg] = -INFINITY;
        l[gg] = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) o[gg][j] = 0.f;
    }

    const int nblk = p1 > p0 ? (p1 - p0 + WB - 1) / WB : 0;
    // Issue the loads of block `blk` (of this wave's blocks w, w + NW, ...).
    // The buffer range ends at the last valid row: rows past it, and whole
    // blocks past the chunk, read as zero without a memory access; so do rows
    // before a sliding window's first position (out-of-range offsets).  An
    // 8-bit cache also loads the block rows' K and V scales, lane j holding
    // those of row j % WB.
    auto load_block = [&](int blk, u32x4_t (&kr)[NB], u32x4_t (&vr)[NB], float& ks, float& vs) {
        const int t0 = p0 + blk * WB;
        const int rows = max(0, min(WB, p1 - t0));
        const int skip = lo - t0;  // rows of the block before the window (> 0 in its first block only)
        const RowLoc loc = rows > 0 ? kv_loc(a, b, kvh, t0) : RowLoc{0, 0};
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(row_ptr<Q8 ? 1 : 2>(a.k, a, loc.row), rows * rowbytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(row_ptr<Q8 ? 1 : 2>(a.v, a, loc.row), rows * rowbytes);
#pragma unroll
        for (int st = 0; st < NB; ++st) {
            const int o = st * RS + rr < skip ? kOutOfRange : off[st];
            kr[st] = buffer_load_u32x4(krs, o);
            vr[st] = buffer_load_u32x4(vrs, o);
        }
        if constexpr (Q8) {
            const int j = lane % WB;
            const int so = j < skip ? kOutOfRange : j * 4;
            ks = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.k_scale + loc.scale, rows * 4), so, 0, kCachePolicyNT));
            vs = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.v_scale + loc.scale, rows * 4), so, 0, kCachePolicyNT));
        }
    };
    // The lane's EPL cached values of load st as bf16 pairs (exact widening of 8-bit codes).
    auto widen_row = [&](const u32x4_t& r, uint32_t (&x)[NP]) {
        if constexpr (Q8) {
            const u32x4_t lo8 = widen8<FMT>(u32x2_t{r[0], r[1]});
            const u32x4_t hi8 = widen8<FMT>(u32x2_t{r[2], r[3]});
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                x[c] = lo8[c];
                x[4 + c] = hi8[c];
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = r[c];
        }
    };
    auto compute_block = [&](int blk, const u32x4_t (&kr)[NB], const u32x4_t (&vr)[NB], float ks, float vs) {
        const int t0 = p0 + blk * WB;
        const int rows = min(WB, p1 - t0);
        const int skip = lo - t0;
        // logits (base-2 units), masked outside [lo, p1); an 8-bit cache
        // scales each logit by its K row's scale and each weight in P.V by
        // its V row's scale (zero outside the range, where codes read as 0)
        const bool edge = rows < WB || skip > 0 || t0 + WB > tmask;
        float sc[NB][GB];
        float vscale[NB];
#pragma unroll
        for (int st = 0; st < NB; ++st) {
            const int r = st * RS + rr;
            const bool ok = !edge || (r < rows && r >= skip);
            float kscale = 1.f;
            if constexpr (Q8) {
                // every lane takes part in both permutes (a lane reading an
                // inactive lane would get zero), then the V scale is masked
                kscale = lane_value(ks, r);
                const float vrow = lane_value(vs, r);
                vscale[st] = ok ? vrow : 0.f;
            }
            uint32_t kk[NP];
            widen_row(kr[st], kk);
#pragma unroll
            for (int gg = 0; gg < GB; ++gg) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < NP; ++c) acc = dot2_bf16(qv[gg][c], kk[c], acc);
                acc = row_sum<RL>(acc) * qk;
                if constexpr (Q8) acc *= kscale;
                sc[st][gg] = (ok && (!edge || t0 + r < lim[gg])) ? acc : -INFINITY;
            }
        }
        // online softmax update for the block, with lazy rescaling
        uint32_t pp[NB / 2][GB];
        bool any_rescale = false;
        float alpha[GB];
#pragma unroll
        for (int gg = 0; gg < GB; ++gg) {
            float mx = sc[0][gg];
#pragma unroll
            for (int st = 1; st < NB; ++st) mx = fmaxf(mx, sc[st][gg]);
            mx = across_rows<RL, true>(mx);
            const bool moved = mx > m[gg] + kRescaleSlack;
            alpha[gg] = moved ? __builtin_amdgcn_exp2f(m[gg] - mx) : 1.f;
            m[gg] = moved ? mx : m[gg];
            any_rescale |= moved;
            // a row with no visible position yet keeps m = -inf; its weights are zero
            const float m_use = m[gg] == -INFINITY ? 0.f : m[gg];
            float lsum = 0.f;
#pragma unroll
            for (int st = 0; st < NB; st += 2) {
                const float pa = __builtin_amdgcn_exp2f(sc[st][gg] - m_use);
                const float pb = __builtin_amdgcn_exp2f(sc[st + 1][gg] - m_use);
                if constexpr (Q8) {
                    pp[st / 2][gg] = pack2_bf16_rne(pa * vscale[st], pb * vscale[st + 1]);
                    lsum += pa + pb;
                } else {
                    const uint32_t pair = pack2_bf16_rne(pa, pb);
                    pp[st / 2][gg] = pair;
                    lsum += bf16_lo_f32(pair) + bf16_hi_f32(pair);
                }
            }
            l[gg] = l[gg] * alpha[gg] + lsum;
        }
        if (__any(any_rescale)) {
#pragma unroll
            for (int gg = 0; gg < GB; ++gg)
#pragma unroll
                for (int j = 0; j < EPL; ++j) o[gg][j] *= alpha[gg];
        }
        // P.V: two positions of one column per v_dot2
#pragma unroll
        for (int st = 0; st < NB; st += 2) {
            uint32_t va[NP], vb[NP];
            widen_row(vr[st], va);
            widen_row(vr[st + 1], vb);
#pragma unroll
            for (int c = 0; c < NP; ++c) {
                const uint32_t lo2 = perm_b32(vb[c], va[c], kPermLoHalves);
                const uint32_t hi2 = perm_b32(vb[c], va[c], kPermHiHalves);
#pragma unroll
                for (int gg = 0; gg < GB; ++gg) {
                    o[gg][2 * c] = dot2_bf16(pp[st / 2][gg], lo2, o[gg][2 * c]);
                    o[gg][2 * c + 1] = dot2_bf16(pp[st / 2][gg], hi2, o[gg][2 * c + 1]);
                }
            }
        }
    };
    // Double-buffered: the loads of a wave's next block are in flight while
    // it computes the current one (two register sets, alternating).
    u32x4_t ka[NB], va[NB], kb[NB], vb[NB];
    float ksa = 0.f, vsa = 0.f, ksb = 0.f, vsb = 0.f;
    if (w < nblk) load_block(w, ka, va, ksa, vsa);
    for (int blk = w; blk < nblk; blk += 2 * NW) {
        load_block(blk + NW, kb, vb, ksb, vsb);
        compute_block(blk, ka, va, ksa, vsa);
        if (blk + NW >= nblk) break;
        load_block(blk + 2 * NW, ka, va, ksa, vsa);
        compute_block(blk + NW, kb, vb, ksb, vsb);
    }

    // Sum the rows of the wave (same softmax state in every row).
#pragma unroll
    for (int gg = 0; gg < GB; ++gg) {
        l[gg] = across_rows<RL, false>(l[gg]);
#pragma unroll
        for (int j = 0; j < EPL; ++j) o[gg][j] = across_rows<RL, false>(o[gg][j]);
    }
    if (rr == 0) {
#pragma unroll
        for (int gg = 0; gg < GB; ++gg)
#pragma unroll
            for (int j = 0; j < EPL; j += 4)
                *reinterpret_cast<f32x4_t*>(&mrg_o[w][gg][EPL * rl + j]) =
                    f32x4_t{o[gg][j], o[gg][j + 1], o[gg][j + 2], o[gg][j + 3]};
        if (rl == 0) {
#pragma unroll
            for (int gg = 0; gg < GB; ++gg) {
                mrg_m[w][gg] = m[gg];
                mrg_l[w][gg] = l[gg];
            }
        }
    }
    if (tid < GB) s_amax[tid] = 0u;
    __syncthreads();

    // Log-sum-exp merge of the four waves, then normalise and store.  Thread
    // t merges values idx = t + 256k (head idx / D, column idx % D), so every
    // wave's 64 values belong to one head.  A chunk of a split sequence stores
    // its fp16 partial row scaled by 2^-e (e from the row's largest value).
    const bool direct = nsplit == 1;
    constexpr int VPT = (GB * D + 255) / 256;  // merged values per thread
    float val[VPT];
    float lse[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int idx = tid + 256 * k;
        val[k] = 0.f;
        lse[k] = -INFINITY;
        if (idx < gcnt * D) {
            const int gg = idx / D, d = idx % D;
            float M = mrg_m[0][gg];
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, mrg_m[ww][gg]);
            float O = 0.f, L = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    const float sw = __builtin_amdgcn_exp2f(mrg_m[ww][gg] - M);
                    O += sw * mrg_o[ww][gg][d];
                    L += sw * mrg_l[ww][gg];
                }
            }
            val[k] = L > 0.f ? O / L : 0.f;
            lse[k] = M + __log2f(L);
        }
    }
    if (direct) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int idx = tid + 256 * k;
            if (idx < gcnt * D) {
                a.out[qrow_offset(a, row, kvh, g0 + idx / D) + idx % D] = val[k];
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int idx = tid + 256 * k;
            const float mx = wave_max(fabsf(val[k]));
            if (lane == 0 && idx < gcnt * D) atomicMax(&s_amax[idx / D], __float_as_uint(mx));
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int idx = tid + 256 * k;
            if (idx < gcnt * D) {
                const int gg = idx / D, d = idx % D;
                const int e = scale_exponent(__uint_as_float(s_amax[gg]));
                const size_t part = ((size_t)unit * a.max_splits + s) * a.GT + g0 + gg;
                const uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_ldexpf(val[k], -e));
                if constexpr (FUSED) {
                    store_coherent(a.part_o + part * D + d, h);
                    if (d == 0) store_coherent8(a.part_ml + part, f32x2_t{lse[k], (float)e});
                } else {
                    a.part_o[part * D + d] = h;
                    if (d == 0) a.part_ml[part] = f32x2_t{lse[k], (float)e};
                }
            }
        }
    }
    if constexpr (FUSED) {
        if (direct) return;
        // Fused combine: the chunks of this (row, kv head, head block) share the merge.
        fused_tail(a, unit, row, kvh, nsplit, g0, gcnt,
                   a.counters + (unit * gridDim.y + blockIdx.y) * kFusedCountersPerUnit, &s_flag);
    }
}

template <int D, int GB, int FMT, bool FUSED>
static hipError_t launch_form(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1) {
    const dim3 grid((unsigned)p.grid_main, (unsigned)p.head_blocks);
    const dim3 block(256);
    if (ev0 || ev1)
        hipExtLaunchKernelGGL((decode_valu_kernel<D, GB, FMT, FUSED>), grid, block, 0, stream, ev0, ev1, 0, a);
    else
        hipLaunchKernelGGL((decode_valu_kernel<D, GB, FMT, FUSED>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int D, int GB, int FMT>
static hipError_t launch_one(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                             hipEvent_t ev1) {
    return a.fused ? launch_form<D, GB, FMT, true>(p, a, stream, ev0, ev1)
                   : launch_form<D, GB, FMT, false>(p, a, stream, ev0, ev1);
}

template <int D, int FMT>
static hipError_t launch_valu_d(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                                hipEvent_t ev1) {
    switch (p.heads_per_block) {
        case 1: return launch_one<D, 1, FMT>(p, a, stream, ev0, ev1);
        case 2: return launch_one<D, 2, FMT>(p, a, stream, ev0, ev1);
        case 4: return launch_one<D, 4, FMT>(p, a, stream, ev0, ev1);
        case 8:
            if constexpr (FMT == kKvBf16) return launch_one<D, 8, FMT>(p, a, stream, ev0, ev1);
            return hipErrorInvalidValue;  // the planner caps 8-bit caches at 4 heads per block
        default: return hipErrorInvalidValue;
    }
}

template <int FMT>
static hipError_t launch_valu_f(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                                hipEvent_t ev1) {
    switch (a.D) {
        case 64: return launch_valu_d<64, FMT>(p, a, stream, ev0, ev1);
        case 128: return launch_valu_d<128, FMT>(p, a, stream, ev0, ev1);
        case 256: return launch_valu_d<256, FMT>(p, a, stream, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_valu(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1) {
    switch (p.kv_format) {
        case kKvBf16: return launch_valu_f<kKvBf16>(p, a, stream, ev0, ev1);
        case kKvFp8: return launch_valu_f<kKvFp8>(p, a, stream, ev0, ev1);
        case kKvInt8: return launch_valu_f<kKvInt8>(p, a, stream, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mqa
