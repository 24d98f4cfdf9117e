// Split-K decode attention on matrix cores, one wave per 16 query heads.
//
// For every group size (e.g. the 48-head multiquery attention of PaLM 540B
// in "Efficiently Scaling Transformer Inference", section 3.4, "Attention
// Layer Partitioning", the 8-head groups of grouped-query attention) and
// every cache format (bf16, E4M3 or int8 codes) a workgroup owns (query row, kv
// head, chunk of positions, block of 16*NG query rows, NG = 1..6).  Compute wave
// w < NG owns heads 16w .. 16w+15 for every position of the chunk; groups
// below 16 pad the head tile.  The chunk's K and V rows are read from HBM
// exactly once per workgroup into an LDS ring of tiles of 32 positions by two
// load-only waves, with direct buffer-to-LDS loads (no registers hold data in
// flight); every compute wave then reads the whole tile from LDS.  A compute
// step takes PT tiles at once (two for 8-bit caches at D = 256, else one); the
// ring holds GSTAGES steps, GSTAGES - 2 of them in flight.  8-bit caches at
// D = 256 with NG <= 3 give each 16-row tile two compute waves, one per tile
// of a step, whose softmax states are merged once after the loop.
//
// Per tile, in each compute wave:
//   * S^T = K q^T on 16x16x32 bf16 tiles: A = two 16-row K tiles (read from
//     LDS), B = this wave's q^T (registers).  Head g = lane mod 16.  8-bit
//     caches feed their codes to the fp8 (16x16x128) or int8 (16x16x64)
//     matrix cores directly, with q split into two 8-bit parts.
//   * base-2 online softmax with lazy rescaling; the two S^T accumulators are
//     exactly the 8 k-slots per lane of the P^T operand of P.V.
//   * O^T += V^T P^T on 16x16x32 tiles: the V^T operand is read from LDS with
//     gfx950's transposing LDS reads (ds_read_b64_tr_b16), so no lane shuffles
//     (8-bit caches: ds_read_b64_tr_b8, codes widened to bf16 in registers).
// The loop is software-pipelined by one tile: q.K of the next tile is issued
// together with P.V of the current one.
// Rows at or past the end of the chunk are out of the buffer range and arrive
// as zeros; their logits are masked, so padding is never read.
#include <atomic>
#include <type_traits>

#include "kernel_common.hpp"
#include "launch.hpp"
#include "lds_tile.hpp"

namespace mqa {

template <int D, int NG, int FMT>
struct MfmaCfg {
    // NC compute waves (SUBS per 16-head tile, below) and NL load-only waves.
    // The loads of a tile all leave right after the ring barrier and queue in
    // the CU's address unit; a wave stalls until its own are accepted, so they
    // are kept off the compute waves.  Two loaders keep the ring's steps in
    // flight within the 63 loads a wave can have outstanding.
    static constexpr int NL = 2;
    static constexpr int STEP = 32;                  // positions per tile
    static constexpr bool Q8 = FMT != kKvBf16;       // 8-bit codes with a scale per row
    static constexpr int EB = Q8 ? 1 : 2;            // bytes per cached element
    // E4M3 caches with D a multiple of 128: q.K runs on fp8 matrix cores
    // (16x16x128) straight from the codes, with q split into two E4M3 parts
    static constexpr bool F8MMA = FMT == kKvFp8 && D % 128 == 0;
    static constexpr int NH8 = F8MMA ? D / 128 : 1;  // 128-wide halves of d
    // int8 caches: q.K on int8 matrix cores (16x16x64), q as 128 hi + lo
    static constexpr bool I8MMA = FMT == kKvInt8;
    static constexpr int NB8 = I8MMA ? D / 64 : 1;   // 64-wide blocks of d
    // Steps in the LDS ring: four, i.e. two steps in flight beyond the two in
    // use (measured with one tile per step).  bf16 D = 256 (128 KB): a fifth
    // tile measured slower on MI355X
    // (PaLM-shaped MQA 29.5 against 30.4 us per step, B=4 len 131072 87.4
    // against 88.2 us); per-workgroup timestamps show the later loop end
    // comes from the compute waves holding the ring barrier, not from loads
    // in flight.  D <= 128 leaves room for two workgroups per CU (B=32,
    // Hkv=8, len 4096: 89.0 us at 4 tiles against 92.1 at 5 and 88.3 at 6,
    // where one workgroup per CU fits; the ragged batch: 751 us at 4 and 5
    // tiles against 943 at 6).  8-bit tiles are half as large; their kernel is
    // bound by its own per-tile work rather than by loads in flight, and a
    // 4-tile ring measured faster than deeper ones (PaLM-shaped MQA: 24.8 us
    // at 4 tiles against 29.0 us at 9; B=4, len 131072: 73.7 against 82.1 us;
    // B=32, Hkv=8, D=128: 51.6 against 53.3 us at 8 tiles)
    static constexpr int GSTAGES = 4;
    static_assert(GSTAGES >= 4, "two steps' tiles in use and at least one more in flight");
    // Ring slots (32-position tiles) a compute step takes at once.  8-bit
    // steps at D = 256 take two: the step's fixed chain (ring barrier, the
    // cross-lane maximum, the rescale test, the latency of each
    // read-product-softmax link) is then paid once per 64 positions (MI355X,
    // split kernel, two runs: B=4 len 131072 fp8 58.7-59.8 against
    // 63.0-63.8 us, int8 70.9-71.3 against 78.8-79.5; PaLM-shaped MQA int8
    // 23.9-24.4 against 25.1-25.6, fp8 even).  At D = 128, where two
    // workgroups share a CU, two slots per step measured slower (B=32, Hkv=8,
    // len 4096, fp8: 51.0 against 46.8 us).
    static constexpr int PT = (Q8 && D >= 256) ? 2 : 1;
    static constexpr int STAGES = GSTAGES * PT;  // ring slots
    // Compute waves per 16-row tile of query rows: SUBS > 1 splits a step's
    // tiles between that many waves, each with its own softmax state, merged
    // once after the loop (while the workgroup stays within 8 waves).  Each
    // wave's chain of dependent work is then one tile per step, and two
    // chains share a SIMD (MI355X, split kernel, two runs: B=4 len 131072
    // fp8 51.9-52.8 against 59.1-59.4 us with one wave per tile, int8 66.0
    // against 70.9-71.1; PaLM-shaped MQA even).
    static constexpr int SUBS = (PT > 1 && NG <= 3) ? PT : 1;
    static constexpr int NU = PT / SUBS;  // tiles of a step per compute wave
    static constexpr int NC = NG * SUBS;  // compute waves
    static constexpr int NW = NC + NL;
    static constexpr int THREADS = 64 * NW;
    static constexpr int KS = D / 32;                // k-steps over d in q.K
    static constexpr int MT = D / 16;                // 16-row tiles of O^T
    static constexpr int ROWB = D * EB;              // bytes of one cached row
    static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
    static constexpr int TILE_BYTES = STEP * ROWB;   // K (or V) bytes of one tile
    static constexpr int SCALE_BYTES = Q8 ? 2 * STEP * 4 : 0;  // the tile rows' K scales, then V scales
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES + SCALE_BYTES;
    static constexpr int LOADS = TILE_BYTES / 1024;  // wave-wide 16-byte loads per tile (K or V)
    static constexpr int KPW = LOADS / NL;           // K loads (and as many V loads) per loader per tile
    static constexpr int PER_WAVE = 2 * KPW + (Q8 ? 1 : 0);  // loads a loader issues per tile (+ a scale row)
    static constexpr int RING_BYTES = STAGES * STAGE_BYTES;
    static constexpr int EPI_BYTES = NG * 16 * (D + 4) * 4;  // the output transpose, after the ring is drained
    static constexpr int LDS_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
    static_assert(D >= 64 && D % 64 == 0, "head size");
    static_assert(LOADS % NL == 0, "every loader issues the same number of loads");
    static_assert((GSTAGES - 1) * PT * PER_WAVE <= 63, "loads in flight fit a wave's counter");
    static_assert(NG >= 1 && NG <= 6, "one to six 16-row tiles of query rows");
    static_assert(NW <= 8, "the launch bound");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// FUSED: the kernel form whose chunks merge the partials themselves (the
// fused combine).  It is a separate instantiation so that the tail's code
// cannot change how the compiler allocates and schedules the tile loop of the
// plain form (with the tail behind a run-time flag in one kernel, MI355X
// measured 11 % slower 8-bit loops: int8 B=4 len 131072 86.6 against 78.0 us).
// One work item: the (unit, chunk) of x-index bx and the head block by.
// next != nullptr (persistent form): thread 0 also fetches the workgroup's
// following item into *next, once its wave has its q.
template <int D, int NG, int FMT, bool FUSED>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, long long bx, int by, long long* next) {
    using C = MfmaCfg<D, NG, FMT>;
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, kg = lane >> 4;
    // compute wave w < NC: 16-row tile hw of the block's query rows, and
    // tiles u0 .. u0 + NU - 1 of each step
    const int hw = w % NG, u0 = (w / NG) * C::NU;

    long long unit;
    int s;
    map_block(bx, a.units, a.max_splits, &unit, &s);
    const int kvh = (int)(unit % a.Hkv);
    const long long row = unit / a.Hkv;
    const int g0 = by * 16 * NG;
    const int gcnt = min(16 * NG, a.GT - g0);  // query rows (token, head) of this block

    int b, len, qbase;
    row_extent(a, row, &b, &len, &qbase);
    b = __builtin_amdgcn_readfirstlane(b);
    len = __builtin_amdgcn_readfirstlane(len);
    qbase = __builtin_amdgcn_readfirstlane(qbase);
    const int gq = a.GT;  // query rows of the unit: T tokens times G heads
    const ChunkSpan span = chunk_span(a.window, a.chunk, a.max_splits, len, s);
    if (s > 0 && span.p0 >= len) {  // whole workgroup: this chunk is past the end
        if (next != nullptr && tid == 0) *next = (long long)gridDim.x + atomicAdd(&a.queue[0], 1u);
        return;
    }
    // Sliding window: rows lo - 32 < t < lo of the first tile lie before it;
    // they are loaded as zeros and masked.
    const int lo = span.lo, p0 = span.p0, p1 = span.p1, nsplit = span.nsplit;
    const int ntiles = p1 > p0 ? (p1 - p0 + C::STEP - 1) / C::STEP : 0;
    const int nsteps = (ntiles + C::PT - 1) / C::PT;  // compute steps of PT tiles (the last may run past the end)

    const int rowbytes = a.Hkv * C::ROWB;  // bytes between consecutive positions of a cache

    // A compute wave's q^T operand (B of q.K): lane (li, kg), k-step ks holds
    // q[head 16w + li][32 ks + 8 kg .. +8]; heads past the group read as zero.
    u32x4_t qb[C::KS];
    // fp8 matrix cores: lane (li, kg) holds, for each 128-wide half h of d,
    // q[head][128h + 32kg .. +31] * 2^qe as the sum of two E4M3 codes (qh +
    // ql), qe per head putting its largest |q| in [128, 256).  A bf16 value
    // has 8 significant bits: the high code keeps 4, and the remainder (at
    // most 8 units of the value's last place) fits the low code exactly, so
    // only parts below E4M3's smallest subnormal (2^-9 of a 2^7..2^8 range)
    // are rounded.  qk8 = 2^-qe undoes the scaling in the logit.
    i32x8_t qh[C::NH8], ql[C::NH8];
    // int8 matrix cores: lane (li, kg) holds, for each 64-wide block b of d,
    // Q = rint(q[head][64b + 16kg .. +15] * 2^qe) as 128 hi + lo (int8
    // each, |hi| <= 64, -64 <= lo < 64), qe per head putting its largest |q|
    // in [2^12, 2^13): each q is rounded to 2^-13 of the head's largest |q|.
    i32x4_t qih[C::NB8], qil[C::NB8];
    float qk8 = 1.f;
    if (w >= C::NC) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qb[ks] = u32x4_t{0u, 0u, 0u, 0u};
    } else if constexpr (C::F8MMA) {
        const size_t q0 = qrow_offset(a, row, kvh, 0);
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + q0, (int)(qrow_offset(a, row, kvh, gq - 1) - q0 + D) * 2);
        const int r = g0 + 16 * hw + li;
        const int qoff = r < gq ? (int)(qrow_offset(a, row, kvh, r) - q0) * 2 : kOutOfRange;
        u32x4_t raw[C::NH8][4];
#pragma unroll
        for (int h = 0; h < C::NH8; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                raw[h][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                            qr, qoff + (128 * h + 32 * kg) * 2 + 16 * j, 0, 0));
        __builtin_amdgcn_s_waitcnt(kVmcntStages<0, 0>());
        float mx = 0.f;
#pragma unroll
        for (int h = 0; h < C::NH8; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    mx = fmaxf(mx, fmaxf(fabsf(bf16_lo_f32(raw[h][j][d])), fabsf(bf16_hi_f32(raw[h][j][d]))));
        mx = max_xor32(max_xor16(mx));  // over the head's lanes li, li + 16, li + 32, li + 48
        int qe = 0;
        if (mx > 0.f) {
            int e2;
            (void)frexpf(mx, &e2);  // mx = f 2^e2, f in [0.5, 1)
            qe = 8 - e2;
        }
        qk8 = __builtin_amdgcn_ldexpf(1.f, -qe);
#pragma unroll
        for (int h = 0; h < C::NH8; ++h)
#pragma unroll
            for (int dw = 0; dw < 8; ++dw) {
                const uint32_t w0 = raw[h][dw >> 1][2 * (dw & 1)], w1 = raw[h][dw >> 1][2 * (dw & 1) + 1];
                const float x0 = __builtin_amdgcn_ldexpf(bf16_lo_f32(w0), qe);
                const float x1 = __builtin_amdgcn_ldexpf(bf16_hi_f32(w0), qe);
                const float x2 = __builtin_amdgcn_ldexpf(bf16_lo_f32(w1), qe);
                const float x3 = __builtin_amdgcn_ldexpf(bf16_hi_f32(w1), qe);
                int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
                hi = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hi, true);
                int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - __builtin_amdgcn_cvt_f32_fp8(hi, 0),
                                                         x1 - __builtin_amdgcn_cvt_f32_fp8(hi, 1), 0, false);
                lo = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - __builtin_amdgcn_cvt_f32_fp8(hi, 2),
                                                     x3 - __builtin_amdgcn_cvt_f32_fp8(hi, 3), lo, true);
                qh[h][dw] = hi;
                ql[h][dw] = lo;
            }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qb[ks] = u32x4_t{0u, 0u, 0u, 0u};
    } else if constexpr (C::I8MMA) {
        const size_t q0 = qrow_offset(a, row, kvh, 0);
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + q0, (int)(qrow_offset(a, row, kvh, gq - 1) - q0 + D) * 2);
        const int r = g0 + 16 * hw + li;
        const int qoff = r < gq ? (int)(qrow_offset(a, row, kvh, r) - q0) * 2 : kOutOfRange;
        u32x4_t raw[C::NB8][2];
#pragma unroll
        for (int b = 0; b < C::NB8; ++b)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                raw[b][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                            qr, qoff + (64 * b + 16 * kg) * 2 + 16 * j, 0, 0));
        __builtin_amdgcn_s_waitcnt(kVmcntStages<0, 0>());
        float mx = 0.f;
#pragma unroll
        for (int b = 0; b < C::NB8; ++b)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    mx = fmaxf(mx, fmaxf(fabsf(bf16_lo_f32(raw[b][j][d])), fabsf(bf16_hi_f32(raw[b][j][d]))));
        mx = max_xor32(max_xor16(mx));
        int qe = 0;
        if (mx > 0.f) {
            int e2;
            (void)frexpf(mx, &e2);  // mx = f 2^e2, f in [0.5, 1)
            qe = 13 - e2;
        }
        qk8 = __builtin_amdgcn_ldexpf(1.f, -qe);
#pragma unroll
        for (int b = 0; b < C::NB8; ++b)
#pragma unroll
            for (int dw = 0; dw < 4; ++dw) {
                // codes 4dw .. 4dw + 3 of the lane's 16: bf16 elements of raw[b][dw / 2]
                const uint32_t w0 = raw[b][dw >> 1][2 * (dw & 1)], w1 = raw[b][dw >> 1][2 * (dw & 1) + 1];
                const float xs[4] = {bf16_lo_f32(w0), bf16_hi_f32(w0), bf16_lo_f32(w1), bf16_hi_f32(w1)};
                uint32_t hi = 0u, lo = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int Q = (int)__builtin_rintf(__builtin_amdgcn_ldexpf(xs[e], qe));
                    const int qh8 = (Q + 64) >> 7;  // round(Q / 128), |qh8| <= 64
                    const int ql8 = Q - 128 * qh8;  // in [-64, 64)
                    hi |= (uint32_t)(qh8 & 0xFF) << (8 * e);
                    lo |= (uint32_t)(ql8 & 0xFF) << (8 * e);
                }
                qih[b][dw] = (int)hi;
                qil[b][dw] = (int)lo;
            }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qb[ks] = u32x4_t{0u, 0u, 0u, 0u};
    } else {
        // the unit's query rows span T tokens, Hq * D elements apart
        const size_t q0 = qrow_offset(a, row, kvh, 0);
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + q0, (int)(qrow_offset(a, row, kvh, gq - 1) - q0 + D) * 2);
        const int r = g0 + 16 * hw + li;
        const int qoff = r < gq ? (int)(qrow_offset(a, row, kvh, r) - q0) * 2 : kOutOfRange;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            qb[ks] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                      qr, qoff + ks * 64 + kg * 16, 0, 0));
        // A compute wave can do nothing before q; waiting here also tells the
        // compiler that no load is pending into registers the loop reads.
        __builtin_amdgcn_s_waitcnt(kVmcntStages<0, 0>());
    }

    // The fetch waits in the memory system behind other workgroups' fetches;
    // issued here, after this wave's last wait for loads before the loop
    // ends, it delays nothing until then.
    if (next != nullptr && tid == 0) *next = (long long)gridDim.x + atomicAdd(&a.queue[0], 1u);

    // Issue a loader's share of the loads of tile `tile` into ring slot
    // tile % STAGES (compute waves issue nothing).  Load jj (0 .. LOADS-1)
    // covers 1 KB of the K tile and, with a second load, the same 1 KB of the
    // V tile; loader l issues jj = l, l + NL, ..., KPW of each.
    // Paged cache: a loader keeps the chunk's page indices in its lanes (lane
    // i: block (p0 >> page_shift) + i) when they fit in a wave, so no block
    // table load sits on the issue path; otherwise each tile looks it up.
    const int blk0 = a.block_table ? (p0 >> a.page_shift) : 0;
    const int nblk = (a.block_table && p1 > p0) ? ((p1 - 1) >> a.page_shift) - blk0 + 1 : 0;
    const bool pages_in_lanes = nblk > 0 && nblk <= 64;
    int chunk_page = 0;
    if (pages_in_lanes && w >= C::NC) {
        if (lane < nblk) chunk_page = a.block_table[(size_t)b * a.max_blocks + blk0 + lane];
        // the first tile's address needs it anyway; waiting here also tells the
        // compiler that no load into it is pending inside the loop
        __builtin_amdgcn_s_waitcnt(kVmcntStages<0, 0>());
    }
    auto tile_loc = [&](int t0) {
        if (pages_in_lanes)
            return page_loc(a, __builtin_amdgcn_readlane(chunk_page, (t0 >> a.page_shift) - blk0), kvh, t0);
        return kv_loc(a, b, kvh, t0);
    };
    auto issue_tile = [&](int tile) {
        if (w < C::NC) return;
        const int t0 = p0 + tile * C::STEP;
        const int rows = max(0, min(C::STEP, p1 - t0));
        const int skip = lo - t0;  // rows before a sliding window (> 0 in the first tile only)
        const RowLoc loc = rows > 0 ? tile_loc(t0) : RowLoc{0, 0};
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(row_ptr<C::EB>(a.k, a, loc.row), rows * rowbytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(row_ptr<C::EB>(a.v, a, loc.row), rows * rowbytes);
        unsigned char* slot = smem + (tile % C::STAGES) * C::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < C::KPW; ++i) {
            const int jj = (w - C::NC) + C::NL * i;
            const int p = jj * 64 + lane;  // 16-byte LDS slot in the tile
            const int t = p / C::CPR, cs = p % C::CPR;
            const int voff = t < skip ? kOutOfRange : t * rowbytes + ((cs ^ tile_key<FMT, D>(t)) * 16);
            unsigned char* dst = slot + jj * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)dst, 16, voff, 0, 0, kCachePolicyNT);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(dst + C::TILE_BYTES), 16, voff, 0, 0,
                                                     kCachePolicyNT);
        }
        if constexpr (C::Q8) {
            // the tile rows' scales (contiguous per kv head): loader 0 the K
            // scales, loader 1 the V scales, one dword per lane of the first 32
            const float* sc = (w == C::NC ? a.k_scale : a.v_scale) + loc.scale;
            const __amdgpu_buffer_rsrc_t srs = make_rsrc(sc, rows * 4);
            if (lane < C::STEP)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_ptr_t)(slot + 2 * C::TILE_BYTES + (w - C::NC) * 128), 4,
                                                         lane < skip ? kOutOfRange : lane * 4, 0, 0, kCachePolicyNT);
        }
    };
    // A step's PT tiles go into ring slots PT (step mod GSTAGES) .. +PT-1.
    auto issue_step = [&](int step) {
#pragma unroll
        for (int u = 0; u < C::PT; ++u) issue_tile(C::PT * step + u);
    };
    // In a loader, the next step's tiles and everything before them have
    // landed once at most GSTAGES - 3 later steps are outstanding; in every
    // wave no LDS read is pending.  The barrier then publishes the loaders'
    // tiles and frees the slots refilled next.  A plain s_barrier, not
    // __syncthreads: the latter's release fence would also wait for the loads
    // still in flight to the ring.
    // The first sync allows one more step outstanding: the prologue issued
    // every free slot's step.
    auto ring_sync = [&](auto later_steps) {
        constexpr int N = decltype(later_steps)::value;
        __builtin_amdgcn_s_waitcnt(kVmcntStages<N, C::PT * C::PER_WAVE>() & ~(0xF << 8));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t oacc[C::MT];  // O^T tile m: rows d = 16m .. 16m+15, column = head
#pragma unroll
    for (int j = 0; j < C::MT; ++j) oacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float qk = a.qk_log2;
    const float qkq = (C::F8MMA || C::I8MMA) ? qk * qk8 : qk;  // 8-bit logits: undo q's power-of-two scaling

    // S^T = K q^T for one tile: A = two 16-row K tiles read from LDS, B = q^T.
    // Accumulator lane (li, kg), element r of tile mq: head li, position 16mq + 4kg + r.
    // Even and odd k-steps accumulate separately (four independent chains on
    // the matrix pipe), summed at the end.
    // 8-bit tiles: lane (li, kg) of k-step ks reads the 8 codes of row t,
    // columns 32 ks + 8 kg .. +7: half kg & 1 of chunk 2 ks + kg / 2.
    int k8_row[2], k8_key[2];
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
        const int t = 16 * mq + li;
        k8_row[mq] = t * C::ROWB + (kg & 1) * 8;
        k8_key[mq] = (tile_key<FMT, D>(t) ^ (kg >> 1)) * 16;
    }
    // fp8 matrix cores: lane (li, kg) reads, for row 16mq + li and half h,
    // the 32 codes 128h + 32kg .. +31 (chunks 8h + 2kg and 8h + 2kg + 1)
    int f8_off[2][C::NH8][2];
#pragma unroll
    for (int mq = 0; mq < 2; ++mq)
#pragma unroll
        for (int h = 0; h < C::NH8; ++h)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int t = 16 * mq + li;
                f8_off[mq][h][x] = t * C::ROWB + (((8 * h + 2 * kg + x) ^ tile_key<FMT, D>(t)) * 16);
            }
    // int8 matrix cores: lane (li, kg) reads, for row 16mq + li and block b,
    // the 16 codes 64b + 16kg .. +15 (chunk 4b + kg)
    int i8_off[2][C::NB8];
#pragma unroll
    for (int mq = 0; mq < 2; ++mq)
#pragma unroll
        for (int b = 0; b < C::NB8; ++b) {
            const int t = 16 * mq + li;
            i8_off[mq][b] = t * C::ROWB + (((4 * b + kg) ^ tile_key<FMT, D>(t)) * 16);
        }
    auto qk_tile = [&](int soff, f32x4_t (&sacc)[2]) {
        const unsigned char* kt = smem + soff;
        if constexpr (C::I8MMA) {
            i32x4_t part[2][2];  // [mq][hi or lo part of q]
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) part[mq][0] = part[mq][1] = i32x4_t{0, 0, 0, 0};
            // every K read of the tile first, then the products: the
            // scheduling barrier keeps the compiler from interleaving them
            // (it otherwise may keep only a few reads ahead, each product
            // then waiting for its read: MI355X, int8 B=4 len 131072 83.5
            // against 77.7 us)
            i32x4_t ka[C::NB8][2];
#pragma unroll
            for (int b = 0; b < C::NB8; ++b)
#pragma unroll
                for (int mq = 0; mq < 2; ++mq)
                    ka[b][mq] = __builtin_bit_cast(i32x4_t, *reinterpret_cast<const u32x4_t*>(kt + i8_off[mq][b]));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < C::NB8; ++b)
#pragma unroll
                for (int mq = 0; mq < 2; ++mq) {
                    part[mq][0] = mfma_16x16x64_i8(ka[b][mq], qih[b], part[mq][0]);
                    part[mq][1] = mfma_16x16x64_i8(ka[b][mq], qil[b], part[mq][1]);
                }
#pragma unroll
            for (int mq = 0; mq < 2; ++mq)
#pragma unroll
                for (int r = 0; r < 4; ++r)  // |128 hi + lo| sums stay below 2^24: exact in fp32
                    sacc[mq][r] = (float)(128 * part[mq][0][r] + part[mq][1][r]);
            return;
        }
        if constexpr (C::F8MMA) {
            f32x4_t part[2][2];  // [mq][high or low part of q]
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) part[mq][0] = part[mq][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // every K read of the tile first, then the products (as above)
            u32x4_t kr[C::NH8][2][2];
#pragma unroll
            for (int h = 0; h < C::NH8; ++h)
#pragma unroll
                for (int mq = 0; mq < 2; ++mq)
#pragma unroll
                    for (int x = 0; x < 2; ++x)
                        kr[h][mq][x] = *reinterpret_cast<const u32x4_t*>(kt + f8_off[mq][h][x]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < C::NH8; ++h)
#pragma unroll
                for (int mq = 0; mq < 2; ++mq) {
                    const u32x4_t k0 = kr[h][mq][0], k1 = kr[h][mq][1];
                    const i32x8_t ka = {(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                                        (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
                    part[mq][0] = mfma_16x16x128_fp8(ka, qh[h], part[mq][0]);
                    part[mq][1] = mfma_16x16x128_fp8(ka, ql[h], part[mq][1]);
                }
            sacc[0] = part[0][0] + part[0][1];
            sacc[1] = part[1][0] + part[1][1];
            return;
        }
        f32x4_t part[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) part[h][mq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) {
                u32x4_t ka;
                if constexpr (C::Q8) {
                    const u32x2_t k8 =
                        *reinterpret_cast<const u32x2_t*>(kt + k8_row[mq] + (k8_key[mq] ^ (2 * ks * 16)));
                    ka = widen8<FMT>(k8);
                } else {
                    const int t = 16 * mq + li;
                    ka = *reinterpret_cast<const u32x4_t*>(kt + swz<D>(t, 4 * ks + kg));
                }
                part[ks & 1][mq] = mfma_16x16x32_bf16(ka, qb[ks], part[ks & 1][mq]);
            }
        }
        // Keep eight K reads ahead of the matrix products (the LDS latency of
        // a read spans several products): eight reads, then one product and
        // one read alternately, then the last eight products.
        // (bf16 tiles only: the widening of 8-bit codes sits between a read
        // and its product, and pinning the order there measured slower)
        if constexpr (!C::Q8) {
            constexpr int NQ = 2 * C::KS;  // reads = products of this tile
            constexpr int AHEAD = NQ / 2 < 8 ? NQ / 2 : 8;
            __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
            static_for<0, NQ - AHEAD>([&](auto) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            });
            __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
        }
        sacc[0] = part[0][0] + part[1][0];
        sacc[1] = part[0][1] + part[1][1];
    };
    // Scale, mask the tail, lazy online softmax; P^T of the tile in registers.
    // Returns whether the running maximum moved (then O must be rescaled by alpha).
    // Query row of this lane's column: token i = (g0 + 16w + li) / G may
    // attend positions below lim = qbase + i + 1 (none for a token before the
    // sequence start); tiles reaching past tmask hold a position some column
    // must not see.
    const int qpos = qbase + (g0 + 16 * hw + li) / a.G;
    const int lim = min(p1, qpos + 1);
    const int tmask = p1 - a.T + 1;
    // 8-bit caches: the logit of a position is scaled by its K row's scale,
    // and its weight in P.V by its V row's scale (l sums the unscaled weights).
    // First part: scale the logits and mask the positions a column must not
    // see (a rare, uniform branch); vsc gets the V scales of 8-bit tiles.
    auto softmax_prep = [&](int tile, int soff, f32x4_t (&sacc)[2], f32x4_t (&vsc)[2]) {
        const int st = p0 + tile * C::STEP;
        if constexpr (C::Q8) {
            const float* scl = reinterpret_cast<const float*>(smem + soff + 2 * C::TILE_BYTES);
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) {
                const f32x4_t ksc = *reinterpret_cast<const f32x4_t*>(scl + 16 * mq + 4 * kg);
                vsc[mq] = *reinterpret_cast<const f32x4_t*>(scl + C::STEP + 16 * mq + 4 * kg);
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[mq][r] *= qkq * ksc[r];
            }
        } else {
#pragma unroll
            for (int mq = 0; mq < 2; ++mq)
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[mq][r] *= qk;
        }
        if (st + C::STEP > tmask || st < lo) {
#pragma unroll
            for (int mq = 0; mq < 2; ++mq)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = st + 16 * mq + 4 * kg + r;
                    sacc[mq][r] = (t < lim && t >= lo) ? sacc[mq][r] : -INFINITY;
                }
        }
    };
    // Second part: the online softmax proper, free of branches so that it can
    // share a basic block (and the issue slots) with the matrix products.
    // It takes the PT tiles of a step at once: one maximum, one rescale test.
    auto softmax_finish = [&](f32x4_t (&sacc)[C::NU][2], const f32x4_t (&vsc)[C::NU][2], u32x4_t (&pb)[C::NU],
                              float& alpha) {
        auto tile_max = [](const f32x4_t (&x)[2]) {
            return fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                         fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
        };
        float mx = tile_max(sacc[0]);
#pragma unroll
        for (int u = 1; u < C::NU; ++u) mx = fmaxf(mx, tile_max(sacc[u]));
        mx = max_xor32(max_xor16(mx));
        const bool moved = mx > m_run + kRescaleSlack;
        alpha = moved ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
        m_run = moved ? mx : m_run;
        // a column with no visible position yet (a later query token's limit
        // can lie past a whole tile) keeps m = -inf; its weights are zero
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float lsum = 0.f;
#pragma unroll
        for (int u = 0; u < C::NU; ++u)
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) {
                if constexpr (C::Q8) {
                    float pr[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pr[r] = __builtin_amdgcn_exp2f(sacc[u][mq][r] - m_use);
                        lsum += pr[r];
                    }
                    pb[u][2 * mq] = pack2_bf16_rne(pr[0] * vsc[u][mq][0], pr[1] * vsc[u][mq][1]);
                    pb[u][2 * mq + 1] = pack2_bf16_rne(pr[2] * vsc[u][mq][2], pr[3] * vsc[u][mq][3]);
                } else {
                    const uint32_t lo = pack2_bf16_rne(__builtin_amdgcn_exp2f(sacc[u][mq][0] - m_use),
                                                       __builtin_amdgcn_exp2f(sacc[u][mq][1] - m_use));
                    const uint32_t hi = pack2_bf16_rne(__builtin_amdgcn_exp2f(sacc[u][mq][2] - m_use),
                                                       __builtin_amdgcn_exp2f(sacc[u][mq][3] - m_use));
                    pb[u][2 * mq] = lo;
                    pb[u][2 * mq + 1] = hi;
                    lsum += (bf16_lo_f32(lo) + bf16_hi_f32(lo)) + (bf16_lo_f32(hi) + bf16_hi_f32(hi));
                }
            }
        l_run = l_run * alpha + lsum;
        return __any(moved);
    };
    // O^T += V^T P^T for one tile.  The A operand (row d = 16m + li, eight
    // positions per lane group) comes straight from LDS with transposing
    // reads: in each 16-lane group, lane 4j + b points at the 8 bytes
    // d = 16m + 4b .. +3 of position row j, and lane li receives column
    // 16m + li of the four rows.  Element e of lane group kg is position
    // 16*(e/4) + 4*kg + e%4, the order of the P^T operand.
    //   Chunk 2m + x (x = 0, 1) of row t sits at the slot of chunk
    // 2(m mod NR) + x plus 2 NR (m div NR) (see kSwzRegs), so NR address
    // registers per row and constant offsets cover all m.
    constexpr int NR = kSwzRegs<D>;
    const int tr_j = li >> 2, tr_b = li & 3;
    const int tr_tlo = 4 * kg + tr_j, tr_thi = 16 + 4 * kg + tr_j;
    const int tr_lo = swz<D>(tr_tlo, tr_b >> 1) + (tr_b & 1) * 8;  // m = 0
    const int tr_hi = swz<D>(tr_thi, tr_b >> 1) + (tr_b & 1) * 8;
    // 8-bit tiles: one ds_read_b64_tr_b8 per 16-row tile m of d.  In lane
    // group kg, lane 2k + x points at the 8 codes d = 16m + 8x .. +7 of
    // position row 16 (k / 4) + 4 kg + k % 4, so lane li receives column
    // 16m + li of the eight positions in the P^T order.
    const int tr8_t = 16 * ((li >> 1) >> 2) + 4 * kg + ((li >> 1) & 3);
    const int tr8_row = tr8_t * C::ROWB + (li & 1) * 8;
    const int tr8_key = tile_key<FMT, D>(tr8_t) * 16;
    // P.V runs in two halves of d (tiles m < MT/2, then the rest), so the
    // V^T operands of only one half occupy registers at a time.
    constexpr int MH = C::MT / 2;
    auto pv_issue = [&](int soff, auto half, u32x2_t (&lo)[MH], u32x2_t (&hi)[MH]) {
        constexpr int M0 = decltype(half)::value * MH;
        const uint32_t vbase = lds_addr(smem + soff + C::TILE_BYTES);
        if constexpr (C::Q8) {
#pragma unroll
            for (int j = 0; j < MH; ++j)
                lo[j] = ds_read_tr8_b64_asm(vbase + tr8_row + (tr8_key ^ ((M0 + j) * 16)));
        } else {
            issue_vt_tile<M0, MH, NR>(vbase + tr_lo, vbase + tr_hi, lo, hi);
        }
    };
    auto pv_mma = [&](const u32x4_t& pb, auto half, u32x2_t (&lo)[MH], u32x2_t (&hi)[MH]) {
        constexpr int M0 = decltype(half)::value * MH;
        if constexpr (C::Q8)
            wait_v8_tile<MH>(lo);
        else
            wait_vt_tile<MH>(lo, hi);
#pragma unroll
        for (int j = 0; j < MH; ++j) {
            u32x4_t va;
            if constexpr (C::Q8)
                va = widen8<FMT>(lo[j]);
            else
                va = u32x4_t{lo[j].x, lo[j].y, hi[j].x, hi[j].y};
            oacc[M0 + j] = mfma_16x16x32_bf16(va, pb, oacc[M0 + j]);
        }
    };

    // Prologue: steps 0 .. GSTAGES-2 in flight, every slot the loop does not
    // refill first (tiles past the end read nothing).  They are issued before
    // the first barrier, which waits for the compute waves' q as well.
#pragma unroll
    for (int st = 0; st < C::GSTAGES - 1; ++st) issue_step(st);

    // Software pipeline: step `step` computes q.K of step + 1 with its
    // softmax and P.V of `step` (P^T made in the previous step), so the matrix
    // pipe and the vector ALU overlap inside each wave.  Order inside a step:
    // q.K of the next step (its K reads kept eight ahead), the V^T reads of
    // the first half of d and the logit scaling while they land; then, in one
    // basic block, P.V of the first half with the second half's V^T reads in
    // its shadow, the rest of the softmax while those land, P.V of the second
    // half.  A wave issues in order, and one 16x16x32 product takes about 17
    // cycles to issue but about 50 before a dependent one may start (MI355X),
    // so the order decides how much of the step is waiting.  Ring slots in use
    // during a step: those of `step` and step + 1; the step refills the slots
    // of step - 1 with step + GSTAGES - 1, so GSTAGES - 2 steps stay in flight.
    constexpr std::integral_constant<int, 0> first_half{};
    constexpr std::integral_constant<int, 1> second_half{};
    auto slot_off = [](int tile) { return (tile % C::STAGES) * C::STAGE_BYTES; };
    u32x4_t pb[C::NU];
#pragma unroll
    for (int u = 0; u < C::NU; ++u) pb[u] = u32x4_t{0u, 0u, 0u, 0u};
    if (nsteps > 0) {
        ring_sync(std::integral_constant<int, C::GSTAGES - 2>{});  // step 0 landed
        if (w < C::NC) {
            f32x4_t sacc[C::NU][2], vsc[C::NU][2];
#pragma unroll
            for (int u = 0; u < C::NU; ++u) qk_tile(slot_off(u0 + u), sacc[u]);
#pragma unroll
            for (int u = 0; u < C::NU; ++u) softmax_prep(u0 + u, slot_off(u0 + u), sacc[u], vsc[u]);
            float alpha;
            softmax_finish(sacc, vsc, pb, alpha);  // O is still zero: no rescale
        }
    }
    for (int step = 0; step < nsteps; ++step) {
        const int t0 = C::PT * step + u0, t1 = t0 + C::PT;  // this wave's first tile of this step and of the next
        ring_sync(std::integral_constant<int, C::GSTAGES - 3>{});  // step + 1 landed (no-op reads past the end)
        issue_step(step + C::GSTAGES - 1);
        if (w >= C::NC) continue;  // the load-only wave
        u32x2_t vlo[C::NU][MH], vhi[C::NU][MH];
        f32x4_t sacc[C::NU][2], vsc[C::NU][2];
        if (step + 1 < nsteps) {
            // q.K of the next step first: the V^T reads issued after its
            // K reads land while its products and the logit scaling run
#pragma unroll
            for (int u = 0; u < C::NU; ++u) qk_tile(slot_off(t1 + u), sacc[u]);
#pragma unroll
            for (int u = 0; u < C::NU; ++u) pv_issue(slot_off(t0 + u), first_half, vlo[u], vhi[u]);
#pragma unroll
            for (int u = 0; u < C::NU; ++u) softmax_prep(t1 + u, slot_off(t1 + u), sacc[u], vsc[u]);
        } else {
#pragma unroll
            for (int u = 0; u < C::NU; ++u) pv_issue(slot_off(t0 + u), first_half, vlo[u], vhi[u]);
            // past the last step: all logits -inf, so the softmax step below
            // leaves m and l unchanged (the max does not move, every weight is 0)
#pragma unroll
            for (int u = 0; u < C::NU; ++u)
#pragma unroll
                for (int mq = 0; mq < 2; ++mq) {
                    sacc[u][mq] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                    vsc[u][mq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
        }
        // One basic block from here (the softmax finish is branch-free): P.V of
        // this step and the softmax of the next, whose vector instructions
        // issue while the products run.
#pragma unroll
        for (int u = 0; u < C::NU; ++u) pv_mma(pb[u], first_half, vlo[u], vhi[u]);
#pragma unroll
        for (int u = 0; u < C::NU; ++u) pv_issue(slot_off(t0 + u), second_half, vlo[u], vhi[u]);
        u32x4_t pb_next[C::NU];
        float alpha;
        const bool moved = softmax_finish(sacc, vsc, pb_next, alpha);
        // tie the softmax results here so the compiler cannot sink their
        // computation below the products (or past the rescale branch)
#pragma unroll
        for (int u = 0; u < C::NU; ++u) asm volatile("" : "+v"(pb_next[u]));
        asm volatile("" : "+v"(l_run), "+v"(alpha));
#pragma unroll
        for (int u = 0; u < C::NU; ++u) pv_mma(pb[u], second_half, vlo[u], vhi[u]);
        if constexpr (!C::Q8) {
            // products and vector instructions alternate
            static_for<0, 2 * MH>([&](auto) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);
            });
        }
#pragma unroll
        for (int u = 0; u < C::NU; ++u) pb[u] = pb_next[u];
        if (moved) {
#pragma unroll
            for (int m = 0; m < C::MT; ++m) oacc[m] = oacc[m] * alpha;
        }
    }

    // No buffer->LDS load of this workgroup may still be landing when its LDS
    // is released (the ring's tail loads read nothing, so this is quick).
    __builtin_amdgcn_s_waitcnt(0);

    // Tiles split between waves: the second wave of each 16-row tile hands
    // its state (m, the lane's part of l, O) to the first through LDS, which
    // merges the two online softmaxes.
    if constexpr (C::SUBS > 1) {
        static_assert(C::SUBS == 2, "pairs of waves");
        constexpr int XV = C::MT + 1;  // 16-byte values per lane: O, then {m, l}
        static_assert(NG * 64 * XV * 16 <= C::LDS_BYTES, "exchange area");
        f32x4_t* xo = reinterpret_cast<f32x4_t*>(smem) + hw * 64 * XV + lane;
        __syncthreads();  // every wave is done with the ring
        if (w >= NG && w < C::NC) {
#pragma unroll
            for (int m = 0; m < C::MT; ++m) xo[64 * m] = oacc[m];
            xo[64 * C::MT] = f32x4_t{m_run, l_run, 0.f, 0.f};
        }
        __syncthreads();
        if (w < NG) {
            const f32x4_t ml = xo[64 * C::MT];
            const float m1 = ml[0], l1 = ml[1];
            const float mm = fmaxf(m_run, m1);
            // a side that saw no position has m = -inf, l = 0 and O = 0
            const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
            const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
            for (int m = 0; m < C::MT; ++m) oacc[m] = oacc[m] * a0 + xo[64 * m] * a1;
            l_run = l_run * a0 + l1 * a1;
            m_run = mm;
        }
    }

    // ---- epilogue: this wave's 16 heads, no merge with other waves.  The
    // accumulators hold four consecutive d of one head per lane; they go
    // through LDS (the ring is free now) so that every store instruction
    // writes whole contiguous head rows.  LDS rows are padded by 16 bytes so
    // the transposing writes spread over the banks.  A sequence that fits in
    // one chunk writes fp32 output; a chunk of a longer one writes its fp16
    // partial row scaled by 2^-e, and {lse, e}.
    l_run = sum_xor32(sum_xor16(l_run));
    const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
    const bool direct = nsplit == 1;
    __syncthreads();  // every wave is done with the ring
    if (w < NG) {
        const int g = 16 * w + li;  // head inside the block
        if (direct) {
            constexpr int ROWF = D + 4;  // floats per padded LDS row
            float* ot = reinterpret_cast<float*>(smem) + w * 16 * ROWF;
            // accumulator rows 4kg .. 4kg+3 of tile m are d = 16m + 4kg .. +3 of head li
#pragma unroll
            for (int m = 0; m < C::MT; ++m)
                *reinterpret_cast<f32x4_t*>(ot + li * ROWF + 16 * m + 4 * kg) = oacc[m] * inv_l;
            constexpr int LPR = D / 4;     // lanes per row, 16 bytes each
            constexpr int RPI = 64 / LPR;  // rows per store instruction
            const int hr = lane / LPR, c = lane % LPR;
#pragma unroll
            for (int h0 = 0; h0 < 16; h0 += RPI) {
                const int h = h0 + hr;
                if (16 * w + h < gcnt && g0 + 16 * w + h < gq)
                    *reinterpret_cast<f32x4_t*>(a.out + qrow_offset(a, row, kvh, g0 + 16 * w + h) +
                                                4 * c) = *reinterpret_cast<const f32x4_t*>(ot + h * ROWF + 4 * c);
            }
        } else {
            float mx = 0.f;
#pragma unroll
            for (int m = 0; m < C::MT; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(oacc[m][r]));
            const int e = scale_exponent(max_xor32(max_xor16(mx)) * inv_l);
            constexpr int ROWH = D + 8;  // halves per padded LDS row
            uint16_t* ot = reinterpret_cast<uint16_t*>(smem) + w * 16 * ROWH;
#pragma unroll
            for (int m = 0; m < C::MT; ++m) {
                const f32x4_t x = oacc[m] * inv_l;
                const u32x2_t pk = {pack2_f16_rne(__builtin_amdgcn_ldexpf(x[0], -e), __builtin_amdgcn_ldexpf(x[1], -e)),
                                    pack2_f16_rne(__builtin_amdgcn_ldexpf(x[2], -e), __builtin_amdgcn_ldexpf(x[3], -e))};
                *reinterpret_cast<u32x2_t*>(ot + li * ROWH + 16 * m + 4 * kg) = pk;
            }
            const size_t part0 = ((size_t)unit * a.max_splits + s) * a.GT + g0 + 16 * w;  // this wave's first row
            uint16_t* dst = a.part_o + part0 * D;
            // 16-byte device-scope stores (sc1) through a descriptor over the
            // wave's rows: the fused merge reads them from another workgroup,
            // and for the separate merge they measured faster than plain
            // stores (PaLM-shaped MQA, split kernel 25.6 against 26.2 us)
            const __amdgpu_buffer_rsrc_t prs = make_rsrc(dst, 16 * D * 2);
            constexpr int LPR = D / 8;     // lanes per row, 16 bytes (8 halves) each
            constexpr int RPI = 64 / LPR;  // rows per store instruction
            const int hr = lane / LPR, c = lane % LPR;
#pragma unroll
            for (int h0 = 0; h0 < 16; h0 += RPI) {
                const int h = h0 + hr;
                if (16 * w + h < gcnt) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ot + h * ROWH + 8 * c);
                    __builtin_amdgcn_raw_buffer_store_b128(v, prs, (h * D + 8 * c) * 2, 0, kCachePolicyCoherent);
                }
            }
            if (kg == 0 && g < gcnt) {
                store_coherent8(a.part_ml + part0 + li, f32x2_t{m_run + __log2f(l_run), (float)e});
            }
        }
    }
    if constexpr (FUSED) {
        if (direct) return;
        // ---- fused combine: the chunks of this (row, kv head, head block) share the merge
        __syncthreads();
        fused_tail(a, unit, row, kvh, nsplit, g0, gcnt,
                   a.counters + (unit * gridDim.y + by) * kFusedCountersPerUnit, reinterpret_cast<int*>(smem));
    }
}

template <int D, int NG, int FMT, bool FUSED>
__global__ __launch_bounds__(512) void decode_mfma_kernel(DecodeArgs a) {
    decode_item<D, NG, FMT, FUSED>(a, blockIdx.x, blockIdx.y, nullptr);
}

// Persistent form: gridDim.x workgroups (as many as are resident at once)
// keep taking work items until none is left, so a workgroup that finishes a
// short chunk starts the next item at once instead of waiting for the
// hardware to dispatch a new workgroup in grid order, and a faster XCD takes
// more items than a slower one.  Workgroup x first takes item x, then items
// gridDim.x + k for k from the queue counter.  (Device-scope atomics on one
// address are serialized; the static first item keeps them off the start of
// the kernel's critical path.)  Thread 0 fetches the following item while the
// current one runs (once its wave has q, or at once for a chunk past the
// sequence's end); the item number reaches the other waves through the 16
// bytes after the kernel's LDS block.  The last workgroup to leave puts both
// counters back to zero for the next call.  Items do not depend on which
// workgroup runs them, so the result is the plain form's, bit for bit.
template <int D, int NG, int FMT>
__global__ __launch_bounds__(512) void decode_mfma_persistent_kernel(DecodeArgs a) {
    using C = MfmaCfg<D, NG, FMT>;
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    volatile long long* slot = reinterpret_cast<volatile long long*>(smem + C::LDS_BYTES);
    const int tid = threadIdx.x;
    long long item = blockIdx.x;
    long long next;  // thread 0: the following item, fetched inside each item
    while (item < a.items) {
        next = a.items;  // (every path through an item fetches; this only ends the loop if one did not)
        decode_item<D, NG, FMT, false>(a, item % a.grid_x, (int)(item / a.grid_x), &next);
        __syncthreads();  // every wave is done with this item's LDS
        if (tid == 0) slot[0] = next;
        __syncthreads();
        item = slot[0];
    }
    if (tid == 0) {
        // every workgroup's last fetch came before its arrival here
        if (atomicAdd(&a.queue[1], 1u) == gridDim.x - 1) {
            atomicExch(&a.queue[0], 0u);
            atomicExch(&a.queue[1], 0u);
        }
    }
}

template <int D, int NG, int FMT, bool FUSED>
static hipError_t launch_mfma_form(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                                   hipEvent_t ev1) {
    using C = MfmaCfg<D, NG, FMT>;
    constexpr int lds = C::LDS_BYTES;
    if (lds > 64 * 1024) {
        static std::atomic<uint64_t> done_mask{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = 1ull << (dev & 63);
        if (!(done_mask.load() & bit)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_mfma_kernel<D, NG, FMT, FUSED>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
            done_mask.fetch_or(bit);
        }
    }
    const dim3 grid((unsigned)p.grid_main, (unsigned)p.head_blocks);
    const dim3 block(C::THREADS);
    if (ev0 || ev1)
        hipExtLaunchKernelGGL((decode_mfma_kernel<D, NG, FMT, FUSED>), grid, block, lds, stream, ev0, ev1, 0, a);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<D, NG, FMT, FUSED>), grid, block, lds, stream, a);
    return hipGetLastError();
}

template <int D, int NG, int FMT>
static hipError_t launch_mfma_persistent(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                                         hipEvent_t ev1) {
    using C = MfmaCfg<D, NG, FMT>;
    constexpr int lds = C::LDS_BYTES + 16;  // + the item slot
    static_assert(lds <= 160 * 1024, "LDS budget of a gfx950 CU");
    const void* fn = reinterpret_cast<const void*>(&decode_mfma_persistent_kernel<D, NG, FMT>);
    // workgroups resident at once on each device (0 until known)
    constexpr int kMaxDevices = 64;
    static std::atomic<int> resident[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int wgs = resident[dev].load();
    if (wgs == 0) {
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        int per_cu = 0, cus = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, C::THREADS, lds);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        wgs = per_cu * cus;
        if (wgs <= 0) return hipErrorInvalidConfiguration;
        resident[dev].store(wgs);
    }
    const long long items = p.grid_main * p.head_blocks;
    const dim3 grid((unsigned)(items < wgs ? items : wgs));
    const dim3 block(C::THREADS);
    if (ev0 || ev1)
        hipExtLaunchKernelGGL((decode_mfma_persistent_kernel<D, NG, FMT>), grid, block, lds, stream, ev0, ev1, 0, a);
    else
        hipLaunchKernelGGL((decode_mfma_persistent_kernel<D, NG, FMT>), grid, block, lds, stream, a);
    return hipGetLastError();
}

template <int D, int NG, int FMT>
static hipError_t launch_mfma(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1) {
    if (p.persist > 0 && !a.fused) return launch_mfma_persistent<D, NG, FMT>(p, a, stream, ev0, ev1);
    return a.fused ? launch_mfma_form<D, NG, FMT, true>(p, a, stream, ev0, ev1)
                   : launch_mfma_form<D, NG, FMT, false>(p, a, stream, ev0, ev1);
}

template <int D, int FMT>
static hipError_t launch_mfma_d(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1) {
    switch (p.heads_per_block / 16) {
        case 1: return launch_mfma<D, 1, FMT>(p, a, stream, ev0, ev1);
        case 2: return launch_mfma<D, 2, FMT>(p, a, stream, ev0, ev1);
        case 3: return launch_mfma<D, 3, FMT>(p, a, stream, ev0, ev1);
        case 4: return launch_mfma<D, 4, FMT>(p, a, stream, ev0, ev1);
        case 5: return launch_mfma<D, 5, FMT>(p, a, stream, ev0, ev1);
        case 6: return launch_mfma<D, 6, FMT>(p, a, stream, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

template <int FMT>
static hipError_t launch_mfma_f(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1) {
    switch (a.D) {
        case 64: return launch_mfma_d<64, FMT>(p, a, stream, ev0, ev1);
        case 128: return launch_mfma_d<128, FMT>(p, a, stream, ev0, ev1);
        case 256: return launch_mfma_d<256, FMT>(p, a, stream, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_mfma(const Plan& p, const DecodeArgs& a, hipStream_t stream, hipEvent_t ev0,
                                    hipEvent_t ev1) {
    switch (p.kv_format) {
        case kKvBf16: return launch_mfma_f<kKvBf16>(p, a, stream, ev0, ev1);
        case kKvFp8: return launch_mfma_f<kKvFp8>(p, a, stream, ev0, ev1);
        case kKvInt8: return launch_mfma_f<kKvInt8>(p, a, stream, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mqa
