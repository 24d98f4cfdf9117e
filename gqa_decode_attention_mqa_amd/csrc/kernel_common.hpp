// Device-side definitions shared by the decode kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace mqa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

// Arguments of the split-K decode kernels, passed by value.
//
// A "row" is one sequence of a decode call (sequence r), bringing T query
// tokens (T > 1: several new tokens decoded at once, causal among
// themselves).  A "unit" is (row, kv head); its T * G query rows (token, head
// in the group) share the unit's keys and values.  A unit's positions are cut into chunks of `chunk` positions,
// one workgroup per (unit, chunk, head block).
struct DecodeArgs {
    const uint16_t* q;         // bf16 [rows, T, Hq, D]
    const void* k;             // [B, Lmax, Hkv, D] (or pages): bf16, or 8-bit codes
    const void* v;             // likewise
    const float* k_scale;      // 8-bit caches: fp32 [B, Hkv, Lmax] (pages: [num_pages, Hkv, page_size]),
    const float* v_scale;      // one per cached row; NULL for bf16
    const int32_t* seq_lens;   // [B]
    float* out;                // fp32 [rows, T, Hq, D]
    uint16_t* part_o;          // fp16 [rows * Hkv * max_splits, T * G, D]: O / l / 2^e per chunk
    f32x2_t* part_ml;          // [rows * Hkv * max_splits, T * G]: {m + log2(l) (base 2), e}
    const int32_t* block_table;  // paged cache: [B, max_blocks] physical page per block of
                                 // 2^page_shift positions; NULL for the contiguous layout
    int page_shift, max_blocks, num_pages;
    uint32_t* counters;        // [rows * Hkv * head_blocks, kFusedCountersPerUnit] counters of the
                               // fused combine; zero between calls (the last arriving chunk wraps its counter)
    long long units;           // rows * Hkv
    int Hq, Hkv, D, Lmax, G;
    int T, GT;                 // query tokens per row; query rows per unit (T * G)
    int chunk, max_splits;
    int window;                // > 0: sliding window, a row of length n attends n-window .. n-1
    int fused;                 // 1: the chunks of a unit merge the partials themselves
    uint32_t fused_wait;       // bound of the fused combine's wait, in 100 MHz real-time ticks
    float qk_log2;             // scale * log2(e): logits are kept in base-2 units
    // Persistent form: a fixed grid of workgroups takes work items (the plain
    // form's workgroups, x fastest) from a queue counter in turn.
    uint32_t* queue;           // {item counter, workgroups done}; zero between calls
    long long items;           // work items: grid_x * head blocks
    long long grid_x;
};

// Arguments of the causal prefill kernel (bf16 q, K and V; fp32 out).
struct PrefillArgs {
    const uint16_t* q;         // bf16 [B, Lmax, Hq, D]
    const uint16_t* k;         // bf16 [B, Lmax, Hkv, D]
    const uint16_t* v;         // likewise
    const int32_t* seq_lens;   // [B], clamped to [0, Lmax]
    float* out;                // fp32 [B, Lmax, Hq, D]
    int B, Hq, Hkv, D, Lmax, G;
    int row_blocks;            // workgroups per (sequence, kv head): ceil(Lmax * G / prefill_rows(D))
    float qk_log2;             // scale * log2(e)
};

struct CombineArgs {
    const uint16_t* part_o;
    const f32x2_t* part_ml;
    const int32_t* seq_lens;
    float* out;
    int Hq, Hkv, D, Lmax, G;
    int T, GT;
    int chunk, max_splits;
    int window;
    int dsplit;                // many-chunk merge: workgroups per query row, each a slice of d
};

// Query row r (0 .. T*G - 1) of unit (row, kv head kvh) is token r / G of the
// row's T query tokens and query head kvh * G + r % G.  Element offset of its
// q (and output) row in the [rows, T, Hq, D] arrays.
__device__ __forceinline__ size_t qrow_offset(const DecodeArgs& a, long long row, int kvh, int r) {
    const int i = r / a.G;
    return (((size_t)row * a.T + i) * a.Hq + (size_t)kvh * a.G + (r - i * a.G)) * (size_t)a.D;
}
// The same for decode rows (combine kernels): [rows, T, Hq, D].
__device__ __forceinline__ size_t qrow_offset(long long row, int T, int Hq, int G, int D, int kvh, int r) {
    const int i = r / G;
    return (((size_t)row * T + i) * Hq + (size_t)kvh * G + (r - i * G)) * (size_t)D;
}

// Buffer offset that lies past the range of every tile descriptor (a tile spans
// at most 32 rows of at most 2^24 bytes): a load from it returns zero and
// touches no memory.
constexpr int kOutOfRange = 0x40000000;

// Positions covered by chunk s (of max_splits) of a row that attends `len`
// positions.  Without a window, chunk s is [s * chunk, (s + 1) * chunk) cut at
// len.  With a window of W positions (local attention: the row sees only its
// last W positions) the first attended position is lo = len - W; the chunks
// then start at base = lo rounded down to a multiple of 32, so tiles and pages
// keep their alignment, and the kernels read positions below lo as zero and
// mask them.  The last chunk runs to len, so it may hold up to 31 positions
// more than `chunk` (the planner sizes max_splits for W positions, not W + 31).
// nsplit is the number of chunks that hold positions (1 for an empty row).
struct ChunkSpan {
    int lo, p0, p1, nsplit;
};
__device__ __forceinline__ ChunkSpan chunk_span(int window, int chunk, int max_splits, int len, int s) {
    ChunkSpan c;
    c.lo = (window > 0 && len > window) ? len - window : 0;
    const int base = c.lo & ~31;
    c.p0 = base + s * chunk;
    c.p1 = s == max_splits - 1 ? len : min(c.p0 + chunk, len);
    const int n = len > base ? (len - base + chunk - 1) / chunk : 1;
    c.nsplit = n < max_splits ? n : max_splits;
    return c;
}

// Where position t0 of kv head kvh of sequence b lives: `row` is the index of
// its D-element cache row (the rows of one position's kv heads are adjacent)
// and `scale` the index of its scale in an 8-bit cache's scale array.  The
// rows t0, t0 + 1, ... a caller reads from there never straddle a page (pages
// hold a power of two >= 32 positions, and every tile or block starts at a
// multiple of its own size <= 32), and neither do their scales.  Only called
// for rows below the sequence length, so the block table entry read is one of
// the sequence's own; page indices outside the pool are clamped into it, so a
// bad table gives wrong data, never a stray read.
struct RowLoc {
    size_t row, scale;
};
__device__ __forceinline__ RowLoc page_loc(const DecodeArgs& a, int page, int kvh, int t0) {
    page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    const size_t off = (size_t)(t0 & ((1 << a.page_shift) - 1));
    return {(((size_t)page << a.page_shift) + off) * a.Hkv + kvh, (((size_t)page * a.Hkv + kvh) << a.page_shift) + off};
}
__device__ __forceinline__ RowLoc kv_loc(const DecodeArgs& a, int b, int kvh, int t0) {
    if (a.block_table) return page_loc(a, a.block_table[(size_t)b * a.max_blocks + (t0 >> a.page_shift)], kvh, t0);
    return {((size_t)b * a.Lmax + t0) * a.Hkv + kvh, ((size_t)b * a.Hkv + kvh) * a.Lmax + t0};
}
// Byte address of cache row `row` of a cache with EB-byte elements.
template <int EB>
__device__ __forceinline__ const unsigned char* row_ptr(const void* cache, const DecodeArgs& a, size_t row) {
    return static_cast<const unsigned char*>(cache) + row * (size_t)a.D * EB;
}

// Attended length of a decode row, with seq_lens clamped to [0, Lmax].
__device__ __forceinline__ void row_extent(const int32_t* seq_lens, long long row, int Lmax, int* b_out,
                                           int* len_out) {
    const int b = (int)row;
    const int lb = seq_lens[b];
    *b_out = b;
    *len_out = lb < 0 ? 0 : (lb > Lmax ? Lmax : lb);
}

// Extent of a row: the cache positions it reads (0 .. len - 1) and the
// position of its token 0, qbase = len - T (token i is the i-th of the T
// newest positions and may attend 0 .. qbase + i; tokens before the sequence
// start attend nothing).
__device__ __forceinline__ void row_extent(const DecodeArgs& a, long long row, int* b_out, int* len_out,
                                           int* qbase_out) {
    row_extent(a.seq_lens, row, a.Lmax, b_out, len_out);
    *qbase_out = *len_out - a.T;
}

// Workgroup -> (unit, chunk).  Consecutive workgroup ids are dispatched to the
// 8 XCDs in turn (id mod 8), and each XCD has its own L2.  When the number of
// units is a multiple of 8, all chunks of a unit are given ids with the same
// residue mod 8, so they run on one XCD and their partials meet in one L2.
__device__ __forceinline__ void map_block(long long x, long long units, int max_splits,
                                          long long* unit, int* split) {
    if ((units & 7) == 0) {
        const long long r = x >> 3;
        *split = (int)(r % max_splits);
        *unit = (r / max_splits) * 8 + (x & 7);
    } else {
        *unit = x / max_splits;
        *split = (int)(x % max_splits);
    }
}

// Buffer resources: raw (unstructured) buffers whose range check makes an
// access at or beyond num_records bytes return zero without touching memory.
constexpr int kBufferFlags = 0x00020000;   // 32-bit data format, as gfx9 raw buffers expect
constexpr int kCachePolicyNT = 2;          // non-temporal: K/V rows are read exactly once

// `base` and `num_bytes` must be uniform across the wave; they are moved to
// scalar registers explicitly, or the compiler would wrap every load in a
// loop over distinct descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int num_bytes) {
    const uint64_t addr = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, __builtin_amdgcn_readfirstlane(num_bytes), kBufferFlags);
}
__device__ __forceinline__ u32x4_t buffer_load_u32x4(__amdgpu_buffer_rsrc_t r, int voffset) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, kCachePolicyNT));
}

// Reductions across the 16-lane rows of a wave without LDS: v_permlane16_swap
// pairs row 0 with 1 and 2 with 3 (lane i meets lane i^16), v_permlane32_swap
// pairs the two halves (lane i meets lane i^32).  Each returns both values.
__device__ __forceinline__ float max_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Two floats -> packed bf16 pair with hardware round-to-nearest-even
// (v_cvt_pk_bf16_f32); `a` lands in the low half.
__device__ __forceinline__ uint32_t pack2_bf16_rne(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo_f32(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// s_waitcnt immediate (gfx9 encoding) that waits until at most STAGES * PER
// vector-memory operations of this wave are outstanding, leaving the LDS and
// export counters unconstrained.  Counts above the 6-bit field wait longer,
// which is always safe.
template <int STAGES, int PER>
constexpr int kVmcntStages() {
    constexpr int n = STAGES * PER > 63 ? 63 : STAGES * PER;
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// Lazy rescaling of the online softmax: the running maximum of a head only
// moves when a tile's maximum exceeds it by more than this many (base-2)
// units, so exp2(s - m) <= 2^8 and the accumulators are rescaled rarely.
constexpr float kRescaleSlack = 8.0f;

// Partial outputs of split chunks are stored as fp16, each (chunk, head) row
// divided by 2^e, the smallest power of two above its largest magnitude, so
// every stored value lies in (-1, 1): the fp16 range can never overflow and
// the rounding is at most 2^-11 of the row's largest value.  e travels with
// the chunk's log-sum-exp; the combine restores values with an exact ldexp.
__device__ __forceinline__ int scale_exponent(float max_abs) {
    return max_abs > 0.f ? __builtin_amdgcn_frexp_expf(max_abs) : 0;
}
__device__ __forceinline__ uint32_t pack2_f16_rne(float a, float b) {
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ float f16_lo_f32(uint32_t pair) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi_f32(uint32_t pair) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair >> 16));
}

// DPP lane permutations used inside 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each 8-lane half row
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within each 16-lane row
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane (i+8) mod 16 within the row
constexpr int kDppRowRor4 = 0x124;       // lane i <- lane (i+4) mod 16 within the row

// Maximum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
    return max_xor32(max_xor16(x));
}

__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16x16x128 product of E4M3 codes (gfx950), unscaled (E8M0 scale 127 = 2^0).
// Lane (i, g) of A holds 32 codes of row i and lane (i, g) of B 32 codes of
// column i, for the same 32 values of k: the sum over k does not depend on
// which k the hardware gives each byte, as long as A and B agree.
__device__ __forceinline__ f32x4_t mfma_16x16x128_fp8(const i32x8_t& a, const i32x8_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16x16x64 product of int8 values with int32 accumulation (gfx950); the
// same agreement of A and B on each byte's k as above.
__device__ __forceinline__ i32x4_t mfma_16x16x64_i8(const i32x4_t& a, const i32x4_t& b, const i32x4_t& c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// v_perm_b32 byte select: result bytes = sel over {hi: bytes 4..7, lo: bytes 0..3}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}
constexpr uint32_t kPermLoHalves = 0x05040100u;  // (lo.lo16) | (hi.lo16 << 16)
constexpr uint32_t kPermHiHalves = 0x07060302u;  // (lo.hi16) | (hi.hi16 << 16)

// Cache element formats (the values of mqa_kv_format).
constexpr int kKvBf16 = 0;
constexpr int kKvFp8 = 1;   // E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; 0x7F/0xFF NaN
constexpr int kKvInt8 = 2;  // two's complement

// Eight 8-bit codes (two dwords, code i in byte i % 4 of dword i / 4) widened
// to eight bf16 values, element i in the low half of dword i / 2 for even i.
// Exact: every E4M3 value and every int8 is a bf16 number.
template <int FMT>
__device__ __forceinline__ u32x4_t widen8(u32x2_t c) {
    if constexpr (FMT == kKvFp8) {
        // v_cvt_scalef32_pk_bf16_fp8 with scale 1: codes of bytes 0,1 (or 2,3) -> two bf16
        return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true))};
    } else {
        // sign-extend each byte, convert to f32 (exact), keep the upper half of the bits
        auto pair = [](uint32_t w, int sh) {
            const float lo = (float)(int)(int8_t)(w >> sh);
            const float hi = (float)(int)(int8_t)(w >> (sh + 8));
            return perm_b32(__float_as_uint(hi), __float_as_uint(lo), kPermHiHalves);
        };
        return u32x4_t{pair(c.x, 0), pair(c.x, 16), pair(c.y, 0), pair(c.y, 16)};
    }
}

// Device-coherent stores and loads for the fused combine's partials: the
// sc1 cache bit, the one gfx950 puts on relaxed agent-scope atomic accesses
// (a store writes through the XCD's L2, a load reads past it).  With it the
// partials need no L2 write-back or invalidate around the arrival counter
// (both of which act on a whole XCD's L2), and 16-byte accesses stay whole.
constexpr int kCachePolicyCoherent = 16;  // sc1
template <typename T>
__device__ __forceinline__ void store_coherent(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent8(void* p, const f32x2_t& v) {
    store_coherent(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v));
}

// Stored partial slot -> fp32: four fp16 values scaled back by 2^e.
__device__ __forceinline__ f32x4_t unpack_partial4(u32x2_t h, int e) {
    return f32x4_t{__builtin_amdgcn_ldexpf(f16_lo_f32(h.x), e), __builtin_amdgcn_ldexpf(f16_hi_f32(h.x), e),
                   __builtin_amdgcn_ldexpf(f16_lo_f32(h.y), e), __builtin_amdgcn_ldexpf(f16_hi_f32(h.y), e)};
}

// Log-sum-exp merge of one 8-value column slot of one query row over S chunk
// partials: ml[s] = {lse_s (base 2), e_s}, o[s] = eight fp16 values of O_s
// scaled by 2^-e_s.  Chunks s >= nsplit carry weight 0 (callers fill them with
// copies of a real chunk, so the maximum is unchanged and every term stays
// finite).  With M = max_s lse_s:
//     out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M),
// summed in ascending s.  A query row with no visible position in any chunk
// (every lse = -inf) gets weight 0 everywhere and a zero row.  Both merge forms
// (the separate kernel and the fused one) call this, so they give the same bits.
template <int S>
__device__ __forceinline__ void merge_slot(const f32x2_t (&ml)[S], const u32x4_t (&o)[S], int nsplit, f32x4_t& r0,
                                           f32x4_t& r1) {
    float M = ml[0].x;
#pragma unroll
    for (int s = 1; s < S; ++s) M = fmaxf(M, ml[s].x);
    M = M == -INFINITY ? 0.f : M;
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float wgt = s < nsplit ? __builtin_amdgcn_exp2f(ml[s].x - M) : 0.f;
        const int e = (int)ml[s].y;
        acc0 += wgt * unpack_partial4(u32x2_t{o[s].x, o[s].y}, e);
        acc1 += wgt * unpack_partial4(u32x2_t{o[s].z, o[s].w}, e);
        wsum += wgt;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    r0 = acc0 * inv;
    r1 = acc1 * inv;
}

// A batch of the fused merge: this thread's items idx0, idx0 + stride, ...
// (IT of them; an item is one (query row, 8-value slot) of the unit's query
// rows g0 ..), with the S chunks' {lse, e} and 16-byte slots of every item
// loaded coherently before any is merged, so the batch costs one round trip.
// Loads of chunks past nsplit repeat the last chunk (in range; merge_slot
// gives them weight 0); items past the end load and store nothing.  ro / rm
// cover the unit's partial rows and {lse, e} pairs (split-major, GT rows per
// split).
template <int S, int IT>
__device__ __forceinline__ void fused_merge_batch(const DecodeArgs& a, __amdgpu_buffer_rsrc_t ro,
                                                  __amdgpu_buffer_rsrc_t rm, long long row, int kvh, int g0,
                                                  int items, int idx0, int stride, int nsplit) {
    const int D = a.D, slots = D / 8;
    f32x2_t ml[IT][S];
    u32x4_t o[IT][S];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = idx0 + it * stride;
        if (idx >= items) continue;
        const int g = g0 + idx / slots, slot = idx % slots;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int sc = s < nsplit ? s : nsplit - 1;
            ml[it][s] = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rm, (sc * a.GT + g) * 8, 0,
                                                                                          kCachePolicyCoherent));
            o[it][s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                        ro, ((sc * a.GT + g) * D + 8 * slot) * 2, 0, kCachePolicyCoherent));
        }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = idx0 + it * stride;
        if (idx < items) {
            const int g = g0 + idx / slots, slot = idx % slots;
            f32x4_t r0, r1;
            merge_slot<S>(ml[it], o[it], nsplit, r0, r1);
            float* dst = a.out + qrow_offset(a, row, kvh, g) + 8 * slot;
            *reinterpret_cast<f32x4_t*>(dst) = r0;
            *reinterpret_cast<f32x4_t*>(dst + 4) = r1;
        }
    }
}

template <int S, int IT>
__device__ __forceinline__ void fused_merge_all(const DecodeArgs& a, __amdgpu_buffer_rsrc_t ro,
                                                __amdgpu_buffer_rsrc_t rm, long long row, int kvh, int g0, int begin,
                                                int end, int nsplit) {
    const int stride = blockDim.x;
    for (int idx0 = begin + threadIdx.x; idx0 < end; idx0 += IT * stride)
        fused_merge_batch<S, IT>(a, ro, rm, row, kvh, g0, end, idx0, stride, nsplit);
}

// Fused log-sum-exp merge of the items begin .. end - 1 of a unit (an item is
// one (query row, 8-value slot) of the query rows g0 .. g0 + gcnt - 1): every
// thread of the workgroup takes items, a batch of them at a time (about 144
// registers of loads in flight per thread).  Every chunk's partial has been
// written with coherent stores; the planner keeps nsplit <= 8 and the unit's
// partials within a 2 GiB buffer range for this form.
__device__ __forceinline__ void fused_combine_part(const DecodeArgs& a, long long unit, long long row, int kvh,
                                                   int nsplit, int g0, int begin, int end) {
    const int D = a.D;
    const size_t first = (size_t)unit * a.max_splits * a.GT;  // (unit, split 0, query row 0)
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.part_o + first * D, a.max_splits * a.GT * D * 2);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.part_ml + first, a.max_splits * a.GT * 8);
    if (nsplit <= 2)
        fused_merge_all<2, 8>(a, ro, rm, row, kvh, g0, begin, end, nsplit);
    else if (nsplit <= 4)
        fused_merge_all<4, 6>(a, ro, rm, row, kvh, g0, begin, end, nsplit);
    else
        fused_merge_all<kFusedMaxSplits, 3>(a, ro, rm, row, kvh, g0, begin, end, nsplit);
}

// The fused combine's tail, run by every workgroup of a unit after it wrote its
// partial with the coherent stores above.  The unit's items are cut into
// nsplit equal parts, and part k is merged by the k-th workgroup to arrive:
//   - arrival: k = counter[0], incremented with wrap-around at nsplit - 1, so
//     the last arrival (k = nsplit - 1) leaves it at zero for the next call;
//   - every earlier arrival waits until counter[0] <= k, which first holds when
//     the last one has wrapped it (the chunks of a unit run side by side when
//     the grid fits the device, and finish within microseconds of each other);
//   - a wait is bounded (a.fused_wait).  One that times out records its part
//     in counter[1] and reads counter[0] again: if the last arrival has come
//     meanwhile it merges the part itself, otherwise the last arrival, which
//     takes and clears counter[1], merges it.  Either way every part is merged
//     at least once after all partials are written; a part merged twice is
//     written twice with the same bits (a bit left behind in counter[1] makes
//     the next call merge one part twice, no more).
// Each part is merged by the same code whoever takes it, so the output does
// not depend on the order of arrival.  Before arriving, each wave waits until
// its stores are complete (acknowledged at the device's coherence point), so
// once counter[0] shows every arrival each partial is readable with coherent
// loads.
__device__ __forceinline__ void fused_tail(const DecodeArgs& a, long long unit, long long row, int kvh, int nsplit,
                                           int g0, int gcnt, uint32_t* counter, int* flag_lds) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    __syncthreads();
    const uint32_t n = (uint32_t)nsplit;
    uint32_t given_up = 0;  // thread 0 of the last arrival: parts recorded in counter[1]
    if (threadIdx.x == 0) {
        const uint32_t k = atomicInc(&counter[0], n - 1);
        uint32_t mine = 1u << k;  // parts this workgroup merges
        if (k == n - 1) {
            // its value is first needed after this workgroup's own part, so
            // the exchange's round trip overlaps that part's loads
            given_up = atomicExch(&counter[1], 0u);
        } else {
            const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(&counter[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) > k) {
                if (__builtin_amdgcn_s_memrealtime() - t0 > a.fused_wait) {
                    // sequentially consistent, so the record is in place before
                    // counter[0] is read again (rare: a wait that timed out)
                    __hip_atomic_fetch_or(&counter[1], mine, __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_AGENT);
                    if (__hip_atomic_fetch_add(&counter[0], 0u, __ATOMIC_SEQ_CST, __HIP_MEMORY_SCOPE_AGENT) > k)
                        mine = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        *flag_lds = (int)mine;
    }
    __syncthreads();
    const uint32_t mine = (uint32_t)flag_lds[0];
    asm volatile("" ::: "memory");
    const int items = gcnt * (a.D / 8);
    for (int q = 0; q < nsplit; ++q)
        if ((mine >> q) & 1u)
            fused_combine_part(a, unit, row, kvh, nsplit, g0, items * q / nsplit, items * (q + 1) / nsplit);
    if (mine != 1u << (nsplit - 1)) return;  // not the last arrival (uniform across the workgroup)
    __syncthreads();  // every thread has read flag_lds[0]
    if (threadIdx.x == 0) flag_lds[0] = (int)given_up;
    __syncthreads();
    const uint32_t more = (uint32_t)flag_lds[0] & (mine - 1u);  // parts 0 .. nsplit - 2
    for (int q = 0; q < nsplit - 1; ++q)
        if ((more >> q) & 1u)
            fused_combine_part(a, unit, row, kvh, nsplit, g0, items * q / nsplit, items * (q + 1) / nsplit);
}

__device__ __forceinline__ u32x4_t load_u32x4(const uint16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}

}  // namespace mqa
