// LDS tiles of cached rows as the matrix-core kernels read them (gfx950):
// the bank-conflict-avoiding layout of a tile, gfx950's transposing LDS reads
// that give the V^T operand of P.V, and small compile-time helpers.
#pragma once

#include "kernel_common.hpp"

namespace mqa {

// LDS bank model: an LDS access is served 256 bytes (all 64
// banks of 4 bytes) at a time, i.e. 16 lanes of a 16-byte read or 32 lanes
// of an 8-byte read per pass; rows of a tile that are a multiple of 256 bytes
// apart hit the same banks.
//
// LDS layout of a bf16 tile: row t (D bf16) is D/8 chunks of 16 bytes, and
// chunk c of row t sits in slot c ^ swz_key<D>(t).  For D >= 128 (every row
// starts on bank 0) the key takes sixteen values over any sixteen consecutive
// rows (the q.K reads of a pass: sixteen rows, one chunk column) and eight
// values differing above bit 0 over rows 8i .. 8i+7 (the transposing V reads
// of a pass: eight rows, two adjacent chunks each).  For D = 64 (two rows per
// 256 bytes) the same holds among the rows of one parity.
template <int D>
__device__ __forceinline__ int swz_key(int t) {
    if constexpr (D >= 128)
        return ((t & 7) << 1) | ((t >> 3) & 1);
    else
        return (((t >> 1) & 3) << 1) | ((t >> 3) & 1);
}
// The key is below 2 * kSwzRegs, so chunk 2m + x of row t sits in slot
// (2 (m mod NR) + x) ^ key, plus 2 NR (m div NR), with NR = kSwzRegs: at byte
// 32 ((m mod NR) ^ (key >> 1)) + 16 (x ^ (key & 1)) + 32 NR (m div NR) of
// the row.  The address for m is therefore the one for m = 0 XOR 32 (m mod
// NR), plus a constant; rows, tiles and ring slots all start on multiples of
// 32 NR bytes (the LDS block itself at address 0), so the XOR never reaches
// above the row.
template <int D>
constexpr int kSwzRegs = D >= 128 ? 8 : 4;

// LDS byte offset of chunk c of row t inside a bf16 tile.
template <int D>
__device__ __forceinline__ int swz(int t, int c) {
    return (t * (D / 8) + (c ^ swz_key<D>(t))) * 16;
}

// 8-bit tiles: row t (D codes) is D/16 chunks of 16 bytes, chunk c in slot
// c ^ swz8_key<D>(t).  With R = 256/D rows per 256 bytes of banks, the key is
// one-to-one over the rows of one bank offset among any 16 consecutive rows
// (the q.K reads of a 16-lane group) and among rows 4i .. 4i+3 and
// 16 + 4i .. 16 + 4i + 3 (the transposing V reads of a 16-lane group).  A key
// also separating two such groups (for 32-lane passes) measured slower on
// MI355X (int8 PaLM MQA 35.0 against 32.5 us, B=4 len 131072 116 against
// 105 us), so the 16-lane form is kept for 8-bit tiles.
template <int D>
__device__ __forceinline__ int swz8_key(int t) {
    constexpr int R = 256 / D;
    return ((t / R) + (t >> 4) * (4 / R)) & (D / 16 - 1);
}

template <int FMT, int D>
__device__ __forceinline__ int tile_key(int t) {
    if constexpr (FMT == kKvBf16)
        return swz_key<D>(t);
    else
        return swz8_key<D>(t);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS byte address of a pointer into this kernel's dynamic LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// gfx950 transposing LDS read of 16-bit elements (ds_read_b64_tr_b16) at
// LDS byte address addr + OFF.  In each group of 16 lanes, lane i receives
// element (i mod 4) of the 8-byte rows addressed by lanes 4j + i/4 of its
// group, j = 0..3 (checked on MI355X).
//
// Issued through inline asm: the compiler builtin makes the compiler wait for
// every buffer-to-LDS load in flight before each such read, which would
// drain the ring.  The compiler does not know this asm reads LDS, so the
// caller must wait for it (s_waitcnt lgkmcnt) and tie the results to that
// wait before using them; any LDS wait the compiler emits for its own reads
// stays correct, since unknown later LDS reads only make it wait longer.
template <int OFF>
__device__ __forceinline__ u32x2_t ds_read_tr16_b64_asm(uint32_t addr) {
    u32x2_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// The same for 8-bit elements (ds_read_b64_tr_b8): in each group of 16
// lanes, lane i receives as element k (k = 0..7) byte (i mod 8) of the 8-byte
// row addressed by lane 2k + i/8 of its group (checked on MI355X).
__device__ __forceinline__ u32x2_t ds_read_tr8_b64_asm(uint32_t addr) {
    u32x2_t r;
    asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Issue the V^T operand reads of 16-row tiles m = M0 .. M0+MH-1 of d of one
// tile: the transposing reads at rows `lo` and `hi` (the lane's two groups of
// four positions).  alo / ahi are the LDS addresses for m = 0; tile m reads
// at that address XOR 32 (m mod NR), plus 32 NR (m div NR) (see kSwzRegs).
// The results are valid only after wait_vt_tile.
template <int M0, int MH, int NR>
__device__ __forceinline__ void issue_vt_tile(uint32_t alo, uint32_t ahi, u32x2_t (&lo)[MH], u32x2_t (&hi)[MH]) {
    static_for<0, MH>([&](auto jc) {
        constexpr int j = decltype(jc)::value, m = M0 + j;
        constexpr int off = 32 * NR * (m / NR);
        lo[j] = ds_read_tr16_b64_asm<off>(alo ^ (32 * (m % NR)));
        hi[j] = ds_read_tr16_b64_asm<off>(ahi ^ (32 * (m % NR)));
    });
}
// Wait until every LDS read of this wave has landed and tie the V^T operands
// to that wait, so no use of them can be scheduled before it.
template <int MT>
__device__ __forceinline__ void wait_vt_tile(u32x2_t (&lo)[MT], u32x2_t (&hi)[MT]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(lo[m]), "+v"(hi[m]));
}

template <int MT>
__device__ __forceinline__ void wait_v8_tile(u32x2_t (&v)[MT]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(v[m]));
}

}  // namespace mqa
