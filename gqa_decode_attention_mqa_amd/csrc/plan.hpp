// Host-side argument checks and launch planning for the decode library.
// This translation unit makes no HIP call, so every check can run on a
// machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/mqa_decode.h"

namespace mqa {

// Number of compute units the planner sizes grids for (MI355X: 256 CUs in
// 8 XCDs of 32).
constexpr int kComputeUnits = 256;
// Every chunk is a multiple of this many positions, the largest tile any
// kernel steps through.
constexpr int kChunkQuantum = 128;
// Query heads per MFMA tile along the N dimension.
constexpr int kMfmaHeadsPerTile = 16;
// Smallest number of query rows per kv head (G times the query tokens) sent
// to the matrix-core kernel by default: every group.  Measured on MI355X on
// the ragged batch (B=256, Hkv=8, D=128, lengths U[1, 8192]) with 512-position
// chunks against the vector kernel: G = 4: 753 vs 776 us (bf16), 456 vs 676 us
// (fp8); G = 2: 723 vs 736 us, 429 vs 452 us; G = 1: 706 vs 730 us, 416 vs
// 447 us.  The vector kernel stays available as an explicit variant.
constexpr int kMfmaMinGroup = 1;
// With at least this many (row, kv head) units the matrix-core chunks are
// capped at kMaxChunkMfmaMany positions: there are workgroups enough without
// long chunks, and short ones balance ragged lengths (ragged batch above:
// 753 us at 512 or 1024 positions against 826 us at 2048; 1024 keeps a
// sequence within the few-chunk combine, 5 us against 17 us for 16 chunks).
constexpr long long kManyUnits = 4 * kComputeUnits;
constexpr long long kMaxChunkMfmaMany = 1024;
// Most query rows one MFMA workgroup serves (six 16-row tiles, one compute
// wave each): 2 tokens of a 48-head group still read the cache once.
constexpr int kMfmaMaxHeads = 96;
// Most query heads one VALU workgroup serves (bf16 cache; 8-bit caches).
constexpr int kValuMaxHeads = 8;
constexpr int kValuMaxHeads8 = 4;
// Up to this many chunks per sequence the combine kernel keeps every chunk of
// a column slot in registers (one thread per (query head, 16-byte slot));
// beyond it, threads of a workgroup split the chunks of one head.
constexpr int kCombineFewMaxSplits = 8;
// Most chunks per unit the fused combine handles: the same register-resident
// merge of every chunk's slot as the few-chunk kernel.
constexpr int kFusedMaxSplits = kCombineFewMaxSplits;
// uint32 counters per unit of the fused combine (arrivals and the merge parts
// given up by timed-out waits; padded to 16 bytes).
constexpr int kFusedCountersPerUnit = 4;
// The split kernel's persistent form: its item counter and a count of the
// workgroups that have left.  The planner chooses it for grids of at least
// kPersistMinItems work items (MI355X, persistent against one workgroup per
// item: the ragged GQA batch, 16384 items, 694 against 761 us, on fp8 394
// against 465; the PaLM-shaped MQA step, 256 items, 28.4 against 25.5).
constexpr int kPersistCounters = 2;
constexpr long long kPersistMinItems = 2048;
constexpr long long kPersistMaxItems = 1LL << 31;  // the queue counter is 32 bits wide
// How long a workgroup of the fused combine waits for the other chunks of its
// unit before leaving its part of the merge to the last one: 20 us of the
// 100 MHz real-time counter.  MQA_FUSED_WAIT_TICKS overrides it (tests force
// the timed-out path with 0).
constexpr unsigned kFusedWaitTicks = 2000;
constexpr unsigned kFusedMaxWaitTicks = 1000000;  // the most MQA_FUSED_WAIT_TICKS may ask: 10 ms
// make_plan's `causal` argument for the causal prefill kernel.
constexpr int kCausalPrefill = 3;
// Causal prefill kernel, per head size D: query rows per workgroup, 16-row
// tiles of them per compute wave (the workgroup has rows / (16 * tiles)
// compute waves), positions per K/V tile and stages of the LDS ring.
// Measured on MI355X, PaLM-shaped (D = 256) and gqa70b-shaped (D = 128)
// prefills:
//   - D = 256: one tile per wave, eight waves; two tiles per wave need more
//     registers than two waves per SIMD leave (8.6 ms against 10.2 ms at one
//     wave per SIMD);
//   - D <= 128: two tiles per wave (each K and V^T read feeds two products),
//     against one: 10.1 ms against 11.1 ms;
//   - two stages of 64-position tiles: 256 rows per workgroup, 32-position
//     tiles or deeper rings were slower or within 2 % (LDS budget: 2 * stages
//     * step * D * 2 bytes per workgroup, two workgroups per CU at D <= 128).
constexpr int prefill_rows(int D) { return D > 0 ? 128 : 0; }
constexpr int prefill_row_tiles(int D) { return D == 256 ? 1 : 2; }
constexpr int prefill_step(int D) { return D > 0 ? 64 : 0; }
constexpr int prefill_stages(int D) { return D > 0 ? 2 : 0; }
constexpr int kPrefillMaxRows = 256;  // the most rows any head size's workgroup takes
// Query heads per workgroup of the few-chunk combine (256 threads, D/8 each).
constexpr int combine_heads_per_block(int D) { return 2048 / D; }

struct Plan {
    int variant = MQA_VARIANT_VALU;  // resolved, never AUTO
    int G = 0;                       // query heads per kv head
    int T = 1;                       // query tokens per row
    int GT = 0;                      // query rows per (row, kv head): T * G
    int heads_per_block = 0;         // padded heads a workgroup serves
    int head_blocks = 1;             // workgroups per (row, kv head, chunk) along heads
    int chunk = 0;                   // positions per split
    int max_splits = 1;              // ceil(span / chunk), >= 1 (span: Lmax, or
                                     // min(Lmax, window) with a sliding window)
    int window = 0;                  // sliding window (0 = none)
    int kv_format = 0;               // mqa_kv_format of the cache
    int combine = 0;                 // 0 none, 1 separate kernel, 2 fused
    long long rows = 0;              // rows (sequences) of the call: B
    int row_blocks = 0;              // causal prefill: workgroups of prefill_rows(D) query rows per
                                     // (sequence, kv head)
    long long grid_main = 0;         // workgroups along x of the split kernel
    int block_main = 256;
    long long grid_combine = 0;
    int combine_dsplit = 1;          // many-chunk merge: workgroups per query row (slices of d)
    size_t workspace_bytes = 0;      // partial outputs + partial LSEs
    size_t part_o_offset = 0;        // byte offsets inside the workspace
    size_t part_ml_offset = 0;
    size_t counters = 0;             // fused-combine counters (uint32, kFusedCountersPerUnit per
                                     // (row, kv head, head block)), kept in a buffer of their own
                                     // that is zero between calls; then the persistent form's queue
    int persist = 0;                 // 1: the split kernel's persistent form (as many workgroups as are
                                     // resident at once take the grid_main * head_blocks items)
};

// Thread-local last-error text.
void set_error(const std::string& msg);
const char* last_error();

// Checks sizes, scale and options; on success fills `plan`.  causal = 0 plans
// a decode call (B rows of T query tokens, T = 1 for a decode step); causal =
// kCausalPrefill plans the causal prefill kernel (B * Hkv * row_blocks
// workgroups of prefill_rows(D) query rows, no split, no merge).
mqa_status make_plan(int B, int Hq, int Hkv, int D, int Lmax, float scale,
                     const mqa_decode_opts* opts, int causal, Plan* plan, int T = 1);

// A paged cache as the kernels see it (see check_paged).
struct PagedCache {
    const int32_t* block_table;
    int num_pages, page_size, max_blocks, page_shift;
};

// Paged-cache checks: page_size a power of two >= 32, counts >= 0, the
// logical length max_blocks * page_size within int, a non-NULL 4-byte aligned
// block table and a non-empty pool when any position can be attended.  On
// success fills `pc` and the logical maximum length `Lmax`.
mqa_status check_paged(int B, const int32_t* block_table, int num_pages, int page_size, int max_blocks,
                       PagedCache* pc, int* Lmax);

// Pointer checks: non-NULL when B > 0 (the caches only when Lmax > 0), 16-byte
// alignment of the bf16/fp32 arrays.
mqa_status check_pointers(int B, int Lmax, const void* q, const void* k, const void* v,
                          const int32_t* seq_lens, const float* out);

}  // namespace mqa
