// Host-side argument checks and launch planning (no HIP calls).
#include "plan.hpp"

#include <cmath>
#include <cstdlib>
#include <string>

namespace mqa {

namespace {
thread_local std::string g_last_error;

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }
long long round_up(long long a, long long b) { return ceil_div(a, b) * b; }

mqa_status fail(mqa_status s, const std::string& msg) {
    set_error(msg);
    return s;
}

// Workgroups the planner aims for when it picks the chunk size: one per CU.
// Measured on MI355X (split kernel), more, shorter chunks lose to their extra
// fixed costs and partial traffic, fewer leave CUs idle (PaLM-shaped MQA:
// chunk 512 -> 28.5 us, 256 -> 34.8 us, 1024 -> 33.6 us; long-context MQA:
// 2048 -> 84.2 us, 1024 -> 92.9 us, 4096 -> 111.3 us).
constexpr long long kTargetWorkgroups = kComputeUnits;
// Chunk bounds: below 256 positions the partial outputs cost more traffic than
// the split saves; longer chunks balance a ragged batch poorly (the vector
// kernel, an explicit variant, gets the tighter bound).  Measured on MI355X:
//   - ragged lengths U[1, 8192], B=32..96, Hkv=8, D=128: whole sequences
//     lose (B=32: 132.1 us against 116.1 at 2048 and 102.0 at 1024);
//   - a uniform batch on a bf16 cache wants about one chunk per CU, up to
//     whole sequences, which also saves the merge and the partials (B=32,
//     Hkv=8, D=128, len 4096: 78.2 us with whole sequences against 90.7 at
//     2048; the same with 4 query tokens 81.6 against 92.7; PaLM-shaped MQA
//     at B=256: 84.6 against 93.6 at 1024; B=16 at len 131072: 320.9 at 8192
//     against 389.3 at 2048);
//   - an 8-bit cache stays at 2048 even then: its loop is bound by the
//     compute waves, so two workgroups per CU win (the uniform GQA batch:
//     fp8 50.5 us at 2048 against 81.3 at 4096, int8 56.9 against 95.2).
// Whether a batch is uniform is known only from the host copy of the lengths
// the caller may pass (mqa_decode_opts.host_seq_lens).  Without it, 2048 is
// kept (1024 from kManyUnits units on): few-unit uniform batches need the
// longer chunks (B=4 at len 131072: 84.2 us at 2048 against 92.9 at 1024).
// With it, a ragged batch of at least one unit per CU gets 1024 (ragged
// B=32..96 above: 102.0 / 191.1 / 287.0 us at 1024 against 116.1 / 215.2 /
// 318.6 at 2048).
constexpr long long kMinChunk = 256;
constexpr long long kMaxChunkMfma = 2048;
constexpr long long kMaxChunkValu = 1024;
// Largest grid the launcher accepts (work-items must stay below 2^32).
constexpr long long kMaxGrid = (1LL << 24) - 1;
}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }
const char* last_error() { return g_last_error.c_str(); }

mqa_status check_pointers(int B, int Lmax, const void* q, const void* k, const void* v,
                          const int32_t* seq_lens, const float* out) {
    if (B == 0) return MQA_OK;
    if (!q || !seq_lens || !out)
        return fail(MQA_ERR_NULL, "q, seq_lens and out must be non-NULL");
    if (Lmax > 0 && (!k || !v))
        return fail(MQA_ERR_NULL, "k_cache and v_cache must be non-NULL when Lmax > 0");
    auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out))
        return fail(MQA_ERR_ALIGN, "q, k_cache, v_cache and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0)
        return fail(MQA_ERR_ALIGN, "seq_lens must be 4-byte aligned");
    return MQA_OK;
}

mqa_status check_paged(int B, const int32_t* block_table, int num_pages, int page_size, int max_blocks,
                       PagedCache* pc, int* Lmax) {
    if (num_pages < 0 || max_blocks < 0 || page_size <= 0)
        return fail(MQA_ERR_SHAPE, "num_pages and max_blocks must be >= 0 and page_size > 0");
    if (page_size < 32 || (page_size & (page_size - 1)) != 0)
        return fail(MQA_ERR_UNSUPPORTED, "page_size must be a power of two >= 32");
    const long long L = (long long)max_blocks * page_size;
    if (L > 0x7FFFFFFFLL)
        return fail(MQA_ERR_UNSUPPORTED, "max_blocks * page_size exceeds the int range");
    if (B > 0 && L > 0) {
        if (!block_table) return fail(MQA_ERR_NULL, "block_table must be non-NULL");
        if ((reinterpret_cast<uintptr_t>(block_table) & 3u) != 0)
            return fail(MQA_ERR_ALIGN, "block_table must be 4-byte aligned");
        if (num_pages == 0) return fail(MQA_ERR_SHAPE, "the page pool is empty");
    }
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    *pc = PagedCache{block_table, num_pages, page_size, max_blocks, shift};
    *Lmax = (int)L;
    return MQA_OK;
}

mqa_status make_plan(int B, int Hq, int Hkv, int D, int Lmax, float scale,
                     const mqa_decode_opts* opts, int causal, Plan* plan, int T) {
    if (B < 0 || Lmax < 0)
        return fail(MQA_ERR_SHAPE, "B and Lmax must be >= 0");
    if (Hq <= 0 || Hkv <= 0 || D <= 0)
        return fail(MQA_ERR_SHAPE, "Hq, Hkv and D must be > 0");
    if (Hq % Hkv != 0)
        return fail(MQA_ERR_SHAPE, "Hq must be a multiple of Hkv");
    if (D != 64 && D != 128 && D != 256)
        return fail(MQA_ERR_UNSUPPORTED, "head size D must be 64, 128 or 256");
    if (!std::isfinite(scale))
        return fail(MQA_ERR_ARG, "scale must be finite");
    // Kernels address a tile of up to 128 positions through 32-bit buffer offsets.
    if ((long long)Hkv * D * 2 * kChunkQuantum > 0x7FFFFFFFLL)
        return fail(MQA_ERR_UNSUPPORTED, "Hkv * D too large for 32-bit tile offsets");

    mqa_decode_opts o{};
    if (opts) o = *opts;
    if (o.variant < MQA_VARIANT_AUTO || o.variant > MQA_VARIANT_MFMA)
        return fail(MQA_ERR_ARG, "unknown variant");
    if (o.chunk < 0 || (o.chunk > 0 && o.chunk % kChunkQuantum != 0))
        return fail(MQA_ERR_ARG, "chunk must be 0 or a positive multiple of 128");
    if (o.combine < 0 || o.combine > 2)
        return fail(MQA_ERR_ARG, "combine must be 0, 1 or 2");
    if (o.schedule < 0 || o.schedule > 2)
        return fail(MQA_ERR_ARG, "schedule must be 0, 1 or 2");
    if (o.window < 0)
        return fail(MQA_ERR_ARG, "window must be >= 0 (0 = no window)");
    if (o.kv_format < MQA_KV_BF16 || o.kv_format > MQA_KV_INT8)
        return fail(MQA_ERR_ARG, "unknown kv_format");
    if (T < 1)
        return fail(MQA_ERR_SHAPE, "the number of query tokens must be >= 1");
    if (T > 1 && o.window > 0)
        return fail(MQA_ERR_ARG, "a sliding window is not supported with several query tokens");
    // a unit's query rows are addressed through one 32-bit buffer range
    if ((long long)T * Hq * D * 2 >= (1LL << 30))
        return fail(MQA_ERR_UNSUPPORTED, "T * Hq * D too large");
    // Chunk starts sit up to 31 positions before a window's first position.
    if (o.window > 0 && Lmax > 0x7FFFFFFF - 64)
        return fail(MQA_ERR_UNSUPPORTED, "Lmax too large for a sliding window");

    Plan p;
    p.G = Hq / Hkv;
    if (causal) {
        // causal prefill: the Lmax * G query rows of each (sequence, kv head)
        // in workgroups of prefill_rows(D) rows, each streaming its causal prefix
        if (o.variant == MQA_VARIANT_VALU || o.window > 0 || o.kv_format != MQA_KV_BF16 || o.chunk || o.combine ||
            o.schedule)
            return fail(MQA_ERR_ARG,
                        "the prefill form takes no variant, window, cache format, chunk, combine or schedule option");
        if ((long long)Lmax * p.G > 0x7FFFFFFFLL - kPrefillMaxRows)
            return fail(MQA_ERR_UNSUPPORTED, "Lmax * Hq / Hkv too large for the prefill kernel");
        p.variant = MQA_VARIANT_MFMA;
        p.T = 1;
        p.GT = p.G;
        p.heads_per_block = prefill_rows(D);  // query rows per workgroup
        p.head_blocks = 1;
        p.rows = B;
        p.row_blocks = (int)ceil_div((long long)Lmax * p.G, prefill_rows(D));
        p.chunk = (int)round_up(Lmax > 0 ? Lmax : 1, kChunkQuantum);
        p.max_splits = 1;
        p.grid_main = (long long)B * Hkv * p.row_blocks;
        p.block_main = 64 * (prefill_rows(D) / (16 * prefill_row_tiles(D)));
        if (p.grid_main > kMaxGrid)
            return fail(MQA_ERR_UNSUPPORTED, "problem too large for one launch (grid limit)");
        *plan = p;
        return MQA_OK;
    }
    p.T = T;
    p.GT = T * p.G;  // query rows sharing one kv head: what the head tiles hold
    p.variant = o.variant;
    if (p.variant == MQA_VARIANT_AUTO)
        p.variant = (p.GT >= kMfmaMinGroup) ? MQA_VARIANT_MFMA : MQA_VARIANT_VALU;

    if (p.variant == MQA_VARIANT_MFMA) {
        const int heads = p.GT < kMfmaMaxHeads ? p.GT : kMfmaMaxHeads;
        p.heads_per_block = (int)round_up(heads, kMfmaHeadsPerTile);
    } else {
        // 8-bit caches: each lane holds twice the columns, so fewer heads per block
        const int cap = o.kv_format == MQA_KV_BF16 ? kValuMaxHeads : kValuMaxHeads8;
        int gb = 1;
        while (gb < p.GT && gb < cap) gb *= 2;
        p.heads_per_block = gb;
    }
    p.head_blocks = (int)ceil_div(p.GT, p.heads_per_block);

    p.rows = B;
    const long long units = p.rows * Hkv * p.head_blocks;

    // Positions one row attends: Lmax, or W with a sliding window of W
    // positions.  Windowed chunks start at the window's first position rounded
    // down to a multiple of 32; the last chunk of a row absorbs those up to 31
    // extra positions, so `span` chunks still cover every row.
    long long span = Lmax;
    if (o.window > 0 && o.window < span) span = o.window;
    p.window = o.window;
    p.kv_format = o.kv_format;

    if (o.chunk > 0) {
        p.chunk = o.chunk;
    } else if (units == 0 || span == 0) {
        p.chunk = kChunkQuantum;
    } else {
        // A windowed step is small, so its chunks may go down to 128
        // positions (measured on MI355X, B=4, Hq=48, D=256, W=8192: 14.6 us at
        // 128 against 16.0 us at 256).
        const bool windowed = o.window > 0 && o.window < Lmax;
        // The host copy of the lengths, when the caller passes one, tells a
        // uniform batch (every length within one quantum of the longest) from
        // a ragged one; see the chunk bounds above.
        long long work = span;  // positions per row the chunks are sized for
        bool uniform = false, ragged = false;
        if (o.host_seq_lens && B > 0 && p.variant == MQA_VARIANT_MFMA) {
            long long lo = span, hi = 0;
            for (int b = 0; b < B; ++b) {
                long long n = o.host_seq_lens[b];
                n = n < 0 ? 0 : (n > Lmax ? Lmax : n);
                if (o.window > 0 && n > o.window) n = o.window;
                lo = n < lo ? n : lo;
                hi = n > hi ? n : hi;
            }
            uniform = hi > 0 && hi - lo < kChunkQuantum;
            ragged = !uniform && hi > 0;
            if (uniform) work = hi;
        }
        const bool coarse = uniform && o.kv_format == MQA_KV_BF16;
        long long c = round_up(ceil_div(work * units, kTargetWorkgroups), kChunkQuantum);
        long long cmax;
        if (p.variant != MQA_VARIANT_MFMA)
            cmax = kMaxChunkValu;
        else if (coarse)
            cmax = round_up(work, kChunkQuantum);  // up to whole sequences
        else if (units >= kManyUnits || (ragged && units >= kComputeUnits))
            cmax = kMaxChunkMfmaMany;
        else
            cmax = kMaxChunkMfma;
        const long long cmin = windowed ? kChunkQuantum : kMinChunk;
        if (c < cmin) c = cmin;
        if (c > cmax) c = cmax;
        const long long whole = round_up(span, kChunkQuantum);
        if (c > whole) c = whole;
        p.chunk = (int)c;
    }
    p.max_splits = span > 0 ? (int)ceil_div(span, p.chunk) : 1;
    if (p.max_splits < 1) p.max_splits = 1;

    p.grid_main = p.rows * Hkv * p.max_splits;
    // matrix cores: one compute wave per 16 heads (two on 8-bit caches at
    // D = 256 with up to 48 heads per block) plus two load-only waves
    if (p.variant == MQA_VARIANT_MFMA) {
        const int tiles = p.heads_per_block / kMfmaHeadsPerTile;
        const int per_tile = (o.kv_format != MQA_KV_BF16 && D >= 256 && tiles <= 3) ? 2 : 1;
        p.block_main = 64 * (tiles * per_tile + 2);
    } else {
        p.block_main = 256;
    }
    if (p.grid_main > kMaxGrid || p.head_blocks > 65535)
        return fail(MQA_ERR_UNSUPPORTED, "problem too large for one launch (grid limit)");

    if (p.max_splits > 1 && p.rows > 0) {
        // the fused merge addresses a unit's partials through one 32-bit buffer range
        const bool fusable = p.max_splits <= kFusedMaxSplits &&
                             (long long)p.max_splits * p.GT * D * 2 <= 0x7FFFFFFFLL;
        if (o.combine == 2 && !fusable)
            return fail(MQA_ERR_ARG, "the fused combine handles at most 8 chunks per sequence "
                                     "(and max_splits * T * G * D * 2 < 2^31)");
        // Default: the separate combine kernel.  In the fused form the chunks
        // of each unit merge the partials at the tail of the split kernel; on
        // MI355X it was no faster (PaLM-shaped MQA: 29.84 us per step by wall
        // clock for both forms), and its waits assume the grid fits the device.
        p.combine = (o.combine == 0) ? 1 : o.combine;
        if (p.combine != 1)
            p.grid_combine = 0;
        else if (p.max_splits <= kCombineFewMaxSplits)  // whole head blocks of each unit
            p.grid_combine = p.rows * Hkv * ceil_div(p.GT, combine_heads_per_block(D));
        else {
            // one workgroup per query row, or up to D/64 of them per row, each
            // merging a slice of d, until the grid covers the CUs: the merge
            // of a row's many chunks is bound by the latency of its loads
            // (MI355X, one sequence of 131072 positions, 48 heads, D = 256,
            // 256 chunks: 5.2 us with 4 slices against 10.3 us with one; 8
            // slices, or slicing on to twice the CUs, 6.3 us: the per-slot
            // sums of more threads then take longer to add)
            const long long rows_q = p.rows * T * Hq;
            int ds = 1;
            while (rows_q * ds < kComputeUnits && ds < D / 64) ds *= 2;
            p.combine_dsplit = ds;
            p.grid_combine = rows_q * ds;
        }
        if (p.grid_combine > kMaxGrid)
            return fail(MQA_ERR_UNSUPPORTED, "problem too large for one launch (combine grid limit)");
        const size_t parts = (size_t)p.rows * Hkv * p.max_splits * p.GT;
        p.part_o_offset = 0;  // fp16 partial rows, then {lse, e} pairs
        p.part_ml_offset = round_up((long long)(parts * D * sizeof(uint16_t)), 256);
        p.workspace_bytes = p.part_ml_offset + round_up((long long)(parts * 2 * sizeof(float)), 256);
        p.counters = (p.combine == 2) ? (size_t)p.rows * Hkv * p.head_blocks * kFusedCountersPerUnit : 0;
    }
    // Persistent schedule: grids of many work items, whose workgroups would
    // otherwise wait on the hardware's in-order dispatch behind longer ones.
    const long long items = p.grid_main * p.head_blocks;
    if (o.schedule == 2 && (p.variant != MQA_VARIANT_MFMA || p.combine == 2))
        return fail(MQA_ERR_ARG, "the persistent schedule needs the MFMA variant and the separate merge");
    // its 32-bit queue counter must not wrap before every workgroup has seen the end
    if (o.schedule == 2 && items >= kPersistMaxItems)
        return fail(MQA_ERR_UNSUPPORTED, "too many work items for the persistent schedule");
    if (items > 0 && (o.schedule == 2 || (o.schedule == 0 && p.variant == MQA_VARIANT_MFMA && p.combine != 2 &&
                                          items >= kPersistMinItems && items < kPersistMaxItems))) {
        p.persist = 1;
        p.counters += kPersistCounters;  // the queue after the fused counters (none then)
    }
    *plan = p;
    return MQA_OK;
}

}  // namespace mqa
