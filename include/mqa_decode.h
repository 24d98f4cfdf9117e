/*
 * mqa_decode.h -- C ABI of the MI355X (gfx950) decode-step attention library.
 *
 * The operation: one autoregressive decode step of multi-query or
 * grouped-query attention against a KV cache.  Each of B sequences brings one
 * new query token with Hq heads; groups of G = Hq / Hkv consecutive query heads
 * share one of Hkv key/value heads.  For sequence b with n = seq_lens[b] cached
 * positions and query head h (key/value head g = h / G):
 *
 *     s_j    = scale * sum_d q[b,h,d] * k_cache[b,j,g,d]        j = 0 .. n-1
 *     out[b,h,:] = sum_j softmax(s)_j * v_cache[b,j,g,:]
 *
 * Sources (restated, not quoted):
 *  - "Efficiently Scaling Transformer Inference", section 3.4, "Attention
 *    Layer Partitioning": multiquery attention shares one key/value head
 *    among all query heads; in decode the query is one token per sequence and
 *    attention Q K^T is computed locally against that sequence's cache.
 *  - "How To Scale Your Model", Part 7 "Transformer Inference": the KV cache
 *    holds each earlier token's key and value projections and a new token
 *    takes its q.k products against them (passage introducing the cache);
 *    grouped-query attention shares each key/value head among several query
 *    heads (passage on shrinking the KV cache); a ragged kernel reads only the
 *    non-padding part of the cache (passage on ragged HBM reads).
 *  - "Tensor Parallelism: Splitting Operations Across GPUs", "Splitting
 *    attention by head": every head has its own softmax and weighted sum.
 *
 * Conventions chosen where the pages are silent:
 *  - the new token's own key/value is already stored at position n-1;
 *  - n == 0 gives an all-zero output row;
 *  - seq_lens values outside [0, Lmax] are clamped to that range on the
 *    device (reading them on the host would need a synchronisation);
 *  - cache positions >= n are never read and may hold anything (NaN included).
 *
 * Memory: every pointer argument is device memory owned by the caller.  The
 * library keeps no pointer after a call returns except inside work already
 * enqueued on `stream`.  Split-K scratch (partial outputs and log-sum-exps) is
 * owned by the library, cached per (device, stream), grown on demand with
 * hipMalloc (which synchronises the device) and freed by
 * mqa_release_workspaces(); so are the fused combine's counters and the
 * persistent schedule's queue counters, zeroed once when allocated and left at
 * zero by every call (up to a merge part recorded by a wait that timed out,
 * which a later call merges again).  Warm the
 * library up with a call of the largest shape before capturing a graph.
 *
 * Errors: every argument check happens on the host before any HIP call, so
 * the checks can run on a machine with no GPU.  No call aborts or throws; a
 * failure returns a status and mqa_last_error() holds a thread-local message.
 * For tests, the environment variable MQA_FAIL_WORKSPACE_ALLOC=1 makes every
 * split-K workspace allocation fail with MQA_ERR_WORKSPACE (before any HIP
 * call).
 *
 * All calls are asynchronous with respect to the host: results are valid once
 * `stream` has been synchronised.  `stream` is a hipStream_t passed as void*
 * (NULL = the default stream).
 */
#ifndef MQA_DECODE_H
#define MQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mqa_status {
    MQA_OK = 0,
    MQA_ERR_NULL = 1,        /* a required pointer is NULL (caches only when Lmax > 0)     */
    MQA_ERR_SHAPE = 2,       /* a size is negative, Hq/Hkv/D is 0, or Hq % Hkv != 0        */
    MQA_ERR_UNSUPPORTED = 3, /* D not in {64, 128, 256}, or a size beyond the index range  */
    MQA_ERR_ALIGN = 4,       /* q / k_cache / v_cache / out not 16-byte aligned            */
    MQA_ERR_WORKSPACE = 5,   /* split-K scratch could not be allocated                    */
    MQA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed                */
    MQA_ERR_ARG = 7          /* a non-finite scale or an invalid option value             */
} mqa_status;

/* Kernel family for the q.K^T and P.V products. */
typedef enum mqa_variant {
    MQA_VARIANT_AUTO = 0, /* planner's choice (the matrix-core kernel, measured fastest)    */
    MQA_VARIANT_VALU = 1, /* vector-ALU dot products                                       */
    MQA_VARIANT_MFMA = 2  /* bf16 matrix-core tiles, 16 query heads per tile (large groups) */
} mqa_variant;

/* Element format of the key/value cache. */
typedef enum mqa_kv_format {
    MQA_KV_BF16 = 0,     /* bfloat16 values                                                */
    MQA_KV_FP8_E4M3 = 1, /* 8-bit E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa
                            bits; 0x7F and 0xFF are NaN) times one fp32 scale per cached row */
    MQA_KV_INT8 = 2      /* two's-complement int8 codes times one fp32 scale per cached row  */
} mqa_kv_format;

/* Optional knobs for mqa_decode_attention_ex; zero-initialise for defaults. */
typedef struct mqa_decode_opts {
    int variant;          /* mqa_variant                                                */
    int chunk;            /* positions per split-K chunk; 0 = planner's choice.  Must be
                             a positive multiple of 128 when set.                        */
    int combine;          /* 0 = planner's choice (the separate kernel),
                             1 = separate combine kernel,
                             2 = combine fused into the split kernel: the chunks of each
                             (sequence, kv head) merge the partials once all have
                             finished, the k-th to finish taking the k-th part of the
                             heads (a bounded wait, 20 us by default or
                             MQA_FUSED_WAIT_TICKS ticks of 10 ns, at most 10 ms; a
                             part whose wait timed out goes to the last chunk); at
                             most 8 chunks per
                             sequence, else MQA_ERR_ARG; both merges give the same bits */
    void *ev_main_begin;  /* optional hipEvent_t pair recorded by the split-K kernel's own
                             dispatch (hipExtLaunchKernelGGL) at its start and end, so  */
    void *ev_main_end;    /* their interval is that kernel's execution time alone      */
    int window;           /* 0 = attend every cached position; W > 0 = local (sliding-
                             window) attention: a sequence of length n attends positions
                             max(0, n - W) .. n-1 only, and earlier positions are never
                             read (see mqa_decode_attention_window); < 0 is MQA_ERR_ARG  */
    int kv_format;        /* mqa_kv_format of k/v (see mqa_decode_attention_quant)         */
    const float *k_scale; /* 8-bit formats: the caches' per-row scales (device memory,     */
    const float *v_scale; /* 4-byte aligned); ignored for MQA_KV_BF16                      */
    void *ev_combine_begin; /* optional hipEvent_t pair recorded by the log-sum-exp merge   */
    void *ev_combine_end;   /* kernel's own dispatch (only when a merge kernel runs)      */
    const int32_t *host_seq_lens; /* optional host copy of seq_lens (B values), read by the
                             planner only to choose the chunk size: when every length lies
                             within 128 positions of the longest (a uniform batch), a bf16
                             cache is split into about one chunk per CU, up to whole
                             sequences; otherwise, or when NULL, chunks stay short enough
                             to balance ragged lengths.  The chunks always cover Lmax (or
                             the window), so the result never depends on this hint, only
                             the speed.                                                   */
    int schedule;         /* how the split-K kernel's work items (chunk of a sequence and
                             kv head, head block) reach workgroups: 0 = planner's choice,
                             1 = one workgroup per item (grid_main x head_blocks
                             workgroups), 2 = persistent: as many workgroups as the GPU
                             holds at once take items in order from a queue counter in the
                             call's workspace (MFMA variant and separate merge only, else
                             MQA_ERR_ARG; fewer than 2^31 items, else MQA_ERR_UNSUPPORTED;
                             not with mqa_decode_attention_noalloc).  The planner picks 2
                             for grids of 2048 to 2^31 - 1 items.  Both give the same
                             bits.                                                         */
} mqa_decode_opts;

/* What the planner decided for a shape (host-only query, no HIP call). */
typedef struct mqa_plan_info {
    int variant;              /* MQA_VARIANT_VALU or MQA_VARIANT_MFMA                  */
    int chunk;                /* positions per split-K chunk                           */
    int max_splits;           /* chunks per sequence: ceil(span / chunk), at least 1, where
                                 span = Lmax, or min(Lmax, window) with a window      */
    int combine;              /* 1 = separate kernel, 2 = fused, 0 = none needed       */
    int head_blocks;          /* query-head blocks per kv head (VALU path: ceil(G/8))  */
    long long grid_main;      /* workgroups of the split-K kernel                      */
    int block_main;           /* threads per workgroup of the split-K kernel           */
    long long grid_combine;   /* workgroups of the combine kernel (0 if none)          */
    size_t workspace_bytes;   /* split-K scratch the call needs                        */
    int persistent;           /* 1 = the split-K kernel runs persistent (schedule 2):
                                 grid_main x head_blocks work items over as many
                                 workgroups as are resident at once                    */
} mqa_plan_info;

/*
 * One decode step.
 *   q         bf16 [B, Hq, D], contiguous (D innermost)
 *   k_cache   bf16 [B, Lmax, Hkv, D], contiguous: position-major per sequence
 *   v_cache   bf16 [B, Lmax, Hkv, D], contiguous
 *   seq_lens  int32 [B]: cached positions per sequence (device memory)
 *   out       fp32 [B, Hq, D], contiguous; fully overwritten
 *   scale     multiplier of q.k (typically 1/sqrt(D)); must be finite
 * B == 0 is a no-op (pointers may then be NULL).  Lmax == 0 is allowed: every
 * output row is zero and k_cache / v_cache may be NULL.
 */
mqa_status mqa_decode_attention(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *seq_lens, float *out, int B, int Hq, int Hkv,
                                int D, int Lmax, float scale, void *stream);

/* Same as mqa_decode_attention with explicit options (opts may be NULL). */
mqa_status mqa_decode_attention_ex(const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *seq_lens, float *out, int B, int Hq,
                                   int Hkv, int D, int Lmax, float scale, void *stream,
                                   const mqa_decode_opts *opts);

/*
 * mqa_decode_attention_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It never calls hipMalloc, hipFree or any allocating routine:
 * the split-K partials live in a static device array of the library,
 * MQA_NOALLOC_SCRATCH_BYTES bytes on each device it runs on, held until the
 * process ends.  Arguments, semantics and results are those of
 * mqa_decode_attention_ex (the same kernels and plan, so the same bits; a grid
 * the planner would run persistent runs one workgroup per work item here), with
 * three extra checks made on the host before any HIP call:
 *   - a call whose split workspace (mqa_plan_info.workspace_bytes) exceeds
 *     MQA_NOALLOC_SCRATCH_BYTES is MQA_ERR_WORKSPACE (choose longer chunks, or
 *     use mqa_decode_attention_ex);
 *   - opts->combine == 2 (the fused merge, whose counters would have to
 *     start at zero) is MQA_ERR_ARG; the separate merge kernel is used;
 *   - opts->schedule == 2 (the persistent schedule, whose queue counter would
 *     have to start at zero) is MQA_ERR_ARG.
 * Every call on a device shares that device's scratch and leaves its contents
 * behind (nothing in it needs clearing: each call writes every partial it
 * reads).  Calls that overlap on one device (several streams, or several host
 * threads) race on the scratch: serialise them.
 */
#define MQA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
mqa_status mqa_decode_attention_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *seq_lens, float *out, int B, int Hq,
                                        int Hkv, int D, int Lmax, float scale, void *stream,
                                        const mqa_decode_opts *opts);

/*
 * Several new tokens per sequence decoded in one call (speculative
 * verification, chunked prefill: "How To Scale Your Model", Part 7
 * "Transformer Inference", passages on prefill and on speculative sampling,
 * where several new tokens are scored against the cache at once).  The T new
 * tokens' keys and values are already in the cache at positions n-T .. n-1
 * (n = seq_lens[b]) and the tokens are causal among themselves: token i
 * (0 .. T-1) attends positions 0 .. n-T+i.  A token whose position would be
 * negative (n < T) gets an all-zero row.  The cache is read once for all T
 * tokens: the T * Hq/Hkv query rows of a key/value head share its tiles.
 *   q        bf16 [B, T, Hq, D]
 *   out      fp32 [B, T, Hq, D], fully overwritten
 *   k_cache, v_cache, seq_lens, scale as for mqa_decode_attention
 *   opts     optional (may be NULL): kernel options and an 8-bit cache format
 *            as for the other calls; a window (opts->window > 0) with T > 1 is
 *            MQA_ERR_ARG
 * T >= 1 (T == 1 is mqa_decode_attention_ex); T * Hq * D * 2 must stay below
 * 2^30 (MQA_ERR_UNSUPPORTED).  Errors and ownership as for
 * mqa_decode_attention.
 */
mqa_status mqa_decode_attention_multi(const void *q, const void *k_cache, const void *v_cache,
                                      const int32_t *seq_lens, float *out, int B, int T, int Hq, int Hkv,
                                      int D, int Lmax, float scale, void *stream,
                                      const mqa_decode_opts *opts);

/*
 * One decode step with local (sliding-window) attention ("How To Scale Your
 * Model", Part 7 "Transformer Inference", passage on mixing in local attention
 * layers: a local layer caps the context a token sees, its attention mask
 * being a diagonal strip of fixed width instead of a triangle).  Seen from the
 * newest position n-1 the strip holds the last `window` positions, so
 * sequence b attends positions max(0, n - window) .. n-1 with n = seq_lens[b]:
 *
 *     out[b,h,:] = sum_{j = max(0, n-window)}^{n-1} softmax(s)_j * v_cache[b,j,g,:]
 *
 * Positions before the window are never read and may hold anything.  The
 * work and the bytes read are those of min(n, window) positions per sequence.
 * window must be >= 1 (MQA_ERR_ARG otherwise); a window of at least Lmax is
 * the plain decode step.  Other arguments, errors and ownership as for
 * mqa_decode_attention.  The same window is available on the other decode
 * calls through mqa_decode_opts.window.
 */
mqa_status mqa_decode_attention_window(const void *q, const void *k_cache, const void *v_cache,
                                       const int32_t *seq_lens, float *out, int B, int Hq, int Hkv,
                                       int D, int Lmax, int window, float scale, void *stream);

/*
 * One decode step against a KV cache stored as 8-bit codes ("How To Scale
 * Your Model", Part 7 "Transformer Inference", passage on quantization: the
 * KV cache can be kept in int8 or fp8 to save memory bandwidth; "Machine
 * Learning Engineering and AI Systems at Scale", section "Quantization": E4M3
 * is the 8-bit inference format and the key/value cache the second thing to
 * quantize).  Each cached row (one position of one kv head) holds D codes
 * and one fp32 scale per tensor, and stands for the values code * scale:
 *   k_codes, v_codes  [B, Lmax, Hkv, D] bytes (kv_format MQA_KV_FP8_E4M3 or
 *                     MQA_KV_INT8), 16-byte aligned
 *   k_scale, v_scale  fp32 [B, Hkv, Lmax] (positions contiguous per kv head),
 *                     4-byte aligned
 *   q, seq_lens, out, scale as for mqa_decode_attention
 *   opts              optional (may be NULL); its kv_format and scale
 *                     pointers are replaced by the explicit arguments
 * The result is the decode step on the dequantized cache.  Codes and scales
 * of positions >= seq_lens[b] are never read.  The bytes read per cached row
 * are 2 * D codes plus two scales, about half of a bf16 cache's.  A
 * kv_format other than the two 8-bit ones is MQA_ERR_ARG; NULL scale
 * pointers (when B > 0 and Lmax > 0) are MQA_ERR_NULL.  A paged 8-bit cache
 * goes through mqa_decode_attention_paged with opts->kv_format and the scale
 * pointers set, the scales then laid out [num_pages, Hkv, page_size].
 */
mqa_status mqa_decode_attention_quant(const void *q, const void *k_codes, const void *v_codes,
                                      const float *k_scale, const float *v_scale,
                                      const int32_t *seq_lens, float *out, int B, int Hq, int Hkv,
                                      int D, int Lmax, int kv_format, float scale, void *stream,
                                      const mqa_decode_opts *opts);

/*
 * One decode step over a paged KV cache.  Instead of one contiguous
 * [Lmax, Hkv, D] region per sequence, the cache is a pool of fixed-size pages
 * and a per-sequence block table maps logical positions to physical pages
 * ("Machine Learning Engineering and AI Systems at Scale", section "The key
 * and value cache": blocks of a few tokens, a per-sequence block table, and
 * shared prefixes as shared blocks; "How To Scale Your Model", Part 7, the
 * passage on ragged reads and paged attention).
 *   k_pages, v_pages  bf16 [num_pages, page_size, Hkv, D], contiguous
 *   block_table       int32 [B, max_blocks]: position j of sequence b is row
 *                     j % page_size of page block_table[b][j / page_size]
 *   seq_lens          int32 [B], clamped on the device to [0, max_blocks * page_size]
 *   q, out, scale     as for mqa_decode_attention
 *   opts              optional, as for mqa_decode_attention_ex (may be NULL)
 * page_size must be a power of two >= 32 (MQA_ERR_UNSUPPORTED otherwise).
 * Only the block table entries of a sequence's first ceil(len / page_size)
 * blocks are read; several sequences may share pages.  A page index outside
 * [0, num_pages) is clamped into the pool on the device (wrong data, never an
 * out-of-range read).  Errors and ownership as for mqa_decode_attention.
 */
mqa_status mqa_decode_attention_paged(const void *q, const void *k_pages, const void *v_pages,
                                      const int32_t *block_table, const int32_t *seq_lens, float *out,
                                      int B, int Hq, int Hkv, int D, int num_pages, int page_size,
                                      int max_blocks, float scale, void *stream,
                                      const mqa_decode_opts *opts);

/*
 * Causal attention over whole sequences with no cache, the computation a KV
 * cache replaces ("How To Scale Your Model", Part 7, passage introducing the
 * KV cache: a token attends only to itself and earlier tokens; prefill is the
 * compute-bound pass over a whole prompt, passage on prefill versus
 * generation; "Efficiently Scaling Transformer Inference", section 3.4,
 * "Attention Layer Partitioning": in prefill the K/V read is amortised over
 * the query tokens).  Row t of sequence b (t < seq_lens[b]) attends positions
 * 0..t; its result equals a decode step at length t+1 with query q_seq[b,t].
 * Rows t >= seq_lens[b] are written as zeros.
 * It runs on the matrix cores: the query rows of a sequence and kv head are
 * its (position, head of the group) pairs in position order, and each
 * workgroup serves 128 consecutive rows, which share one read of their
 * causal prefix, streamed through LDS in 64-position tiles
 * (mqa_prefill_plan reports the rows per workgroup and the grid).  No
 * scratch memory.
 *   q_seq    bf16 [B, Lmax, Hq, D]
 *   k_cache  bf16 [B, Lmax, Hkv, D];  v_cache likewise
 *   seq_lens int32 [B] (device)
 *   out_seq  fp32 [B, Lmax, Hq, D], fully overwritten
 * Errors and ownership as for mqa_decode_attention.
 */
mqa_status mqa_prefill_attention(const void *q_seq, const void *k_cache, const void *v_cache,
                                 const int32_t *seq_lens, float *out_seq, int B, int Hq,
                                 int Hkv, int D, int Lmax, float scale, void *stream);

/*
 * Host-only validation and planning for a decode call with these sizes and
 * options: runs every argument check mqa_decode_attention runs (pointers are
 * not inspected) and, on success, fills *info when info is non-NULL.
 * Makes no HIP call.
 */
mqa_status mqa_decode_plan(int B, int Hq, int Hkv, int D, int Lmax, float scale,
                           const mqa_decode_opts *opts, mqa_plan_info *info);

/* The plan of a mqa_prefill_attention call (host only, no HIP call): fills
 * *info when non-NULL and the query rows one workgroup serves when
 * rows_per_block is non-NULL. */
mqa_status mqa_prefill_plan(int B, int Hq, int Hkv, int D, int Lmax, float scale, mqa_plan_info *info,
                            int *rows_per_block);

/* mqa_decode_plan for a mqa_decode_attention_multi call with T tokens per
 * sequence (host only, no HIP call). */
mqa_status mqa_decode_plan_multi(int B, int T, int Hq, int Hkv, int D, int Lmax, float scale,
                                 const mqa_decode_opts *opts, mqa_plan_info *info);

/* Static description of a status code (never NULL). */
const char *mqa_status_string(mqa_status status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char *mqa_last_error(void);

/* Frees every cached split-K workspace.  Must not race with calls in flight:
 * synchronise the streams that used the library first. */
void mqa_release_workspaces(void);

/*
 * Calibration: the read rate of a pure streaming read on this device, the
 * ceiling the decode kernels are read against (decode attention is bound by
 * streaming the cache from HBM: "How To Scale Your Model", Part 7 "Transformer
 * Inference", the passage on the arithmetic intensity of attention).
 * `workgroups` workgroups of 256 threads each read one contiguous slice of
 * ceil(bytes / workgroups) bytes (rounded up to 16) of `buf` with 16-byte
 * non-temporal loads (the cache policy of the K/V tiles) and write one
 * word to sink[w]; no other memory is written.
 *   buf        device memory, 16-byte aligned; bytes a multiple of 16
 *   sink       uint32 [number of slices] (at most `workgroups`), device memory
 *   ev_begin, ev_end  optional hipEvent_t pair recorded by the kernel's own
 *              dispatch, so their interval is its execution time alone
 * bytes == 0 is a no-op.  NULL pointers are MQA_ERR_NULL, misalignment
 * MQA_ERR_ALIGN, workgroups outside [1, 2^24] MQA_ERR_ARG, a slice above
 * 1 GiB MQA_ERR_UNSUPPORTED, all checked before any HIP call.
 */
mqa_status mqa_stream_read_probe(const void *buf, size_t bytes, int workgroups, uint32_t *sink, void *stream,
                                 void *ev_begin, void *ev_end);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int mqa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MQA_DECODE_H */
