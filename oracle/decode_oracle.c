/*
 * Plain CPU fp64 oracle for one decode step of multi-query / grouped-query
 * attention against a KV cache, plus the textbook causal attention that the
 * cache replaces.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library.  It is deliberately slow and literal: every loop follows
 * the definition, with no blocking, fusion or reordering.
 *
 * What it computes (sources, restated):
 *  - "How To Scale Your Model", Part 7 "Transformer Inference" (passage that
 *    introduces the KV cache): each token's key and value projections are
 *    written once into a cache; a later token forms its dot products q_i.k_j
 *    against the cached keys, and a token attends only to earlier tokens and
 *    itself.
 *  - "Efficiently Scaling Transformer Inference", section 3.4, "Attention
 *    Layer Partitioning": with multiquery attention all query heads share one
 *    key head and one value head; a decode step brings one query token per
 *    sequence and computes dot-product attention Q K^T against the cache.
 *  - "Tensor Parallelism: Splitting Operations Across GPUs", sections
 *    "Splitting attention by head" (each head has its own softmax and its own
 *    weighted sum of values) and "The GQA ceiling: a worked memory audit"
 *    (grouped-query attention: consecutive groups of query heads share one
 *    key/value head).
 *
 * Readings where the pages are silent:
 *  - query head h uses key/value head h / (Hq / Hkv);
 *  - the logits are scale * q.k with `scale` supplied by the caller;
 *  - a sequence of length 0 produces an all-zero output row;
 *  - positions >= seq_lens[b] are never read (they may hold anything).
 *
 * Inputs are raw bfloat16 bit patterns (uint16_t).  Each value is widened to
 * double exactly: the 16 bits are the top half of an IEEE binary32.
 *
 * Parity pins for every function here live in the CPU test suite (closed
 * forms, a library attention routine in float64, invariants, and the
 * decode == last-causal-row identity).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of one bfloat16 bit pattern. */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int check_shape(int B, int Hq, int Hkv, int D, int Lmax)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Lmax < 0) return -1;
    if (Hq % Hkv != 0) return -2;
    return 0;
}

int oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One decode step.
 *   q        [B, Hq, D]          bf16 bits
 *   k, v     [B, Lmax, Hkv, D]   bf16 bits (the cache; position-major)
 *   seq_lens [B]                 each in [0, Lmax]
 *   out      [B, Hq, D]          double, fully written
 *   lse      [B, Hq] or NULL     natural-log log-sum-exp of the scaled logits
 *                                (-INFINITY when the sequence is empty)
 * For each (b, h) with n = seq_lens[b] and g = h / (Hq / Hkv):
 *   s_j   = scale * sum_d q[b,h,d] * k[b,j,g,d]          for j in [0, n)
 *   w_j   = exp(s_j - max_j s_j)
 *   out   = (sum_j w_j * v[b,j,g,:]) / (sum_j w_j)
 * Returns 0 on success, a negative code on a bad shape or length.
 */
int oracle_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const int32_t *seq_lens, int B, int Hq, int Hkv, int D,
                  int Lmax, double scale, double *out, double *lse)
{
    int rc = check_shape(B, Hq, Hkv, D, Lmax);
    if (rc) return rc;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > Lmax) return -3;

    const int G = Hq / Hkv;
    const long long pairs = (long long)B * Hq;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < pairs; ++bh) {
        const int b = (int)(bh / Hq);
        const int h = (int)(bh % Hq);
        const int g = h / G;
        const int n = seq_lens[b];
        double *o = out + ((size_t)b * Hq + h) * D;

        if (n == 0) {
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            if (lse) lse[bh] = -INFINITY;
            continue;
        }

        double *s = (double *)malloc((size_t)n * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const uint16_t *qrow = q + ((size_t)b * Hq + h) * D;

        /* logits */
        for (int j = 0; j < n; ++j) {
            const uint16_t *krow = k + (((size_t)b * Lmax + j) * Hkv + g) * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += bf16_bits_to_double(qrow[d]) * bf16_bits_to_double(krow[d]);
            s[j] = scale * acc;
        }

        /* softmax weights, shifted by the maximum for range safety */
        double m = s[0];
        for (int j = 1; j < n; ++j)
            if (s[j] > m) m = s[j];
        double Z = 0.0;
        for (int j = 0; j < n; ++j) {
            s[j] = exp(s[j] - m);
            Z += s[j];
        }

        /* weighted sum of the value rows */
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int j = 0; j < n; ++j) {
            const uint16_t *vrow = v + (((size_t)b * Lmax + j) * Hkv + g) * D;
            for (int d = 0; d < D; ++d)
                o[d] += s[j] * bf16_bits_to_double(vrow[d]);
        }
        for (int d = 0; d < D; ++d) o[d] /= Z;
        if (lse) lse[bh] = m + log(Z);
        free(s);
    }
    return failed ? -4 : 0;
}

/*
 * One decode step over a paged cache ("Machine Learning Engineering and AI
 * Systems at Scale", section "The key and value cache": fixed-size blocks of
 * positions and a per-sequence block table mapping logical positions to
 * physical blocks; "How To Scale Your Model", Part 7, passage on ragged reads
 * and paged attention).
 *   k_pages, v_pages [num_pages, page_size, Hkv, D]  bf16 bits
 *   block_table      [B, max_blocks]: physical page of each block of
 *                    page_size logical positions; entries past a sequence's
 *                    last block are never read
 *   seq_lens         [B], each in [0, max_blocks * page_size]
 * Position j of sequence b is row (j mod page_size) of page
 * block_table[b][j / page_size].  The attention itself is the one of
 * oracle_decode, step for step.  Returns 0, or a negative code on a bad shape,
 * length or page index.
 */
int oracle_decode_paged(const uint16_t *q, const uint16_t *k_pages,
                        const uint16_t *v_pages, const int32_t *block_table,
                        const int32_t *seq_lens, int B, int Hq, int Hkv, int D,
                        int num_pages, int page_size, int max_blocks,
                        double scale, double *out)
{
    if (num_pages < 0 || page_size <= 0 || max_blocks < 0) return -1;
    int rc = check_shape(B, Hq, Hkv, D, 0);
    if (rc) return rc;
    for (int b = 0; b < B; ++b) {
        const int n = seq_lens[b];
        if (n < 0 || (long long)n > (long long)max_blocks * page_size) return -3;
        for (int blk = 0; blk * page_size < n; ++blk) {
            const int page = block_table[(size_t)b * max_blocks + blk];
            if (page < 0 || page >= num_pages) return -5;
        }
    }

    const int G = Hq / Hkv;
    const long long pairs = (long long)B * Hq;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < pairs; ++bh) {
        const int b = (int)(bh / Hq);
        const int h = (int)(bh % Hq);
        const int g = h / G;
        const int n = seq_lens[b];
        const int32_t *table = block_table + (size_t)b * max_blocks;
        double *o = out + ((size_t)b * Hq + h) * D;

        if (n == 0) {
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            continue;
        }
        double *s = (double *)malloc((size_t)n * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const uint16_t *qrow = q + ((size_t)b * Hq + h) * D;

        /* logits, each key row found through the block table */
        for (int j = 0; j < n; ++j) {
            const size_t row = (size_t)table[j / page_size] * page_size + (size_t)(j % page_size);
            const uint16_t *krow = k_pages + (row * Hkv + g) * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += bf16_bits_to_double(qrow[d]) * bf16_bits_to_double(krow[d]);
            s[j] = scale * acc;
        }

        /* softmax weights, shifted by the maximum for range safety */
        double m = s[0];
        for (int j = 1; j < n; ++j)
            if (s[j] > m) m = s[j];
        double Z = 0.0;
        for (int j = 0; j < n; ++j) {
            s[j] = exp(s[j] - m);
            Z += s[j];
        }

        /* weighted sum of the value rows, found the same way */
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int j = 0; j < n; ++j) {
            const size_t row = (size_t)table[j / page_size] * page_size + (size_t)(j % page_size);
            const uint16_t *vrow = v_pages + (row * Hkv + g) * D;
            for (int d = 0; d < D; ++d)
                o[d] += s[j] * bf16_bits_to_double(vrow[d]);
        }
        for (int d = 0; d < D; ++d) o[d] /= Z;
        free(s);
    }
    return failed ? -4 : 0;
}

/*
 * One decode step with local (sliding-window) attention ("How To Scale Your
 * Model", Part 7 "Transformer Inference", passage on mixing in local attention
 * layers: local attention caps the context a token sees, its mask being a
 * diagonal strip rather than a triangle).  A strip of width `window` seen from
 * the newest position n-1 covers positions max(0, n - window) .. n-1, so for
 * each (b, h), with lo = max(0, n - window):
 *   s_j   = scale * sum_d q[b,h,d] * k[b,j,g,d]          for j in [lo, n)
 *   out   = sum_{j in [lo, n)} softmax(s)_j * v[b,j,g,:]
 * Positions below lo are never read.  window >= 1; shapes as oracle_decode.
 * Returns 0, or a negative code on a bad shape, length or window.
 */
int oracle_decode_window(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const int32_t *seq_lens, int B, int Hq, int Hkv, int D,
                         int Lmax, int window, double scale, double *out)
{
    int rc = check_shape(B, Hq, Hkv, D, Lmax);
    if (rc) return rc;
    if (window < 1) return -6;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > Lmax) return -3;

    const int G = Hq / Hkv;
    const long long pairs = (long long)B * Hq;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < pairs; ++bh) {
        const int b = (int)(bh / Hq);
        const int h = (int)(bh % Hq);
        const int g = h / G;
        const int n = seq_lens[b];
        const int lo = n > window ? n - window : 0;
        double *o = out + ((size_t)b * Hq + h) * D;

        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (n == 0) continue;

        double *s = (double *)malloc((size_t)(n - lo) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const uint16_t *qrow = q + ((size_t)b * Hq + h) * D;

        /* logits of the positions inside the window; s[j - lo] is position j */
        for (int j = lo; j < n; ++j) {
            const uint16_t *krow = k + (((size_t)b * Lmax + j) * Hkv + g) * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += bf16_bits_to_double(qrow[d]) * bf16_bits_to_double(krow[d]);
            s[j - lo] = scale * acc;
        }

        double m = s[0];
        for (int j = lo + 1; j < n; ++j)
            if (s[j - lo] > m) m = s[j - lo];
        double Z = 0.0;
        for (int j = lo; j < n; ++j) {
            s[j - lo] = exp(s[j - lo] - m);
            Z += s[j - lo];
        }

        for (int j = lo; j < n; ++j) {
            const uint16_t *vrow = v + (((size_t)b * Lmax + j) * Hkv + g) * D;
            for (int d = 0; d < D; ++d)
                o[d] += s[j - lo] * bf16_bits_to_double(vrow[d]);
        }
        for (int d = 0; d < D; ++d) o[d] /= Z;
        free(s);
    }
    return failed ? -4 : 0;
}

/*
 * Local (sliding-window) causal attention over whole sequences with no cache,
 * as the pages describe it for training and prefill: the score matrix is
 * masked to a diagonal strip of width `window` (row i keeps columns j with
 * i - window < j <= i), then a row softmax and the product with V.  Written
 * in the same masked full-matrix form as oracle_causal_prefill, independently
 * of the decode loops.  Shapes as oracle_causal_prefill; rows i >= n are zero.
 */
int oracle_local_prefill(const uint16_t *q_seq, const uint16_t *k,
                         const uint16_t *v, const int32_t *seq_lens, int B,
                         int Hq, int Hkv, int D, int Lmax, int window,
                         double scale, double *out_seq)
{
    int rc = check_shape(B, Hq, Hkv, D, Lmax);
    if (rc) return rc;
    if (window < 1) return -6;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > Lmax) return -3;

    const int G = Hq / Hkv;
    const long long rows = (long long)B * Lmax * Hq;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 4)
    for (long long r = 0; r < rows; ++r) {
        const int h = (int)(r % Hq);
        const int i = (int)((r / Hq) % Lmax);
        const int b = (int)(r / ((long long)Hq * Lmax));
        const int n = seq_lens[b];
        double *o = out_seq + (size_t)r * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (i >= n) continue;

        const int kvh = h / G;
        double *S = (double *)malloc((size_t)n * sizeof(double));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const uint16_t *qrow = q_seq + (size_t)r * D;
        for (int j = 0; j < n; ++j) {
            if (j > i || j <= i - window) { /* outside the strip */
                S[j] = -INFINITY;
                continue;
            }
            const uint16_t *krow = k + (((size_t)b * Lmax + j) * Hkv + kvh) * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += bf16_bits_to_double(qrow[d]) * bf16_bits_to_double(krow[d]);
            S[j] = scale * acc;
        }
        double rowmax = -INFINITY;
        for (int j = 0; j < n; ++j)
            if (S[j] > rowmax) rowmax = S[j];
        double denom = 0.0;
        for (int j = 0; j < n; ++j) denom += exp(S[j] - rowmax);
        for (int j = 0; j < n; ++j) {
            if (S[j] == -INFINITY) continue; /* masked entries: never touch their V */
            const double p = exp(S[j] - rowmax) / denom;
            const uint16_t *vrow = v + (((size_t)b * Lmax + j) * Hkv + kvh) * D;
            for (int d = 0; d < D; ++d) o[d] += p * bf16_bits_to_double(vrow[d]);
        }
        free(S);
    }
    return failed ? -4 : 0;
}

/*
 * Value of one 8-bit E4M3 floating-point code, the 8-bit format the pages name
 * for inference ("Machine Learning Engineering and AI Systems at Scale",
 * section "Quantization": E4M3 for weights and activations), decoded from its
 * fields: sign bit 7, a 4-bit exponent in bits 6..3 with bias 7, a 3-bit
 * mantissa in bits 2..0.  Exponent 0 is subnormal (mantissa * 2^-9); the
 * all-ones exponent with all-ones mantissa is NaN; there is no infinity (the
 * largest finite magnitude is 448).
 */
double oracle_fp8_e4m3_value(uint8_t code)
{
    const int sign = code >> 7;
    const int e = (code >> 3) & 15;
    const int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Value of one stored 8-bit code: E4M3 (format 1) or two's-complement int8
 * (format 2). */
static double code_value(uint8_t code, int format)
{
    if (format == 1) return oracle_fp8_e4m3_value(code);
    return (double)(int8_t)code;
}

/*
 * One decode step against a KV cache quantized to 8 bits per element ("How
 * To Scale Your Model", Part 7 "Transformer Inference", passage on
 * quantization: the KV cache can be stored in int8 or fp8 to save memory
 * bandwidth; "Machine Learning Engineering and AI Systems at Scale", section
 * "Quantization": E4M3 is the inference format, and the key/value cache is
 * the second thing to quantize).  Each cached row (one position of one kv
 * head) holds D codes and one fp32 scale per tensor; its values are
 * code * scale:
 *   kq, vq     [B, Lmax, Hkv, D]   8-bit codes (format 1: E4M3, 2: int8)
 *   ks, vs     [B, Hkv, Lmax]      fp32 scales, one per cached row
 *   K[b,j,g,d] = code(kq[b,j,g,d]) * ks[b,g,j]     (likewise V)
 * and the attention is the one of oracle_decode on those values, step for
 * step.  Returns 0, or a negative code on a bad shape, length or format.
 */
int oracle_decode_quant(const uint16_t *q, const uint8_t *kq, const uint8_t *vq,
                        const float *ks, const float *vs, const int32_t *seq_lens,
                        int B, int Hq, int Hkv, int D, int Lmax, int format,
                        double scale, double *out)
{
    int rc = check_shape(B, Hq, Hkv, D, Lmax);
    if (rc) return rc;
    if (format != 1 && format != 2) return -7;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > Lmax) return -3;

    const int G = Hq / Hkv;
    const long long pairs = (long long)B * Hq;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < pairs; ++bh) {
        const int b = (int)(bh / Hq);
        const int h = (int)(bh % Hq);
        const int g = h / G;
        const int n = seq_lens[b];
        double *o = out + ((size_t)b * Hq + h) * D;

        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (n == 0) continue;

        double *s = (double *)malloc((size_t)n * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const uint16_t *qrow = q + ((size_t)b * Hq + h) * D;
        const float *kscale = ks + ((size_t)b * Hkv + g) * Lmax;
        const float *vscale = vs + ((size_t)b * Hkv + g) * Lmax;

        /* logits against the dequantized keys */
        for (int j = 0; j < n; ++j) {
            const uint8_t *krow = kq + (((size_t)b * Lmax + j) * Hkv + g) * D;
            const double sk = (double)kscale[j];
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += bf16_bits_to_double(qrow[d]) * (code_value(krow[d], format) * sk);
            s[j] = scale * acc;
        }

        double m = s[0];
        for (int j = 1; j < n; ++j)
            if (s[j] > m) m = s[j];
        double Z = 0.0;
        for (int j = 0; j < n; ++j) {
            s[j] = exp(s[j] - m);
            Z += s[j];
        }

        /* weighted sum of the dequantized value rows */
        for (int j = 0; j < n; ++j) {
            const uint8_t *vrow = vq + (((size_t)b * Lmax + j) * Hkv + g) * D;
            const double sv = (double)vscale[j];
            for (int d = 0; d < D; ++d)
                o[d] += s[j] * (code_value(vrow[d], format) * sv);
        }
        for (int d = 0; d < D; ++d) o[d] /= Z;
        free(s);
    }
    return failed ? -4 : 0;
}

/*
 * Decode of T new tokens per sequence at once (speculative verification,
 * chunked prefill: "How To Scale Your Model", Part 7 "Transformer Inference",
 * passages on prefill and on speculative sampling, where several new tokens
 * are scored against the cache in one step).  The T tokens' own keys and
 * values are already in the cache at positions n-T .. n-1 (n = seq_lens[b]),
 * and they are causal among themselves: token i (0 .. T-1) sits at position
 * n-T+i and attends positions 0 .. n-T+i.  A token whose position would be
 * negative (n < T) attends nothing and gets a zero row.
 *   q    [B, T, Hq, D]   bf16 bits
 *   k, v [B, Lmax, Hkv, D]
 *   out  [B, T, Hq, D]   double
 * Each (b, i, h) is the attention of oracle_decode with length n-T+i+1.
 * Returns 0, or a negative code on a bad shape, length or token count.
 */
int oracle_decode_multi(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const int32_t *seq_lens, int B, int T, int Hq, int Hkv, int D,
                        int Lmax, double scale, double *out)
{
    int rc = check_shape(B, Hq, Hkv, D, Lmax);
    if (rc) return rc;
    if (T < 1) return -8;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > Lmax) return -3;

    const int G = Hq / Hkv;
    const long long rows = (long long)B * T * Hq;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long r = 0; r < rows; ++r) {
        const int h = (int)(r % Hq);
        const int i = (int)((r / Hq) % T);
        const int b = (int)(r / ((long long)Hq * T));
        const int g = h / G;
        const int n = seq_lens[b] - T + 1 + i; /* positions token i attends */
        double *o = out + (size_t)r * D;

        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (n <= 0) continue;

        double *s = (double *)malloc((size_t)n * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const uint16_t *qrow = q + (size_t)r * D;
        for (int j = 0; j < n; ++j) {
            const uint16_t *krow = k + (((size_t)b * Lmax + j) * Hkv + g) * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += bf16_bits_to_double(qrow[d]) * bf16_bits_to_double(krow[d]);
            s[j] = scale * acc;
        }
        double m = s[0];
        for (int j = 1; j < n; ++j)
            if (s[j] > m) m = s[j];
        double Z = 0.0;
        for (int j = 0; j < n; ++j) {
            s[j] = exp(s[j] - m);
            Z += s[j];
        }
        for (int j = 0; j < n; ++j) {
            const uint16_t *vrow = v + (((size_t)b * Lmax + j) * Hkv + g) * D;
            for (int d = 0; d < D; ++d)
                o[d] += s[j] * bf16_bits_to_double(vrow[d]);
        }
        for (int d = 0; d < D; ++d) o[d] /= Z;
        free(s);
    }
    return failed ? -4 : 0;
}

/*
 * Full causal self-attention over a whole sequence, recomputed with no cache
 * (the work the KV cache avoids).
 *   q_seq   [B, Lmax, Hq, D]   bf16 bits: one query per position
 *   k, v    [B, Lmax, Hkv, D]  bf16 bits
 *   seq_lens[B]
 *   out_seq [B, Lmax, Hq, D]   double; row i < n attends positions 0..i,
 *                              rows i >= n are zero.
 * Written as the textbook masked form: the full score row S[i, 0..n) is
 * built, entries with j > i are set to -infinity, then a row softmax and the
 * product with V follow.  It deliberately does not reuse the decode loop.
 */
int oracle_causal_prefill(const uint16_t *q_seq, const uint16_t *k,
                          const uint16_t *v, const int32_t *seq_lens, int B,
                          int Hq, int Hkv, int D, int Lmax, double scale,
                          double *out_seq)
{
    int rc = check_shape(B, Hq, Hkv, D, Lmax);
    if (rc) return rc;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > Lmax) return -3;

    const int G = Hq / Hkv;
    const long long rows = (long long)B * Lmax * Hq;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 4)
    for (long long r = 0; r < rows; ++r) {
        const int h = (int)(r % Hq);
        const int i = (int)((r / Hq) % Lmax);
        const int b = (int)(r / ((long long)Hq * Lmax));
        const int n = seq_lens[b];
        double *o = out_seq + (size_t)r * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (i >= n) continue;

        const int kvh = h / G;
        double *S = (double *)malloc((size_t)n * sizeof(double));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const uint16_t *qrow = q_seq + (size_t)r * D;
        for (int j = 0; j < n; ++j) {
            const uint16_t *krow = k + (((size_t)b * Lmax + j) * Hkv + kvh) * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += bf16_bits_to_double(qrow[d]) * bf16_bits_to_double(krow[d]);
            S[j] = (j > i) ? -INFINITY : scale * acc;
        }
        double rowmax = -INFINITY;
        for (int j = 0; j < n; ++j)
            if (S[j] > rowmax) rowmax = S[j];
        double denom = 0.0;
        for (int j = 0; j < n; ++j) denom += exp(S[j] - rowmax);
        for (int j = 0; j < n; ++j) {
            const double p = exp(S[j] - rowmax) / denom;
            if (p == 0.0) continue; /* masked entries: never touch their V */
            const uint16_t *vrow = v + (((size_t)b * Lmax + j) * Hkv + kvh) * D;
            for (int d = 0; d < D; ++d) o[d] += p * bf16_bits_to_double(vrow[d]);
        }
        free(S);
    }
    return failed ? -4 : 0;
}
