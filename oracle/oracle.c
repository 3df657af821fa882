/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for the stable LSD
 * radix sort, the positive-value stream compaction and the bitonic tile.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; the two meet only through the seeded input
 * generators and through comparisons made by the tests.
 *
 * What it computes, and the passages it follows:
 *
 *  - oracle_lsd_sort_u32: the least-significant-digit radix sort as a
 *    sequence of stable counting sorts, one per digit, from the lowest digit
 *    up ("CUDA 算子笔记 3", section "Radix Sort", the CPU code: zero the
 *    counts, count each digit, turn the counts into exclusive starts, then
 *    place each element at its digit's next free slot in input order, swap
 *    buffers).  The textbook chapter ("第10章 并行模式：排序", 10.3 Radix Sort
 *    算法) gives the same four steps and states that the sort is stable; the
 *    WebGPU chapter ("WebGPU Unleashed", 4.1 래딕스 정렬) states that each
 *    digit pass must be stable for the LSD order to be correct.  The pages
 *    always sort all 32 bits; here a bit range [begin_bit, end_bit) selects
 *    the ordering field and the last digit is narrowed to the bits left.
 *    Values, when given, move with their keys (10.6 Key-Value排序).
 *  - oracle_sort_pairs_f32: the float exercise of the same chapter (八、习题,
 *    the IEEE 754 preprocessing question) answered by the usual
 *    order-preserving bit transform: negative patterns are inverted, the
 *    sign bit of non-negative patterns is set; the sort runs on the
 *    transformed bits and the transform is undone on the way out.  Only
 *    integer operations touch the keys.
 *  - oracle_digit_histograms: the per-pass digit counts the multi-bit
 *    radix sort starts from ("CUDA 算子笔记 3", section 一次处理多位, the first
 *    kernel: one read of the keys counts every pass's digits).
 *  - oracle_compact_positive_f32: "CUDA 算子笔记 3", section Stream
 *    Compaction: keep the values greater than zero, in input order, at the
 *    front of the output; the rest of the output holds zeros (the worked
 *    example shows the zero tail); the kept count is returned.
 *  - oracle_bitonic_tile: each run of `tile` consecutive keys is sorted on
 *    its own by the same field, stably.  A bitonic network that compares
 *    (field, original index) pairs -- the form used on the GPU because the
 *    network itself is not stable ("第10章", 10.7 稳定排序 vs 不稳定排序) --
 *    reaches exactly this result, so the oracle is the definition.
 *  - oracle_lsd_sort_u64: the same digit-by-digit stable counting sort on
 *    64-bit keys; with 8-bit digits a full 64-bit key takes eight passes
 *    ("第10章", 八、习题: the exercise on iteration counts for 64-bit
 *    integers).
 *  - oracle_sort_typed: keys of six types (u32, i32, f32, u64, i64, f64),
 *    ascending or descending, with optional u32 values.  Each key is mapped
 *    to an unsigned "order pattern" whose unsigned order is the type's
 *    order: unsigned keys as they are, signed keys offset by 2^(w-1)
 *    (two's complement values -2^(w-1) .. 2^(w-1)-1 onto 0 .. 2^w-1), floats
 *    by the sign-dependent transform above (the float exercise of 八、习题);
 *    descending order replaces the pattern p by its complement 2^w - 1 - p
 *    (the exercise on descending sorts), which reverses the order and keeps
 *    equal keys equal, so the sort stays stable.  The bit range selects bits
 *    of that pattern.  The oracle sorts (pattern, original index) with the
 *    LSD sort and then gathers the original keys and values by index, so it
 *    never needs an inverse transform.
 *  - oracle_sort_two_keys: the multi-key exercise of 八、习题 done as the
 *    exercise states it: a stable sort by the first key, then a stable sort
 *    of that result by the second key.  The result is ordered by the second
 *    key, then by the first, then by input position.
 *  - oracle_digit_histograms_typed: per-pass digit counts of the order
 *    patterns of any of the six key types (up to eight passes).
 *  - oracle_scan_u32: the prefix sum the sort and the compaction are built
 *    on ("CUDA 算子笔记 3", the scan methods of the Stream Compaction
 *    section; "WebGPU Unleashed", 4.1: a digit pass as a prefix sum of digit
 *    occurrences), exclusive or inclusive, in unsigned 32-bit arithmetic
 *    (sums wrap modulo 2^32), by a plain running sum.
 *  - oracle_select: the general form of the compaction ("CUDA 算子笔记 3",
 *    Stream Compaction: predicate, scan, scatter): keep the elements whose
 *    value satisfies `value OP threshold` (OP one of <, <=, >, >=, ==, !=,
 *    compared as u32, i32 or f32 values with C semantics, so every
 *    comparison with a NaN is false except !=), in input order, with
 *    optional values moved alongside.  In partition mode the rejected
 *    elements follow the kept ones, also in input order: the stable split
 *    that one radix-sort pass per bit performs ("CUDA 算子笔记 3", Radix
 *    Sort, the one-bit split).  Returns the kept count.
 *
 * Floating point: the compaction predicate is the C comparison x > 0.0f on
 * the float value, as the pages write it.  This file must be built without
 * -ffast-math; a pin test checks that positive subnormals are kept, which
 * would fail if denormals were flushed in the calling process.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS (-1)
#define ORACLE_NO_MEMORY (-2)

/* The digit of `key` that starts at bit `shift` and is `width` bits wide. */
static uint32_t digit_at(uint32_t key, int shift, int width)
{
    uint32_t mask = (width >= 32) ? 0xFFFFFFFFu : ((1u << width) - 1u);
    return (key >> shift) & mask;
}

/*
 * One stable counting-sort pass on the digit at [shift, shift + width).
 * src/dst keys (and values when src_vals != NULL).
 */
static void counting_sort_pass(const uint32_t *src_keys, const uint32_t *src_vals,
                               uint32_t *dst_keys, uint32_t *dst_vals, uint64_t n,
                               int shift, int width, uint64_t *cnt)
{
    uint64_t buckets = (uint64_t)1 << width;
    uint64_t d, j, sum;

    for (d = 0; d < buckets; ++d)
        cnt[d] = 0;
    for (j = 0; j < n; ++j)
        cnt[digit_at(src_keys[j], shift, width)] += 1;

    /* exclusive scan: cnt[d] becomes the first output slot of digit d */
    sum = 0;
    for (d = 0; d < buckets; ++d) {
        uint64_t c = cnt[d];
        cnt[d] = sum;
        sum += c;
    }

    /* scatter in input order: equal digits keep their relative order */
    for (j = 0; j < n; ++j) {
        uint32_t dg = digit_at(src_keys[j], shift, width);
        uint64_t slot = cnt[dg];
        cnt[dg] = slot + 1;
        dst_keys[slot] = src_keys[j];
        if (src_vals)
            dst_vals[slot] = src_vals[j];
    }
}

/*
 * Stable LSD radix sort of (keys, vals) by bits [begin_bit, end_bit) of the
 * key, with digits of `digit_bits` bits (1..16); the last digit is narrowed.
 * vals_in/vals_out may both be NULL (keys only).  Inputs are not modified.
 * Returns 0, or a negative code on bad arguments or allocation failure.
 */
int oracle_lsd_sort_u32(const uint32_t *keys_in, const uint32_t *vals_in,
                        uint32_t *keys_out, uint32_t *vals_out, uint64_t n,
                        int begin_bit, int end_bit, int digit_bits)
{
    uint32_t *ka, *kb, *va = NULL, *vb = NULL, *tk, *tv;
    uint64_t *cnt;
    int shift;
    int pairs = (vals_in != NULL);

    if (begin_bit < 0 || end_bit > 32 || begin_bit > end_bit)
        return ORACLE_BAD_ARGS;
    if (digit_bits < 1 || digit_bits > 16)
        return ORACLE_BAD_ARGS;
    if ((vals_in == NULL) != (vals_out == NULL))
        return ORACLE_BAD_ARGS;
    if (n == 0)
        return ORACLE_OK;

    ka = (uint32_t *)malloc(n * sizeof(uint32_t));
    kb = (uint32_t *)malloc(n * sizeof(uint32_t));
    cnt = (uint64_t *)malloc(((size_t)1 << digit_bits) * sizeof(uint64_t));
    if (pairs) {
        va = (uint32_t *)malloc(n * sizeof(uint32_t));
        vb = (uint32_t *)malloc(n * sizeof(uint32_t));
    }
    if (!ka || !kb || !cnt || (pairs && (!va || !vb))) {
        free(ka); free(kb); free(cnt); free(va); free(vb);
        return ORACLE_NO_MEMORY;
    }

    memcpy(ka, keys_in, n * sizeof(uint32_t));
    if (pairs)
        memcpy(va, vals_in, n * sizeof(uint32_t));

    for (shift = begin_bit; shift < end_bit; shift += digit_bits) {
        int width = end_bit - shift;
        if (width > digit_bits)
            width = digit_bits;
        counting_sort_pass(ka, va, kb, vb, n, shift, width, cnt);
        tk = ka; ka = kb; kb = tk;
        tv = va; va = vb; vb = tv;
    }

    memcpy(keys_out, ka, n * sizeof(uint32_t));
    if (pairs)
        memcpy(vals_out, va, n * sizeof(uint32_t));

    free(ka); free(kb); free(cnt); free(va); free(vb);
    return ORACLE_OK;
}

/* Order-preserving transform of an IEEE 754 binary32 bit pattern. */
static uint32_t f32_to_order(uint32_t u)
{
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

/* Inverse of f32_to_order. */
static uint32_t order_to_f32(uint32_t o)
{
    return (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
}

void oracle_f32_to_order(const uint32_t *bits_in, uint32_t *order_out, uint64_t n)
{
    uint64_t i;
    for (i = 0; i < n; ++i)
        order_out[i] = f32_to_order(bits_in[i]);
}

void oracle_order_to_f32(const uint32_t *order_in, uint32_t *bits_out, uint64_t n)
{
    uint64_t i;
    for (i = 0; i < n; ++i)
        bits_out[i] = order_to_f32(order_in[i]);
}

/*
 * Stable sort of float keys (given as raw bit patterns) with optional u32
 * values.  [begin_bit, end_bit) selects bits of the transformed pattern;
 * (0, 32) is the full IEEE 754 totalOrder.  Output keys are the original
 * bit patterns in sorted order.
 */
int oracle_sort_pairs_f32(const uint32_t *key_bits_in, const uint32_t *vals_in,
                          uint32_t *key_bits_out, uint32_t *vals_out, uint64_t n,
                          int begin_bit, int end_bit, int digit_bits)
{
    uint32_t *ord;
    uint64_t i;
    int rc;

    if (n == 0)
        return oracle_lsd_sort_u32(key_bits_in, vals_in, key_bits_out, vals_out, 0,
                                   begin_bit, end_bit, digit_bits);
    ord = (uint32_t *)malloc(n * sizeof(uint32_t));
    if (!ord)
        return ORACLE_NO_MEMORY;
    for (i = 0; i < n; ++i)
        ord[i] = f32_to_order(key_bits_in[i]);
    rc = oracle_lsd_sort_u32(ord, vals_in, key_bits_out, vals_out, n, begin_bit,
                             end_bit, digit_bits);
    if (rc == ORACLE_OK)
        for (i = 0; i < n; ++i)
            key_bits_out[i] = order_to_f32(key_bits_out[i]);
    free(ord);
    return rc;
}

/*
 * Digit counts for every 8-bit pass over [begin_bit, end_bit):
 * counts[p * 256 + d] = number of keys whose pass-p digit equals d, where
 * pass p covers bits [begin_bit + 8p, min(begin_bit + 8p + 8, end_bit)).
 * With transform_f32 != 0 the keys are float bit patterns and the counts
 * are taken on their order-preserving transform.  counts must hold
 * ceil((end_bit - begin_bit) / 8) * 256 entries.  Returns the pass count,
 * or a negative code.
 */
int oracle_digit_histograms(const uint32_t *keys, uint64_t n, int begin_bit, int end_bit,
                            int transform_f32, uint64_t *counts)
{
    int passes, p;
    uint64_t i;

    if (begin_bit < 0 || end_bit > 32 || begin_bit > end_bit)
        return ORACLE_BAD_ARGS;
    passes = (end_bit - begin_bit + 7) / 8;
    for (i = 0; i < (uint64_t)passes * 256u; ++i)
        counts[i] = 0;
    for (p = 0; p < passes; ++p) {
        int shift = begin_bit + 8 * p;
        int width = end_bit - shift;
        if (width > 8)
            width = 8;
        for (i = 0; i < n; ++i) {
            uint32_t k = transform_f32 ? f32_to_order(keys[i]) : keys[i];
            counts[(uint64_t)p * 256u + digit_at(k, shift, width)] += 1;
        }
    }
    return passes;
}

/*
 * Keep x > 0.0f in input order at the front of out, fill the rest with
 * +0.0f, return the kept count.  in/out are float arrays of length n.
 */
uint64_t oracle_compact_positive_f32(const float *in, float *out, uint64_t n)
{
    uint64_t i, k = 0;
    for (i = 0; i < n; ++i) {
        float x = in[i];
        if (x > 0.0f) {
            memcpy(&out[k], &in[i], sizeof(float));
            k += 1;
        }
    }
    for (i = k; i < n; ++i)
        out[i] = 0.0f;
    return k;
}

/*
 * Each run [s, min(s + tile, n)) of the keys, s = 0, tile, 2 tile, ..., is
 * stably sorted on its own by bits [begin_bit, end_bit).
 */
int oracle_bitonic_tile(const uint32_t *keys_in, uint32_t *keys_out, uint64_t n,
                        uint64_t tile, int begin_bit, int end_bit)
{
    uint64_t s;
    int rc;

    if (tile == 0)
        return ORACLE_BAD_ARGS;
    for (s = 0; s < n; s += tile) {
        uint64_t len = (n - s < tile) ? (n - s) : tile;
        rc = oracle_lsd_sort_u32(keys_in + s, NULL, keys_out + s, NULL, len, begin_bit,
                                 end_bit, 8);
        if (rc != ORACLE_OK)
            return rc;
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* 64-bit keys, key types and multi-key sorts                                */
/* ------------------------------------------------------------------------ */

/* The digit of a 64-bit key that starts at bit `shift` and is `width` bits wide. */
static uint64_t digit_at64(uint64_t key, int shift, int width)
{
    uint64_t low_bits = (width >= 64) ? ~(uint64_t)0 : (((uint64_t)1 << width) - 1);
    return (key >> shift) & low_bits;
}

/* One stable counting-sort pass of 64-bit keys (values optional). */
static void counting_sort_pass64(const uint64_t *src_keys, const uint32_t *src_vals,
                                 uint64_t *dst_keys, uint32_t *dst_vals, uint64_t n,
                                 int shift, int width, uint64_t *cnt)
{
    uint64_t buckets = (uint64_t)1 << width;
    uint64_t d, j, running;

    for (d = 0; d < buckets; ++d)
        cnt[d] = 0;
    for (j = 0; j < n; ++j)
        cnt[digit_at64(src_keys[j], shift, width)] += 1;
    /* exclusive scan: cnt[d] becomes the first output slot of digit d */
    running = 0;
    for (d = 0; d < buckets; ++d) {
        uint64_t here = cnt[d];
        cnt[d] = running;
        running += here;
    }
    /* scatter in input order */
    for (j = 0; j < n; ++j) {
        uint64_t dg = digit_at64(src_keys[j], shift, width);
        uint64_t at = cnt[dg]++;
        dst_keys[at] = src_keys[j];
        if (src_vals)
            dst_vals[at] = src_vals[j];
    }
}

/*
 * Stable LSD radix sort of 64-bit keys (with optional u32 values) by bits
 * [begin_bit, end_bit), 0 <= begin_bit <= end_bit <= 64, digits of
 * `digit_bits` bits (1..16), the last one narrowed.
 */
int oracle_lsd_sort_u64(const uint64_t *keys_in, const uint32_t *vals_in,
                        uint64_t *keys_out, uint32_t *vals_out, uint64_t n,
                        int begin_bit, int end_bit, int digit_bits)
{
    uint64_t *ka, *kb, *tk, *cnt;
    uint32_t *va = NULL, *vb = NULL, *tv;
    int shift;
    int pairs = (vals_in != NULL);

    if (begin_bit < 0 || end_bit > 64 || begin_bit > end_bit)
        return ORACLE_BAD_ARGS;
    if (digit_bits < 1 || digit_bits > 16)
        return ORACLE_BAD_ARGS;
    if ((vals_in == NULL) != (vals_out == NULL))
        return ORACLE_BAD_ARGS;
    if (n == 0)
        return ORACLE_OK;

    ka = (uint64_t *)malloc(n * sizeof(uint64_t));
    kb = (uint64_t *)malloc(n * sizeof(uint64_t));
    cnt = (uint64_t *)malloc(((size_t)1 << digit_bits) * sizeof(uint64_t));
    if (pairs) {
        va = (uint32_t *)malloc(n * sizeof(uint32_t));
        vb = (uint32_t *)malloc(n * sizeof(uint32_t));
    }
    if (!ka || !kb || !cnt || (pairs && (!va || !vb))) {
        free(ka); free(kb); free(cnt); free(va); free(vb);
        return ORACLE_NO_MEMORY;
    }
    memcpy(ka, keys_in, n * sizeof(uint64_t));
    if (pairs)
        memcpy(va, vals_in, n * sizeof(uint32_t));

    for (shift = begin_bit; end_bit > shift; shift += digit_bits) {
        /* the last digit keeps only the bits left in the range */
        int width = (end_bit - shift < digit_bits) ? end_bit - shift : digit_bits;
        counting_sort_pass64(ka, va, kb, vb, n, shift, width, cnt);
        tk = ka; ka = kb; kb = tk;
        tv = va; va = vb; vb = tv;
    }

    memcpy(keys_out, ka, n * sizeof(uint64_t));
    if (pairs)
        memcpy(vals_out, va, n * sizeof(uint32_t));
    free(ka); free(kb); free(cnt); free(va); free(vb);
    return ORACLE_OK;
}

/* Key types of oracle_sort_typed (the same numbering as the library's). */
#define ORACLE_KEY_U32 0
#define ORACLE_KEY_I32 1
#define ORACLE_KEY_F32 2
#define ORACLE_KEY_U64 3
#define ORACLE_KEY_I64 4
#define ORACLE_KEY_F64 5

static int key_bits_of(int key_type)
{
    if (key_type >= ORACLE_KEY_U32 && key_type <= ORACLE_KEY_F32)
        return 32;
    if (key_type >= ORACLE_KEY_U64 && key_type <= ORACLE_KEY_F64)
        return 64;
    return 0;
}

/*
 * The order pattern of key i (see the header): unsigned, w = 32 or 64 bits,
 * such that comparing patterns as unsigned integers compares the keys.
 */
static uint64_t order_pattern(int key_type, int descending, const void *keys, uint64_t i)
{
    uint64_t p = 0, top;
    int w = key_bits_of(key_type);
    uint64_t all = (w == 64) ? ~(uint64_t)0 : (uint64_t)0xFFFFFFFFu;

    switch (key_type) {
    case ORACLE_KEY_U32:
        p = ((const uint32_t *)keys)[i];
        break;
    case ORACLE_KEY_I32:
        /* value + 2^31, as an unsigned 32-bit number */
        p = (uint64_t)((int64_t)((const int32_t *)keys)[i] + ((int64_t)1 << 31));
        break;
    case ORACLE_KEY_F32:
        p = f32_to_order(((const uint32_t *)keys)[i]);
        break;
    case ORACLE_KEY_U64:
        p = ((const uint64_t *)keys)[i];
        break;
    case ORACLE_KEY_I64:
        /* value + 2^63 modulo 2^64: the two's complement pattern plus 2^63 */
        p = ((const uint64_t *)keys)[i] + ((uint64_t)1 << 63);
        break;
    case ORACLE_KEY_F64:
        top = (uint64_t)1 << 63;
        p = ((const uint64_t *)keys)[i];
        p = (p & top) ? ~p : (p | top);
        break;
    }
    if (descending)
        p = all - p;
    return p;
}

/*
 * Stable sort of keys of `key_type` (ascending, or descending when
 * `descending` is nonzero) by bits [begin_bit, end_bit) of their order
 * patterns, with optional u32 values; keys_out receives the original keys.
 * Keys are u32/i32/f32 arrays (4 bytes each) or u64/i64/f64 arrays (8 bytes).
 */
int oracle_sort_typed(int key_type, int descending, const void *keys_in,
                      const uint32_t *vals_in, void *keys_out, uint32_t *vals_out,
                      uint64_t n, int begin_bit, int end_bit, int digit_bits)
{
    uint64_t *pat, *pat_sorted, i;
    uint32_t *idx, *idx_sorted;
    int w = key_bits_of(key_type);
    int rc;

    if (w == 0 || begin_bit < 0 || end_bit > w || begin_bit > end_bit)
        return ORACLE_BAD_ARGS;
    if ((vals_in == NULL) != (vals_out == NULL))
        return ORACLE_BAD_ARGS;
    if (n == 0)
        return ORACLE_OK;
    if (n > 0xFFFFFFFFu)
        return ORACLE_BAD_ARGS;

    pat = (uint64_t *)malloc(n * sizeof(uint64_t));
    pat_sorted = (uint64_t *)malloc(n * sizeof(uint64_t));
    idx = (uint32_t *)malloc(n * sizeof(uint32_t));
    idx_sorted = (uint32_t *)malloc(n * sizeof(uint32_t));
    if (!pat || !pat_sorted || !idx || !idx_sorted) {
        free(pat); free(pat_sorted); free(idx); free(idx_sorted);
        return ORACLE_NO_MEMORY;
    }
    for (i = 0; i < n; ++i) {
        pat[i] = order_pattern(key_type, descending, keys_in, i);
        idx[i] = (uint32_t)i;
    }
    rc = oracle_lsd_sort_u64(pat, idx, pat_sorted, idx_sorted, n, begin_bit, end_bit,
                             digit_bits);
    if (rc == ORACLE_OK) {
        for (i = 0; i < n; ++i) {
            uint64_t src = idx_sorted[i];
            if (w == 32)
                ((uint32_t *)keys_out)[i] = ((const uint32_t *)keys_in)[src];
            else
                ((uint64_t *)keys_out)[i] = ((const uint64_t *)keys_in)[src];
            if (vals_in)
                vals_out[i] = vals_in[src];
        }
    }
    free(pat); free(pat_sorted); free(idx); free(idx_sorted);
    return rc;
}

/*
 * Per-pass 8-bit digit counts of the order patterns of `key_type` keys over
 * bits [begin_bit, end_bit) (passes = ceil((end - begin) / 8) <= 8):
 * counts[p * 256 + d].  Returns the pass count, or a negative code.
 */
int oracle_digit_histograms_typed(int key_type, int descending, const void *keys, uint64_t n,
                                  int begin_bit, int end_bit, uint64_t *counts)
{
    int passes, p, w = key_bits_of(key_type);
    uint64_t i;

    if (w == 0 || begin_bit < 0 || end_bit > w || begin_bit > end_bit)
        return ORACLE_BAD_ARGS;
    passes = (end_bit - begin_bit + 7) / 8;
    for (i = 0; i < (uint64_t)passes * 256u; ++i)
        counts[i] = 0;
    for (i = 0; i < n; ++i) {
        uint64_t pat = order_pattern(key_type, descending, keys, i);
        for (p = 0; p < passes; ++p) {
            int shift = begin_bit + 8 * p;
            int width = end_bit - shift;
            if (width > 8)
                width = 8;
            counts[(uint64_t)p * 256u + digit_at64(pat, shift, width)] += 1;
        }
    }
    return passes;
}

/*
 * The multi-key exercise: stably sort by `first`, then stably sort that
 * result by `second`.  Outputs the permuted first keys, second keys and
 * (optional) values.
 */
int oracle_sort_two_keys(const uint32_t *first, const uint32_t *second, const uint32_t *vals,
                         uint32_t *first_out, uint32_t *second_out, uint32_t *vals_out,
                         uint64_t n)
{
    uint32_t *idx, *perm1, *tmp_keys, *second_by1, *perm;
    uint64_t i;
    int rc;

    if ((vals == NULL) != (vals_out == NULL))
        return ORACLE_BAD_ARGS;
    if (n == 0)
        return ORACLE_OK;
    if (n > 0xFFFFFFFFu)
        return ORACLE_BAD_ARGS;
    idx = (uint32_t *)malloc(n * sizeof(uint32_t));
    perm1 = (uint32_t *)malloc(n * sizeof(uint32_t));
    tmp_keys = (uint32_t *)malloc(n * sizeof(uint32_t));
    second_by1 = (uint32_t *)malloc(n * sizeof(uint32_t));
    perm = (uint32_t *)malloc(n * sizeof(uint32_t));
    if (!idx || !perm1 || !tmp_keys || !second_by1 || !perm) {
        free(idx); free(perm1); free(tmp_keys); free(second_by1); free(perm);
        return ORACLE_NO_MEMORY;
    }
    for (i = 0; i < n; ++i)
        idx[i] = (uint32_t)i;
    /* step 1: stable sort of the positions by the first key */
    rc = oracle_lsd_sort_u32(first, idx, tmp_keys, perm1, n, 0, 32, 8);
    if (rc == ORACLE_OK) {
        /* step 2: stable sort of that order by the second key */
        for (i = 0; i < n; ++i)
            second_by1[i] = second[perm1[i]];
        rc = oracle_lsd_sort_u32(second_by1, perm1, tmp_keys, perm, n, 0, 32, 8);
    }
    if (rc == ORACLE_OK) {
        for (i = 0; i < n; ++i) {
            first_out[i] = first[perm[i]];
            second_out[i] = second[perm[i]];
            if (vals)
                vals_out[i] = vals[perm[i]];
        }
    }
    free(idx); free(perm1); free(tmp_keys); free(second_by1); free(perm);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Scan and select                                                           */
/* ------------------------------------------------------------------------ */

/* out[i] = in[0] + ... + in[i - 1] (exclusive) or + in[i] (inclusive), mod 2^32. */
void oracle_scan_u32(const uint32_t *in, uint32_t *out, uint64_t n, int inclusive)
{
    uint32_t running = 0;
    uint64_t i;
    for (i = 0; i < n; ++i) {
        uint32_t x = in[i];
        if (inclusive) {
            running += x;
            out[i] = running;
        } else {
            out[i] = running;
            running += x;
        }
    }
}

/* Comparison operators of oracle_select (the library uses the same numbering). */
#define ORACLE_OP_LT 0
#define ORACLE_OP_LE 1
#define ORACLE_OP_GT 2
#define ORACLE_OP_GE 3
#define ORACLE_OP_EQ 4
#define ORACLE_OP_NE 5

static int compare_u32(uint32_t a, uint32_t b, int op)
{
    switch (op) {
    case ORACLE_OP_LT: return a < b;
    case ORACLE_OP_LE: return a <= b;
    case ORACLE_OP_GT: return a > b;
    case ORACLE_OP_GE: return a >= b;
    case ORACLE_OP_EQ: return a == b;
    default: return a != b;
    }
}

static int compare_i32(int32_t a, int32_t b, int op)
{
    switch (op) {
    case ORACLE_OP_LT: return a < b;
    case ORACLE_OP_LE: return a <= b;
    case ORACLE_OP_GT: return a > b;
    case ORACLE_OP_GE: return a >= b;
    case ORACLE_OP_EQ: return a == b;
    default: return a != b;
    }
}

static int compare_f32(float a, float b, int op)
{
    switch (op) {
    case ORACLE_OP_LT: return a < b;
    case ORACLE_OP_LE: return a <= b;
    case ORACLE_OP_GT: return a > b;
    case ORACLE_OP_GE: return a >= b;
    case ORACLE_OP_EQ: return a == b;
    default: return a != b;
    }
}

/* Whether element i satisfies the predicate (key_type 0 = u32, 1 = i32, 2 = f32). */
static int selected(int key_type, int op, uint32_t threshold_bits, const uint32_t *in, uint64_t i)
{
    uint32_t u = in[i];
    if (key_type == ORACLE_KEY_U32)
        return compare_u32(u, threshold_bits, op);
    if (key_type == ORACLE_KEY_I32) {
        int32_t a, b;
        memcpy(&a, &u, 4);
        memcpy(&b, &threshold_bits, 4);
        return compare_i32(a, b, op);
    } else {
        float a, b;
        memcpy(&a, &u, 4);
        memcpy(&b, &threshold_bits, 4);
        return compare_f32(a, b, op);
    }
}

/*
 * Keeps the elements of in[n] (4-byte u32, i32 or f32 values, given as bit
 * patterns) with `value OP threshold`, in input order, at the front of out;
 * vals (optional) move alongside into vals_out.  partition == 0: out[k..n)
 * is left untouched; partition != 0: out[k..n) receives the rejected
 * elements in input order.  Returns k, or a negative code.
 */
int64_t oracle_select(int key_type, int op, uint32_t threshold_bits, const uint32_t *in,
                      const uint32_t *vals, uint32_t *out, uint32_t *vals_out, uint64_t n,
                      int partition)
{
    uint64_t i, k = 0, r = 0;

    if (key_type < ORACLE_KEY_U32 || key_type > ORACLE_KEY_F32 || op < 0 || op > ORACLE_OP_NE)
        return ORACLE_BAD_ARGS;
    if ((vals == NULL) != (vals_out == NULL))
        return ORACLE_BAD_ARGS;
    for (i = 0; i < n; ++i) {
        if (selected(key_type, op, threshold_bits, in, i)) {
            out[k] = in[i];
            if (vals)
                vals_out[k] = vals[i];
            k += 1;
        }
    }
    if (partition) {
        for (i = 0; i < n; ++i) {
            if (!selected(key_type, op, threshold_bits, in, i)) {
                out[k + r] = in[i];
                if (vals)
                    vals_out[k + r] = vals[i];
                r += 1;
            }
        }
    }
    return (int64_t)k;
}
