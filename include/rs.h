/*
 * rs.h -- C ABI of the MI355X (gfx950) stable LSD radix sort library.
 *
 * Entry points:
 *   rs_sort_keys_u32        stable sort of 32-bit keys
 *   rs_sort_pairs_u32       stable sort of 32-bit keys with 32-bit values
 *   rs_sort_pairs_f32       stable sort of float keys (IEEE 754 total order)
 *                           with 32-bit values
 *   rs_sort_keys            stable sort of u32/i32/f32/u64/i64/f64 keys,
 *   rs_sort_pairs           ascending or descending, with or without values
 *   rs_sort_two_keys_u32    stable sort by (major, minor) u32 key pairs
 *   rs_digit_counts         every 8-bit pass's digit counts of typed keys
 *   rs_exclusive_scan_u32   prefix sums (exclusive / inclusive), mod 2^32
 *   rs_inclusive_scan_u32
 *   rs_select               keep x OP threshold in order (u32/i32/f32, values)
 *   rs_partition            kept in order, then rejected in order (stable split)
 *   rs_compact_positive_f32 keep x > 0 in order, zero-fill the rest, count
 *   rs_compact_positive_f32_noalloc  the same with static scratch (no temp)
 *   rs_bitonic_tile         sort each run of at most 1024 keys in LDS
 *   rs_status_string        text of a status code
 *
 * Common rules.
 *  - Every data pointer is a DEVICE pointer (hipMalloc or torch CUDA tensor
 *    storage) unless stated.  Inputs are read-only and never modified;
 *    outputs are fully written when the call returns RS_OK.  Input, output
 *    and temporary ranges must not overlap each other (RS_ERR_OVERLAP).
 *  - Every data pointer must be 16-byte aligned (RS_ERR_MISALIGNED); the
 *    kernels use 16-byte vector loads where the layout allows.
 *  - Work is enqueued on `stream` (NULL = the null stream) and the call
 *    returns without synchronising; the caller synchronises.
 *  - All argument checks happen on the host before anything is enqueued: a
 *    call that returns an error has launched nothing and written nothing.
 *    RS_ERR_HIP reports a failed launch (hipGetLastError) after enqueueing.
 *  - Temporary storage follows the two-call query idiom the textbook chapter
 *    shows for library radix sorts ("第10章 并行模式：排序", 10.8 Thrust/CUB):
 *    with d_temp == NULL the required size is written to *temp_bytes and
 *    nothing is launched; otherwise *temp_bytes must be at least that size.
 *    The caller owns the temp buffer and need not initialise it.  The size
 *    depends only on n (and on whether values are sorted).
 *  - The library keeps no mutable state between calls (apart from the
 *    opt-in timing hook below): concurrent calls on different streams with
 *    different temp buffers are independent.  Launch grids are sized once
 *    per process from the device current at the first call; a grid only
 *    affects speed, never results.
 *  - n < 2^30 (RS_ERR_UNSUPPORTED_SIZE otherwise): cross-tile prefix states
 *    hold 30-bit counts beside 2 status bits.  Sorts of 64-bit keys and
 *    two-key sorts take n < 2^29, which keeps every byte offset into an
 *    array of 8-byte keys below 2^32.
 *  - Scheduling assumption of the persistent kernels (sort passes,
 *    compaction, scan, select and partition): their grid never exceeds the
 *    number of blocks that fit on the device at once, tiles are handed out
 *    in increasing order per group of blocks (one group per XCD), and a tile
 *    waits only on tiles with smaller ids.  Progress needs at least one block
 *    of every group (up to 8) to become resident.  That holds on an
 *    otherwise idle device and beside kernels that finish without waiting
 *    on this one (they only delay blocks that have not started; blocks that
 *    started keep running).  Two such kernels started at the same time on
 *    different streams of one device, each holding every CU of some XCD
 *    while waiting for the other to free it, or a device partitioned so
 *    that a kernel's blocks could be preempted indefinitely, are outside
 *    this contract.
 */
#ifndef RS_H
#define RS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rs_status {
    RS_OK = 0,
    RS_ERR_INVALID_VALUE = 1,    /* null pointer with n > 0, bad bit range, bad tile */
    RS_ERR_UNSUPPORTED_SIZE = 2, /* n >= 2^30 (2^29 for 8-byte and two-key sorts) */
    RS_ERR_TEMP_TOO_SMALL = 3,   /* *temp_bytes below the queried size */
    RS_ERR_OVERLAP = 4,          /* two of the buffers overlap */
    RS_ERR_MISALIGNED = 5,       /* a pointer is not 16-byte aligned */
    RS_ERR_HIP = 6               /* a HIP launch or runtime call failed */
} rs_status;

#define RS_MAX_N ((uint64_t)1 << 30)
#define RS_MAX_N64 ((uint64_t)1 << 29)

/*
 * Key types of rs_sort_keys / rs_sort_pairs / rs_digit_counts.  Keys are
 * arrays of 4-byte (u32, i32, f32) or 8-byte (u64, i64, f64) elements.
 * Each key maps to an unsigned order pattern of the same width whose
 * unsigned order is the type's order: unsigned keys as they are, signed keys
 * with the sign bit flipped (value + 2^(w-1)), floats with every bit of a
 * negative pattern flipped and the sign bit of any other set, which is IEEE
 * 754 totalOrder (-NaN < -inf < ... < -0.0 < +0.0 < ... < +inf < +NaN,
 * subnormals kept); a descending sort uses the complement of the pattern
 * ("第10章 并行模式：排序 - GPU上的排序", 八、习题: the exercises on
 * descending sorts, float preprocessing and 64-bit keys).  Equal keys keep
 * their input order in both directions.
 */
typedef enum rs_key_type {
    RS_KEY_U32 = 0,
    RS_KEY_I32 = 1,
    RS_KEY_F32 = 2,
    RS_KEY_U64 = 3,
    RS_KEY_I64 = 4,
    RS_KEY_F64 = 5
} rs_key_type;

/*
 * Stable LSD radix sort of keys by bits [begin_bit, end_bit).
 *
 * Defines: the least-significant-digit sort as one stable counting sort per
 * 8-bit digit, lowest digit first ("CUDA 算子笔记 3", sections Radix Sort
 * and 一次处理多位; "第10章 并行模式：排序", 10.3 Radix Sort算法; "WebGPU
 * Unleashed", 4.1 래딕스 정렬, on why each digit pass must be stable).
 *
 * keys_in  [n] u32, read only.          keys_out [n] u32, written.
 * n        element count, 0 <= n < 2^30.
 * begin_bit, end_bit: 0 <= begin_bit <= end_bit <= 32.  The ordering field
 *          is (key >> begin_bit) & (2^(end_bit-begin_bit) - 1); bits outside
 *          it are carried but ignored; equal fields keep input order.
 *          begin_bit == end_bit copies the input.
 * d_temp, temp_bytes: see the query idiom above.
 * Up to 16384 keys the whole sort runs in one workgroup in LDS (one launch,
 * the temp buffer is not touched).  Above, a clear launch and one digit-count
 * launch come first; then, up to 3 * 2^20 keys with two or more digit passes,
 * the hybrid path ("第10章 并行模式：排序", 10.5, 策略2 混合排序): a pass on
 * the top digit, then one workgroup per bucket sorting the lower digits in
 * LDS, or, when a bucket holds more than 16384 keys, every LSD pass in one
 * launch (the device decides; both launches are always enqueued); above
 * that, one launch per digit pass.
 */
rs_status rs_sort_keys_u32(const uint32_t *keys_in, uint32_t *keys_out, uint64_t n,
                           int begin_bit, int end_bit, void *d_temp, size_t *temp_bytes,
                           hipStream_t stream);

/*
 * Stable LSD radix sort of (key, value) pairs by key bits [begin_bit,
 * end_bit); values move with their keys ("第10章 并行模式：排序", 10.6
 * Key-Value排序).  vals_in [n] u32 read only, vals_out [n] u32 written; the
 * other arguments are as for rs_sort_keys_u32.
 */
rs_status rs_sort_pairs_u32(const uint32_t *keys_in, uint32_t *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, uint64_t n,
                            int begin_bit, int end_bit, void *d_temp, size_t *temp_bytes,
                            hipStream_t stream);

/*
 * Stable sort of float keys with u32 values.  Keys are ordered through the
 * order-preserving transform of their bit patterns (negative patterns
 * inverted, the sign bit of the others set), which the textbook's float
 * exercise asks for ("第10章 并行模式：排序", 八、习题); the result is IEEE
 * 754 totalOrder: -NaN < -inf < ... < -0.0 < +0.0 < ... < +inf < +NaN,
 * subnormals kept.  No float arithmetic touches a key.  [begin_bit,
 * end_bit) selects bits of the transformed pattern; (0, 32) is the full
 * order.  keys_out holds the original bit patterns in sorted order.
 */
rs_status rs_sort_pairs_f32(const float *keys_in, float *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, uint64_t n,
                            int begin_bit, int end_bit, void *d_temp, size_t *temp_bytes,
                            hipStream_t stream);

/*
 * Stable LSD radix sort of typed keys (see rs_key_type), ascending or (with
 * descending != 0) descending, by bits [begin_bit, end_bit) of the keys'
 * order patterns, 0 <= begin_bit <= end_bit <= 32 (4-byte keys) or 64
 * (8-byte keys); (0, 32) or (0, 64) is the full order.  With 8-bit digits a
 * 64-bit key takes eight passes ("第10章 并行模式：排序", 八、习题, the
 * iteration-count exercise).  keys_in [n] read only, keys_out [n] written
 * (the original bit patterns in sorted order).  n < 2^30 for 4-byte keys,
 * n < 2^29 for 8-byte keys.  Temp, streams and errors as for
 * rs_sort_keys_u32 (RS_ERR_INVALID_VALUE also for an unknown key type).
 * Up to 16384 4-byte keys the sort runs in one workgroup; 8-byte keys always
 * take the digit-count launch and one launch per pass.
 */
rs_status rs_sort_keys(rs_key_type key_type, int descending, const void *keys_in, void *keys_out,
                       uint64_t n, int begin_bit, int end_bit, void *d_temp, size_t *temp_bytes,
                       hipStream_t stream);

/*
 * As rs_sort_keys, with u32 values that move with their keys (vals_in [n]
 * read only, vals_out [n] written).
 */
rs_status rs_sort_pairs(rs_key_type key_type, int descending, const void *keys_in, void *keys_out,
                        const uint32_t *vals_in, uint32_t *vals_out, uint64_t n, int begin_bit,
                        int end_bit, void *d_temp, size_t *temp_bytes, hipStream_t stream);

/*
 * Multi-key sort ("第10章 并行模式：排序", 八、习题, the exercise on sorting
 * by one key and then stably by another): orders n elements by major key,
 * then by minor key, then by input position.  It is one stable LSD sort of
 * the 64-bit key major * 2^32 + minor, read from and written back to two
 * u32 arrays (the passes in between keep 8-byte keys in temp).  The result
 * equals a stable sort by the minor key followed by a stable sort by the
 * major key.  major_in/minor_in [n] read only, major_out/minor_out [n]
 * written; vals_in/vals_out [n] u32, or both NULL for keys only.  n < 2^29.
 * The temp size (query with d_temp == NULL) depends only on n and always
 * allows for values.  Temp, streams and errors as for rs_sort_keys_u32.
 */
rs_status rs_sort_two_keys_u32(const uint32_t *major_in, const uint32_t *minor_in,
                               uint32_t *major_out, uint32_t *minor_out, const uint32_t *vals_in,
                               uint32_t *vals_out, uint64_t n, void *d_temp, size_t *temp_bytes,
                               hipStream_t stream);

/*
 * Digit counts of every 8-bit pass over bits [begin_bit, end_bit) of the
 * order patterns of typed keys, in one read of the keys (the first kernel of
 * the multi-bit radix sort, "CUDA 算子笔记 3", section 一次处理多位):
 * d_counts[p * 256 + d] = number of keys whose pass-p digit is d, pass p
 * covering bits [begin_bit + 8p, min(begin_bit + 8p + 8, end_bit)).
 * d_counts: ceil((end_bit - begin_bit) / 8) * 256 u32 in device memory,
 * 4-byte aligned, overwritten (zeros when n == 0; untouched when
 * begin_bit == end_bit).  keys [n], 16-byte aligned, read only.  These are
 * the counts every sort call computes first.  Errors as for rs_sort_keys.
 */
rs_status rs_digit_counts(rs_key_type key_type, int descending, const void *keys, uint64_t n,
                          int begin_bit, int end_bit, uint32_t *d_counts, hipStream_t stream);

/*
 * Prefix sums of u32 elements in one pass over the data, by a decoupled
 * look-back over per-tile sums ("CUDA 算子笔记 3", the scan methods of the
 * Stream Compaction section: each element read and written once):
 * exclusive out[i] = in[0] + ... + in[i-1], inclusive out[i] = in[0] + ... +
 * in[i], both modulo 2^32.  in [n] read only, out [n] written (in == out is
 * allowed: every tile reads its elements before any of its outputs are
 * stored, and no tile reads another's elements).  n < 2^30.  Temp with the
 * query idiom (d_temp == NULL writes the size).  Errors as for the sorts.
 */
rs_status rs_exclusive_scan_u32(const uint32_t *in, uint32_t *out, uint64_t n, void *d_temp,
                                size_t *temp_bytes, hipStream_t stream);
rs_status rs_inclusive_scan_u32(const uint32_t *in, uint32_t *out, uint64_t n, void *d_temp,
                                size_t *temp_bytes, hipStream_t stream);

/* Comparison of rs_select / rs_partition: element OP threshold. */
typedef enum rs_compare_op {
    RS_OP_LT = 0,
    RS_OP_LE = 1,
    RS_OP_GT = 2,
    RS_OP_GE = 3,
    RS_OP_EQ = 4,
    RS_OP_NE = 5
} rs_compare_op;

/*
 * Select: out[0..k) = the elements x of in with `x OP threshold`, in input
 * order, *d_count = k; out[k..n) is not written ("CUDA 算子笔记 3", Stream
 * Compaction: predicate, scan of the predicate, scatter -- here with any
 * comparison).  key_type: RS_KEY_U32, RS_KEY_I32 or RS_KEY_F32 (4-byte
 * elements compared as unsigned, signed or IEEE float values; a NaN compares
 * unequal to everything and fails every other comparison).
 * threshold_bits: the bit pattern of the threshold in that type.
 * vals_in/vals_out: optional u32 values moved with the kept elements (both
 * NULL for none).  in [n] and vals_in read only.  d_count: one u32 in device
 * memory.  n < 2^30.  Temp with the query idiom (the size depends on n and
 * on whether values are given).  Errors as for rs_compact_positive_f32.
 */
rs_status rs_select(rs_key_type key_type, rs_compare_op op, uint32_t threshold_bits, const void *in,
                    void *out, const uint32_t *vals_in, uint32_t *vals_out, uint32_t *d_count,
                    uint64_t n, void *d_temp, size_t *temp_bytes, hipStream_t stream);

/*
 * Stable partition: out[0..k) = the elements with `x OP threshold` in input
 * order, out[k..n) = the others in input order, *d_count = k (the one-bit
 * split that a radix-sort pass performs per bit, "CUDA 算子笔记 3", Radix
 * Sort).  A first launch counts the kept elements, so each tile can place its
 * rejected run at k + the rejected elements of earlier tiles.  Arguments as
 * for rs_select; every output element is written.
 */
rs_status rs_partition(rs_key_type key_type, rs_compare_op op, uint32_t threshold_bits,
                       const void *in, void *out, const uint32_t *vals_in, uint32_t *vals_out,
                       uint32_t *d_count, uint64_t n, void *d_temp, size_t *temp_bytes,
                       hipStream_t stream);

/*
 * Stream compaction: out[0..k) = the inputs with x > 0.0f in input order,
 * out[k..n) = +0.0f, *d_count = k ("CUDA 算子笔记 3", section Stream
 * Compaction and its decoupled look-back method).  The predicate is taken
 * on the bit pattern, so positive subnormals are kept and NaNs are not.
 *
 * in [n] f32 read only; out [n] f32 written; d_count: one u32 in device
 * memory, written (0 when n == 0).  d_temp/temp_bytes: query idiom.
 */
rs_status rs_compact_positive_f32(const float *in, float *out, uint32_t *d_count, uint64_t n,
                                  void *d_temp, size_t *temp_bytes, hipStream_t stream);

/*
 * rs_compact_positive_f32 without a temp buffer, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It runs the same kernels with the
 * library's static scratch: a file-scope device array of 131,328 bytes (the
 * tile counters and one state word per 32768-element tile for every n <
 * 2^30), which each device the library runs on holds until the process ends.
 * It calls no allocating routine.  n >= 2^30 returns RS_ERR_UNSUPPORTED_SIZE.
 * The first call on a device looks up that device's copy of the array.
 * Every call on one device shares its scratch, clearing it on the stream
 * before use: calls that overlap on one device (different streams or host
 * threads without ordering between them) race and give wrong results.
 * Other arguments, results and errors as for rs_compact_positive_f32.
 */
rs_status rs_compact_positive_f32_noalloc(const float *in, float *out, uint32_t *d_count, uint64_t n,
                                          hipStream_t stream);

/*
 * Each run keys[s .. min(s + tile, n)), s = 0, tile, 2 tile, ..., is sorted
 * on its own in LDS by a bitonic network ("gpu排序__gpu", the in-block
 * bitonic sort of up to 1024 elements; "第10章 并行模式：排序", 10.2 Bitonic
 * Sort) comparing (field, position) so that the result is the stable order.
 * tile in [1, 1024]; begin_bit/end_bit as for rs_sort_keys_u32.  No temp.
 */
rs_status rs_bitonic_tile(const uint32_t *keys_in, uint32_t *keys_out, uint64_t n,
                          uint32_t tile, int begin_bit, int end_bit, hipStream_t stream);

/* Static text for a status code (never NULL). */
const char *rs_status_string(rs_status status);

/*
 * Measurement hook.  When enabled, the library brackets every kernel it
 * launches with hipEventRecord on the call's stream and keeps the events;
 * rs_timing_collect waits for them and returns per-launch durations.  It is
 * process-wide and not meant for concurrent use; off by default.  The events
 * are created with hipEventDisableSystemFence (timing only: recording them
 * writes back and invalidates no caches), yet each still adds about 2 us
 * between launches, so time throughput with the hook off or on few calls.
 *
 * rs_timing_enable(1) clears previous records and starts recording;
 * rs_timing_enable(0) stops.  rs_timing_collect writes up to `cap` records
 * (kernel id, milliseconds) in launch order and returns the number of
 * records held (which may exceed cap), or -1 on a HIP error.
 */
typedef enum rs_kernel_id {
    RS_KERNEL_UPSWEEP = 0,      /* all passes' digit counts, one read of the keys */
    RS_KERNEL_ONESWEEP = 1,     /* one digit pass: rank, look-back, scatter */
    RS_KERNEL_SORT_INIT = 2,    /* clears the sort's counters and states */
    RS_KERNEL_COMPACT_INIT = 3, /* clears the compaction's counter and states */
    RS_KERNEL_COMPACT = 4,      /* single-pass compaction */
    RS_KERNEL_BITONIC = 5,      /* LDS bitonic tiles */
    RS_KERNEL_COPY = 6,         /* device copy for an empty bit range */
    RS_KERNEL_TILE_SORT = 7,    /* whole sort of n <= 16384 keys in one block */
    RS_KERNEL_BUCKET_SORT = 8,  /* hybrid sort: each top-digit bucket sorted in LDS */
    RS_KERNEL_SCAN_INIT = 9,    /* clears the scan's counters and states */
    RS_KERNEL_SCAN = 10,        /* single-pass prefix sum */
    RS_KERNEL_SELECT_INIT = 11, /* clears select/partition counters and states */
    RS_KERNEL_SELECT_COUNT = 12,/* partition: kept elements of the whole input */
    RS_KERNEL_SELECT = 13       /* single-pass select / partition */
} rs_kernel_id;

rs_status rs_timing_enable(int enable);
int rs_timing_collect(int *kernel_ids, float *ms, int cap);

#ifdef __cplusplus
}
#endif

#endif /* RS_H */
