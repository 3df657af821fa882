// rs_api.cpp -- the C ABI declared in include/rs.h: argument checks, temp
// sizing and dispatch to the kernel launchers.  Every check runs on the host
// before anything is enqueued, so an error return means nothing was launched.
#include <hip/hip_runtime_api.h>

#include <mutex>
#include <vector>

#include "internal.hpp"
#include "rs.h"

namespace rs {

namespace {

struct Range {
    uintptr_t lo, hi;
};

Range range_of(const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}

bool overlaps(const std::vector<Range>& rs) {
    for (size_t i = 0; i < rs.size(); ++i)
        for (size_t j = i + 1; j < rs.size(); ++j)
            if (rs[i].lo < rs[i].hi && rs[j].lo < rs[j].hi && rs[i].lo < rs[j].hi &&
                rs[j].lo < rs[i].hi)
                return true;
    return false;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bad_bits(int begin_bit, int end_bit) {
    return begin_bit < 0 || end_bit > 32 || begin_bit > end_bit;
}

// ---- measurement hook ------------------------------------------------------------
struct TimingRecord {
    int id;
    hipEvent_t start, stop;
};

std::mutex g_timing_mutex;
bool g_timing_enabled = false;
std::vector<TimingRecord> g_timing;

void clear_timing_locked() {
    for (auto& r : g_timing) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    g_timing.clear();
}

bool key_type_ok(int t) { return t >= RS_KEY_U32 && t <= RS_KEY_F64; }
bool is_key64(int t) { return t >= RS_KEY_U64; }

// Forward order transform of a key type and direction (see KeyXform).
KeyXform forward_xform(int key_type, bool descending) {
    KeyXform x{0u, 0u, 0u, 0u};
    switch (key_type) {
    case RS_KEY_I32:
    case RS_KEY_I64:
        x.pos_hi = x.neg_hi = 0x80000000u;   // flip the sign bit
        break;
    case RS_KEY_F32:
        x.pos_hi = 0x80000000u;              // non-negative: set the sign bit
        x.neg_hi = 0xFFFFFFFFu;              // negative: flip every bit
        break;
    case RS_KEY_F64:
        x.pos_hi = 0x80000000u;
        x.neg_hi = 0xFFFFFFFFu;
        x.neg_lo = 0xFFFFFFFFu;
        break;
    default:
        break;
    }
    if (descending) {   // the complement reverses the order
        x.pos_hi = ~x.pos_hi;
        x.neg_hi = ~x.neg_hi;
        x.pos_lo = ~x.pos_lo;
        x.neg_lo = ~x.neg_lo;
    }
    return x;
}

SortKind sort_kind(int key_type, bool descending, bool soa) {
    SortKind k{};
    k.key64 = is_key64(key_type) || soa;
    k.soa = soa;
    k.xf = forward_xform(key_type, descending);
    k.transforms = k.xf.pos_hi || k.xf.neg_hi || (k.key64 && (k.xf.pos_lo || k.xf.neg_lo));
    return k;
}

// One sort call: keys_in/keys_out are u32 or u64 arrays (soa: the minor /
// low-word arrays, with hi_in/hi_out the major arrays).
rs_status sort_common(int key_type, bool descending, bool soa, const void* keys_in, void* keys_out,
                      const uint32_t* hi_in, uint32_t* hi_out, const uint32_t* vals_in,
                      uint32_t* vals_out, uint64_t n, int begin_bit, int end_bit, void* d_temp,
                      size_t* temp_bytes, hipStream_t stream, bool pairs) {
    if (temp_bytes == nullptr) return RS_ERR_INVALID_VALUE;
    if (!key_type_ok(key_type)) return RS_ERR_INVALID_VALUE;
    const SortKind kind = sort_kind(key_type, descending, soa);
    const int key_bits = kind.key64 ? 64 : 32;
    if (begin_bit < 0 || end_bit > key_bits || begin_bit > end_bit) return RS_ERR_INVALID_VALUE;
    if (n >= (kind.key64 ? RS_MAX_N64 : RS_MAX_N)) return RS_ERR_UNSUPPORTED_SIZE;
    // a two-key sort's values are optional, so its size query (made without
    // pointers) always counts them
    const size_t need = sort_temp_bytes(n, pairs || soa, kind);
    if (d_temp == nullptr) {
        *temp_bytes = need;
        return RS_OK;
    }
    if (n == 0) return RS_OK;
    if (keys_in == nullptr || keys_out == nullptr) return RS_ERR_INVALID_VALUE;
    if (soa && (hi_in == nullptr || hi_out == nullptr)) return RS_ERR_INVALID_VALUE;
    if (pairs && (vals_in == nullptr || vals_out == nullptr)) return RS_ERR_INVALID_VALUE;
    if (!aligned16(keys_in) || !aligned16(keys_out) || !aligned16(d_temp)) return RS_ERR_MISALIGNED;
    if (soa && (!aligned16(hi_in) || !aligned16(hi_out))) return RS_ERR_MISALIGNED;
    if (pairs && (!aligned16(vals_in) || !aligned16(vals_out))) return RS_ERR_MISALIGNED;
    if (*temp_bytes < need) return RS_ERR_TEMP_TOO_SMALL;
    const size_t key_bytes = (kind.key64 && !soa) ? 8 : 4;
    std::vector<Range> rs{range_of(keys_in, n * key_bytes), range_of(keys_out, n * key_bytes),
                          range_of(d_temp, need)};
    if (soa) {
        rs.push_back(range_of(hi_in, n * 4));
        rs.push_back(range_of(hi_out, n * 4));
    }
    if (pairs) {
        rs.push_back(range_of(vals_in, n * 4));
        rs.push_back(range_of(vals_out, n * 4));
    }
    if (overlaps(rs)) return RS_ERR_OVERLAP;

    hipError_t e;
    if (begin_bit == end_bit) {
        // an empty ordering field: every key compares equal, the stable
        // order is the input order
        timing_before(stream, RS_KERNEL_COPY);
        e = hipMemcpyAsync(keys_out, keys_in, n * key_bytes, hipMemcpyDeviceToDevice, stream);
        if (e == hipSuccess && soa)
            e = hipMemcpyAsync(hi_out, hi_in, n * 4, hipMemcpyDeviceToDevice, stream);
        if (e == hipSuccess && pairs)
            e = hipMemcpyAsync(vals_out, vals_in, n * 4, hipMemcpyDeviceToDevice, stream);
        timing_after(stream);
    } else {
        SortIo io{static_cast<const uint32_t*>(keys_in), static_cast<uint32_t*>(keys_out), hi_in, hi_out,
                  pairs ? vals_in : nullptr, pairs ? vals_out : nullptr, static_cast<uint32_t>(n)};
        e = launch_sort(io, kind, begin_bit, end_bit, d_temp, stream);
    }
    return e == hipSuccess ? RS_OK : RS_ERR_HIP;
}

}  // namespace

void timing_before(hipStream_t s, int kernel_id) {
    std::lock_guard<std::mutex> lock(g_timing_mutex);
    if (!g_timing_enabled) return;
    TimingRecord r{kernel_id, nullptr, nullptr};
    // Timing-only events: no system-scope fence (cache writeback and
    // invalidation) when they are recorded, which would also slow the launch
    // that follows.
    if (hipEventCreateWithFlags(&r.start, hipEventDisableSystemFence) != hipSuccess) return;
    if (hipEventCreateWithFlags(&r.stop, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipEventDestroy(r.start);
        return;
    }
    (void)hipEventRecord(r.start, s);
    g_timing.push_back(r);
}

void timing_after(hipStream_t s) {
    std::lock_guard<std::mutex> lock(g_timing_mutex);
    if (!g_timing_enabled || g_timing.empty()) return;
    (void)hipEventRecord(g_timing.back().stop, s);
}

}  // namespace rs

extern "C" {

rs_status rs_sort_keys_u32(const uint32_t* keys_in, uint32_t* keys_out, uint64_t n, int begin_bit,
                           int end_bit, void* d_temp, size_t* temp_bytes, hipStream_t stream) {
    return rs::sort_common(RS_KEY_U32, false, false, keys_in, keys_out, nullptr, nullptr, nullptr,
                           nullptr, n, begin_bit, end_bit, d_temp, temp_bytes, stream, false);
}

rs_status rs_sort_pairs_u32(const uint32_t* keys_in, uint32_t* keys_out, const uint32_t* vals_in,
                            uint32_t* vals_out, uint64_t n, int begin_bit, int end_bit,
                            void* d_temp, size_t* temp_bytes, hipStream_t stream) {
    return rs::sort_common(RS_KEY_U32, false, false, keys_in, keys_out, nullptr, nullptr, vals_in,
                           vals_out, n, begin_bit, end_bit, d_temp, temp_bytes, stream, true);
}

rs_status rs_sort_pairs_f32(const float* keys_in, float* keys_out, const uint32_t* vals_in,
                            uint32_t* vals_out, uint64_t n, int begin_bit, int end_bit,
                            void* d_temp, size_t* temp_bytes, hipStream_t stream) {
    return rs::sort_common(RS_KEY_F32, false, false, keys_in, keys_out, nullptr, nullptr, vals_in,
                           vals_out, n, begin_bit, end_bit, d_temp, temp_bytes, stream, true);
}

rs_status rs_sort_keys(rs_key_type key_type, int descending, const void* keys_in, void* keys_out,
                       uint64_t n, int begin_bit, int end_bit, void* d_temp, size_t* temp_bytes,
                       hipStream_t stream) {
    return rs::sort_common(key_type, descending != 0, false, keys_in, keys_out, nullptr, nullptr,
                           nullptr, nullptr, n, begin_bit, end_bit, d_temp, temp_bytes, stream, false);
}

rs_status rs_sort_pairs(rs_key_type key_type, int descending, const void* keys_in, void* keys_out,
                        const uint32_t* vals_in, uint32_t* vals_out, uint64_t n, int begin_bit,
                        int end_bit, void* d_temp, size_t* temp_bytes, hipStream_t stream) {
    return rs::sort_common(key_type, descending != 0, false, keys_in, keys_out, nullptr, nullptr,
                           vals_in, vals_out, n, begin_bit, end_bit, d_temp, temp_bytes, stream, true);
}

rs_status rs_sort_two_keys_u32(const uint32_t* major_in, const uint32_t* minor_in,
                               uint32_t* major_out, uint32_t* minor_out, const uint32_t* vals_in,
                               uint32_t* vals_out, uint64_t n, void* d_temp, size_t* temp_bytes,
                               hipStream_t stream) {
    if ((vals_in == nullptr) != (vals_out == nullptr)) return RS_ERR_INVALID_VALUE;
    return rs::sort_common(RS_KEY_U64, false, true, minor_in, minor_out, major_in, major_out,
                           vals_in, vals_out, n, 0, 64, d_temp, temp_bytes, stream,
                           vals_in != nullptr);
}

rs_status rs_digit_counts(rs_key_type key_type, int descending, const void* keys, uint64_t n,
                          int begin_bit, int end_bit, uint32_t* d_counts, hipStream_t stream) {
    using namespace rs;
    if (!key_type_ok(key_type)) return RS_ERR_INVALID_VALUE;
    const SortKind kind = sort_kind(key_type, descending != 0, false);
    const int key_bits = kind.key64 ? 64 : 32;
    if (begin_bit < 0 || end_bit > key_bits || begin_bit > end_bit) return RS_ERR_INVALID_VALUE;
    if (n >= (kind.key64 ? RS_MAX_N64 : RS_MAX_N)) return RS_ERR_UNSUPPORTED_SIZE;
    if (begin_bit == end_bit) return RS_OK;   // no passes, nothing to count
    if (d_counts == nullptr || (n > 0 && keys == nullptr)) return RS_ERR_INVALID_VALUE;
    if ((reinterpret_cast<uintptr_t>(d_counts) & 3u) != 0) return RS_ERR_MISALIGNED;
    if (n > 0 && !aligned16(keys)) return RS_ERR_MISALIGNED;
    const size_t passes = static_cast<size_t>(end_bit - begin_bit + 7) / 8;
    if (n > 0 && overlaps({range_of(keys, n * (kind.key64 ? 8 : 4)), range_of(d_counts, passes * 1024)}))
        return RS_ERR_OVERLAP;
    SortIo io{static_cast<const uint32_t*>(keys), nullptr, nullptr, nullptr, nullptr, nullptr,
              static_cast<uint32_t>(n)};
    const hipError_t e = launch_digit_counts(io, kind, begin_bit, end_bit, d_counts, stream);
    return e == hipSuccess ? RS_OK : RS_ERR_HIP;
}

rs_status rs_compact_positive_f32(const float* in, float* out, uint32_t* d_count, uint64_t n,
                                  void* d_temp, size_t* temp_bytes, hipStream_t stream) {
    using namespace rs;
    if (temp_bytes == nullptr) return RS_ERR_INVALID_VALUE;
    if (n >= RS_MAX_N) return RS_ERR_UNSUPPORTED_SIZE;
    const size_t need = compact_temp_bytes(n);
    if (d_temp == nullptr) {
        *temp_bytes = need;
        return RS_OK;
    }
    if (d_count == nullptr) return RS_ERR_INVALID_VALUE;
    if (n > 0 && (in == nullptr || out == nullptr)) return RS_ERR_INVALID_VALUE;
    if ((reinterpret_cast<uintptr_t>(d_count) & 3u) != 0 || !aligned16(d_temp))
        return RS_ERR_MISALIGNED;
    if (n > 0 && (!aligned16(in) || !aligned16(out))) return RS_ERR_MISALIGNED;
    if (*temp_bytes < need) return RS_ERR_TEMP_TOO_SMALL;
    std::vector<Range> rs{range_of(d_count, 4), range_of(d_temp, need)};
    if (n > 0) {
        rs.push_back(range_of(in, n * 4));
        rs.push_back(range_of(out, n * 4));
    }
    if (overlaps(rs)) return RS_ERR_OVERLAP;
    hipError_t e;
    if (n == 0)
        e = launch_fill_zero(d_count, 1, stream, RS_KERNEL_COMPACT_INIT);
    else
        e = launch_compact(in, out, d_count, static_cast<uint32_t>(n), d_temp, stream);
    return e == hipSuccess ? RS_OK : RS_ERR_HIP;
}

static rs_status scan_common(const uint32_t* in, uint32_t* out, uint64_t n, void* d_temp,
                             size_t* temp_bytes, hipStream_t stream, bool inclusive) {
    using namespace rs;
    if (temp_bytes == nullptr) return RS_ERR_INVALID_VALUE;
    if (n >= RS_MAX_N) return RS_ERR_UNSUPPORTED_SIZE;
    const size_t need = scan_temp_bytes(n);
    if (d_temp == nullptr) {
        *temp_bytes = need;
        return RS_OK;
    }
    if (n == 0) return RS_OK;
    if (in == nullptr || out == nullptr) return RS_ERR_INVALID_VALUE;
    if (!aligned16(in) || !aligned16(out) || !aligned16(d_temp)) return RS_ERR_MISALIGNED;
    if (*temp_bytes < need) return RS_ERR_TEMP_TOO_SMALL;
    // in and out may be the same array; neither may overlap the temp, nor
    // each other partially
    if (in != out && overlaps({range_of(in, n * 4), range_of(out, n * 4)})) return RS_ERR_OVERLAP;
    if (overlaps({range_of(in, n * 4), range_of(d_temp, need)}) ||
        overlaps({range_of(out, n * 4), range_of(d_temp, need)}))
        return RS_ERR_OVERLAP;
    const hipError_t e = launch_scan(in, out, static_cast<uint32_t>(n), inclusive, d_temp, stream);
    return e == hipSuccess ? RS_OK : RS_ERR_HIP;
}

rs_status rs_exclusive_scan_u32(const uint32_t* in, uint32_t* out, uint64_t n, void* d_temp,
                                size_t* temp_bytes, hipStream_t stream) {
    return scan_common(in, out, n, d_temp, temp_bytes, stream, false);
}

rs_status rs_inclusive_scan_u32(const uint32_t* in, uint32_t* out, uint64_t n, void* d_temp,
                                size_t* temp_bytes, hipStream_t stream) {
    return scan_common(in, out, n, d_temp, temp_bytes, stream, true);
}

static rs_status select_common(int key_type, int op, uint32_t threshold_bits, const void* in,
                               void* out, const uint32_t* vals_in, uint32_t* vals_out,
                               uint32_t* d_count, uint64_t n, void* d_temp, size_t* temp_bytes,
                               hipStream_t stream, bool partition) {
    using namespace rs;
    if (temp_bytes == nullptr) return RS_ERR_INVALID_VALUE;
    if (key_type != RS_KEY_U32 && key_type != RS_KEY_I32 && key_type != RS_KEY_F32)
        return RS_ERR_INVALID_VALUE;
    if (op < RS_OP_LT || op > RS_OP_NE) return RS_ERR_INVALID_VALUE;
    if ((vals_in == nullptr) != (vals_out == nullptr)) return RS_ERR_INVALID_VALUE;
    if (n >= RS_MAX_N) return RS_ERR_UNSUPPORTED_SIZE;
    const bool pairs = vals_in != nullptr;
    const size_t need = select_temp_bytes(n, pairs);
    if (d_temp == nullptr) {
        *temp_bytes = need;
        return RS_OK;
    }
    if (d_count == nullptr) return RS_ERR_INVALID_VALUE;
    if (n > 0 && (in == nullptr || out == nullptr)) return RS_ERR_INVALID_VALUE;
    if ((reinterpret_cast<uintptr_t>(d_count) & 3u) != 0 || !aligned16(d_temp)) return RS_ERR_MISALIGNED;
    if (n > 0 && (!aligned16(in) || !aligned16(out))) return RS_ERR_MISALIGNED;
    if (pairs && n > 0 && (!aligned16(vals_in) || !aligned16(vals_out))) return RS_ERR_MISALIGNED;
    if (*temp_bytes < need) return RS_ERR_TEMP_TOO_SMALL;
    std::vector<Range> rs{range_of(d_count, 4), range_of(d_temp, need)};
    if (n > 0) {
        rs.push_back(range_of(in, n * 4));
        rs.push_back(range_of(out, n * 4));
        if (pairs) {
            rs.push_back(range_of(vals_in, n * 4));
            rs.push_back(range_of(vals_out, n * 4));
        }
    }
    if (overlaps(rs)) return RS_ERR_OVERLAP;
    hipError_t e;
    if (n == 0)
        e = launch_fill_zero(d_count, 1, stream, RS_KERNEL_SELECT_INIT);
    else
        e = launch_select(key_type, op, threshold_bits, static_cast<const uint32_t*>(in),
                          static_cast<uint32_t*>(out), vals_in, vals_out, d_count,
                          static_cast<uint32_t>(n), partition, d_temp, stream);
    return e == hipSuccess ? RS_OK : RS_ERR_HIP;
}

rs_status rs_select(rs_key_type key_type, rs_compare_op op, uint32_t threshold_bits, const void* in,
                    void* out, const uint32_t* vals_in, uint32_t* vals_out, uint32_t* d_count,
                    uint64_t n, void* d_temp, size_t* temp_bytes, hipStream_t stream) {
    return select_common(key_type, op, threshold_bits, in, out, vals_in, vals_out, d_count, n,
                         d_temp, temp_bytes, stream, false);
}

rs_status rs_partition(rs_key_type key_type, rs_compare_op op, uint32_t threshold_bits,
                       const void* in, void* out, const uint32_t* vals_in, uint32_t* vals_out,
                       uint32_t* d_count, uint64_t n, void* d_temp, size_t* temp_bytes,
                       hipStream_t stream) {
    return select_common(key_type, op, threshold_bits, in, out, vals_in, vals_out, d_count, n,
                         d_temp, temp_bytes, stream, true);
}

rs_status rs_compact_positive_f32_noalloc(const float* in, float* out, uint32_t* d_count,
                                          uint64_t n, hipStream_t stream) {
    using namespace rs;
    if (n >= RS_MAX_N || compact_temp_bytes(n) > compact_static_scratch_bytes())
        return RS_ERR_UNSUPPORTED_SIZE;
    if (d_count == nullptr) return RS_ERR_INVALID_VALUE;
    if (n > 0 && (in == nullptr || out == nullptr)) return RS_ERR_INVALID_VALUE;
    if ((reinterpret_cast<uintptr_t>(d_count) & 3u) != 0) return RS_ERR_MISALIGNED;
    if (n > 0 && (!aligned16(in) || !aligned16(out))) return RS_ERR_MISALIGNED;
    if (n > 0 && overlaps({range_of(d_count, 4), range_of(in, n * 4), range_of(out, n * 4)}))
        return RS_ERR_OVERLAP;
    hipError_t e;
    if (n == 0)
        e = launch_fill_zero(d_count, 1, stream, RS_KERNEL_COMPACT_INIT);
    else
        e = launch_compact_static(in, out, d_count, static_cast<uint32_t>(n), stream);
    return e == hipSuccess ? RS_OK : RS_ERR_HIP;
}

rs_status rs_bitonic_tile(const uint32_t* keys_in, uint32_t* keys_out, uint64_t n, uint32_t tile,
                          int begin_bit, int end_bit, hipStream_t stream) {
    using namespace rs;
    if (bad_bits(begin_bit, end_bit)) return RS_ERR_INVALID_VALUE;
    if (tile < 1 || tile > 1024) return RS_ERR_INVALID_VALUE;
    if (n >= RS_MAX_N) return RS_ERR_UNSUPPORTED_SIZE;
    if (n == 0) return RS_OK;
    if (keys_in == nullptr || keys_out == nullptr) return RS_ERR_INVALID_VALUE;
    if (!aligned16(keys_in) || !aligned16(keys_out)) return RS_ERR_MISALIGNED;
    if (overlaps({range_of(keys_in, n * 4), range_of(keys_out, n * 4)})) return RS_ERR_OVERLAP;
    const hipError_t e = launch_bitonic(keys_in, keys_out, static_cast<uint32_t>(n), tile,
                                        begin_bit, end_bit, stream);
    return e == hipSuccess ? RS_OK : RS_ERR_HIP;
}

const char* rs_status_string(rs_status status) {
    switch (status) {
        case RS_OK: return "RS_OK: success";
        case RS_ERR_INVALID_VALUE: return "RS_ERR_INVALID_VALUE: invalid argument";
        case RS_ERR_UNSUPPORTED_SIZE:
            return "RS_ERR_UNSUPPORTED_SIZE: n must be below 2^30 (2^29 for 64-bit and two-key sorts)";
        case RS_ERR_TEMP_TOO_SMALL: return "RS_ERR_TEMP_TOO_SMALL: temporary buffer too small";
        case RS_ERR_OVERLAP: return "RS_ERR_OVERLAP: buffers overlap";
        case RS_ERR_MISALIGNED: return "RS_ERR_MISALIGNED: pointer not 16-byte aligned";
        case RS_ERR_HIP: return "RS_ERR_HIP: HIP launch or runtime error";
    }
    return "unknown rs_status";
}

rs_status rs_timing_enable(int enable) {
    std::lock_guard<std::mutex> lock(rs::g_timing_mutex);
    if (enable) rs::clear_timing_locked();
    rs::g_timing_enabled = enable != 0;
    return RS_OK;
}

int rs_timing_collect(int* kernel_ids, float* ms, int cap) {
    std::lock_guard<std::mutex> lock(rs::g_timing_mutex);
    const int held = static_cast<int>(rs::g_timing.size());
    for (int i = 0; i < held; ++i) {
        const rs::TimingRecord& r = rs::g_timing[i];
        if (hipEventSynchronize(r.stop) != hipSuccess) return -1;
        float t = 0.f;
        if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return -1;
        if (i < cap) {
            if (kernel_ids) kernel_ids[i] = r.id;
            if (ms) ms[i] = t;
        }
    }
    return held;
}

}  // extern "C"
