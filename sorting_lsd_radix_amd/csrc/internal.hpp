// internal.hpp -- host-side interfaces between the C ABI (rs_api.cpp) and the
// kernel launchers (radix.hip, compact.hip, bitonic.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "rs.h"

namespace rs {

// Measurement hook: brackets a launch with events when timing is enabled.
void timing_before(hipStream_t s, int kernel_id);
void timing_after(hipStream_t s);

// ---- persistent tile kernels ----------------------------------------------------

// Compute units of the current device (cached).
int device_cus();

// Launch shape of a persistent tile kernel: grid (at most `resident` blocks),
// block groups (one per XCD) and tiles per chunk (see next_chunked_tile).
struct TileGrid {
    uint32_t grid, groups, chunk_log2;
};
TileGrid tile_grid(uint32_t tiles, uint32_t resident, uint32_t max_chunk);
// Chunk caps.  Sort passes: 16 tiles (with 32 blocks per XCD each XCD then
// works on two chunks at once; 2^28 pair pass 0.871 -> 0.848 ms, keys-only
// sort 2.10 -> 2.00 ms against 32; chunks of 8, 12, 20 and 24 tiles were all
// slower than 16); also the select with values, whose 16384-element tiles
// make twice as many tiles.  Compaction, scan and the select without values
// (32768-element tiles): 32 (their 64-tile look-back steps do not gain from
// shorter chains, and 16 made the compaction and scan 3-8 % slower).
constexpr uint32_t kPassChunk = 16;
constexpr uint32_t kStreamChunk = 32;

// ---- radix sort ---------------------------------------------------------------

// Order transform of a sort's keys: each 32-bit word of a key is XOR-ed with
// pos_* when the key's sign bit (top bit of the word `hi`; a 32-bit key is a
// lone `hi` word) is clear and with neg_* when it is set.
struct KeyXform {
    uint32_t pos_hi, neg_hi;   // masks of the word holding the sign bit
    uint32_t pos_lo, neg_lo;   // masks of the low word of a 64-bit key
};

// What kind of keys a sort moves.
struct SortKind {
    bool key64;        // 8-byte keys (two words, low first)
    bool soa;          // two-key sort: low words and high words in two arrays
    bool transforms;   // xf is not the identity
    KeyXform xf;       // forward order transform
};

// Buffers of a sort (device pointers).  keys_in/keys_out hold n u32 keys, n
// 8-byte keys, or (soa) the n low words; hi_in/hi_out the n high words of a
// two-key sort.  vals_* are null for keys only.
struct SortIo {
    const uint32_t* keys_in;
    uint32_t* keys_out;
    const uint32_t* hi_in;
    uint32_t* hi_out;
    const uint32_t* vals_in;
    uint32_t* vals_out;
    uint32_t n;
};

// Temp bytes for a sort of n keys (depends only on n, pairs and the kind).
size_t sort_temp_bytes(uint64_t n, bool pairs, const SortKind& kind);

// Enqueues the whole sort (begin_bit < end_bit).  Arguments are already validated.
hipError_t launch_sort(const SortIo& io, const SortKind& kind, int begin_bit, int end_bit,
                       void* temp, hipStream_t stream);

// Zeroes d_counts[passes][256] and adds every pass's digit counts of the
// (transformed) keys of io into it.
hipError_t launch_digit_counts(const SortIo& io, const SortKind& kind, int begin_bit, int end_bit,
                               uint32_t* d_counts, hipStream_t stream);

// Zeroes `words` u32 starting at p (a fill kernel; no memset nodes).
hipError_t launch_fill_zero(uint32_t* p, uint64_t words, hipStream_t stream, int kernel_id);

// ---- compaction ----------------------------------------------------------------

size_t compact_temp_bytes(uint64_t n);
hipError_t launch_compact(const float* in, float* out, uint32_t* d_count, uint32_t n, void* temp,
                          hipStream_t stream);
// The same compaction with the library's static per-device scratch instead of
// a temp buffer (no allocation); fails if n needs more than that scratch.
size_t compact_static_scratch_bytes();
hipError_t launch_compact_static(const float* in, float* out, uint32_t* d_count, uint32_t n,
                                 hipStream_t stream);

// ---- scan, select, partition ------------------------------------------------------

size_t scan_temp_bytes(uint64_t n);
hipError_t launch_scan(const uint32_t* in, uint32_t* out, uint32_t n, bool inclusive, void* temp,
                       hipStream_t stream);
size_t select_temp_bytes(uint64_t n, bool pairs);
hipError_t launch_select(int key_type, int op, uint32_t threshold_bits, const uint32_t* in,
                         uint32_t* out, const uint32_t* vals_in, uint32_t* vals_out,
                         uint32_t* d_count, uint32_t n, bool partition, void* temp,
                         hipStream_t stream);

// ---- bitonic tile -------------------------------------------------------------

hipError_t launch_bitonic(const uint32_t* keys_in, uint32_t* keys_out, uint32_t n, uint32_t tile,
                          int begin_bit, int end_bit, hipStream_t stream);

}  // namespace rs
