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
TileGrid tile_grid(uint32_t tiles, uint32_t resident);

// ---- radix sort ---------------------------------------------------------------

// Temp bytes for a sort of n keys with `passes` 8-bit passes.
size_t sort_temp_bytes(uint64_t n, bool pairs, int passes);

// Enqueues the whole sort (passes >= 1).  Arguments are already validated.
hipError_t launch_sort(const uint32_t* keys_in, uint32_t* keys_out, const uint32_t* vals_in,
                       uint32_t* vals_out, uint32_t n, int begin_bit, int end_bit, bool is_f32,
                       void* temp, hipStream_t stream);

// Zeroes `words` u32 starting at p (a fill kernel; no memset nodes).
hipError_t launch_fill_zero(uint32_t* p, uint64_t words, hipStream_t stream, int kernel_id);

// ---- compaction ----------------------------------------------------------------

size_t compact_temp_bytes(uint64_t n);
hipError_t launch_compact(const float* in, float* out, uint32_t* d_count, uint32_t n, void* temp,
                          hipStream_t stream);

// ---- bitonic tile -------------------------------------------------------------

hipError_t launch_bitonic(const uint32_t* keys_in, uint32_t* keys_out, uint32_t n, uint32_t tile,
                          int begin_bit, int end_bit, hipStream_t stream);

}  // namespace rs
