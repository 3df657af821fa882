// device_common.hpp -- wave64 and memory-scope helpers shared by the gfx950
// kernels of the radix sort, the compaction and the bitonic tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"   // KeyXform

namespace rs {

constexpr int kWave = 64;          // CDNA wavefront width

// 16-byte vector of u32 (a clang vector type, usable with the nontemporal builtins)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRadixBits = 8;      // digit width of every sort pass
// Word 3 of a raw buffer descriptor on gfx9-family chips (32-bit data format).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kRadix = 1 << kRadixBits;

// Cross-tile state word: 2 status bits over a 30-bit count.
constexpr uint32_t kStateCountMask = 0x3FFFFFFFu;
constexpr uint32_t kStateAggregate = 1u << 30;   // the tile's own count is ready
constexpr uint32_t kStatePrefix = 2u << 30;      // the inclusive prefix is ready

__device__ __forceinline__ uint32_t lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ uint32_t count_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) {
    return __ballot(p);
}

// Loads/stores of tile states at device (agent) scope, so that tiles running
// on different XCDs, each behind its own L2, see each other's words.
__device__ __forceinline__ uint32_t load_state(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_state(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t fetch_add_agent(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tile scheduler of the persistent tile kernels (sort passes, compaction).
// Block b belongs to group b mod groups (groups = min(8, grid)); workgroups
// are dispatched round-robin over the 8 XCDs, so with 8 groups a group is the
// set of blocks on one XCD.  The tiles form chunks of 2^chunk_log2
// consecutive tiles, and group g owns the chunks g, g + groups, g + 2 groups,
// ...; its blocks take that sequence in order from one counter.  Neighbouring
// tiles thus run at the same time on one XCD, and the cache lines their
// output runs share are merged in that XCD's L2 before they reach memory.
// A block starts each tile it takes at once (the pipelined scan takes its
// next tile during the current one's look-back and starts it when the
// current one, a smaller tile, is done), every group has a block, and a
// group hands out its tiles in increasing order.  So the smallest unfinished
// tile is either running (every earlier tile is done, and its look-back
// ends), or taken by a block whose current tile is smaller, hence done, so
// that it starts at once, or not yet handed out, and then every tile its
// group has handed out is smaller, hence done, and a block of that group is
// free to take it: look-back always makes progress.
// Layout: sched[g] = tiles taken by group g.
__device__ __forceinline__ uint32_t next_chunked_tile(uint32_t* sched, uint32_t groups,
                                                      uint32_t chunk_log2, uint32_t group,
                                                      uint32_t tiles) {
    const uint32_t k = fetch_add_agent(&sched[group], 1u);
    const uint64_t chunk = static_cast<uint64_t>(k >> chunk_log2) * groups + group;
    const uint64_t t = (chunk << chunk_log2) | (k & ((1u << chunk_log2) - 1u));
    return t < tiles ? static_cast<uint32_t>(t) : tiles;
}

// Order transform of a sort's keys.  Every key type and direction maps a key
// to an unsigned pattern whose unsigned order is the wanted order by XOR-ing
// each 32-bit word with a mask chosen by the key's sign bit (the top bit of
// the word `hi`, which holds it; a 32-bit key is a lone `hi` word):
//   u32/u64  ascending: 0                 descending: all ones
//   i32/i64  ascending: sign bit flipped  descending: the other bits flipped
//   f32/f64  ascending: negative keys all bits flipped, others the sign bit;
//            descending: the complement of that.
// The inverse has the same form with the masks of the two signs swapped
// when the masks flip the sign bit.  (KeyXform is declared in internal.hpp.)
// Written as u ^ pos ^ (sign & (pos ^ neg)) so that each instruction reads at
// most one of the (uniform) masks: a CDNA vector instruction reads at most
// one scalar register.
__device__ __forceinline__ uint32_t xform32(uint32_t u, const KeyXform& x) {
    const uint32_t sign = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31);
    return (u ^ x.pos_hi) ^ (sign & (x.pos_hi ^ x.neg_hi));
}

__device__ __forceinline__ uint64_t xform64(uint64_t k, const KeyXform& x) {
    const bool neg = static_cast<int64_t>(k) < 0;
    const uint32_t mh = neg ? x.neg_hi : x.pos_hi;
    const uint32_t ml = neg ? x.neg_lo : x.pos_lo;
    return k ^ ((static_cast<uint64_t>(mh) << 32) | ml);
}

// The same sum with LDS-crossbar shuffles (six dependent ds_bpermute steps);
// slower on its own, but the one-sweep pair passes, which sit at the edge of
// their register budget, run faster with it than with the DPP form.
__device__ __forceinline__ uint32_t wave_inclusive_sum_shfl(uint32_t x) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        uint32_t y = __shfl_up(x, off, kWave);
        if (lane >= static_cast<uint32_t>(off)) x += y;
    }
    return x;
}

// Inclusive sum over the 64 lanes of a wave (all 64 lanes active), with DPP
// moves instead of LDS crossbar shuffles: a Hillis-Steele scan inside each row
// of 16 lanes (shifts by 1, 2, 4, 8, zeros shifted in), then row 15's total
// broadcast into rows 1 and 3 and lane 31's into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    constexpr int kRowShr = 0x110;      // row_shr:n is kRowShr + n
    constexpr int kRowBcast15 = 0x142;
    constexpr int kRowBcast31 = 0x143;
    x += __builtin_amdgcn_update_dpp(0u, x, kRowShr + 1, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, kRowShr + 2, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, kRowShr + 4, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, kRowShr + 8, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0u, x, kRowBcast15, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0u, x, kRowBcast31, 0xC, 0xF, false);
    return x;
}

}  // namespace rs
