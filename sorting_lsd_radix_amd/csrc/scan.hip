// scan.hip -- device-wide prefix sum and select / partition for gfx950.
//
// The building blocks the sort and the compaction are made of, as calls of
// their own ("CUDA 算子笔记 3": the scan methods of the Stream Compaction
// section -- scan-then-propagate, reduce-then-scan and the decoupled
// look-back, which reads and writes each element once -- and the one-bit
// split of its Radix Sort section, a stable partition by a predicate;
// "WebGPU Unleashed", 4.1: a digit pass as a prefix sum of occurrences).
//
//  * rs_exclusive_scan_u32 / rs_inclusive_scan_u32: one pass; each tile of
//    32768 elements publishes its sum, then looks back over earlier tiles'
//    published sums until it meets an inclusive prefix (64-bit state words:
//    two status bits above a 32-bit sum, so sums wrap modulo 2^32 like the
//    elements');
//  * rs_select: the compaction with any of six comparisons against a
//    threshold (u32, i32 or f32 elements) and optional u32 values;
//  * rs_partition: the stable split: kept elements in order, then the
//    rejected ones in order after them.  A count launch first totals the kept
//    elements, so the rejected run of a tile starts at total + rejected
//    elements of earlier tiles.
//
// All three use the persistent XCD-chunked tile scheduler of the sort passes
// and wave-0 look-back over 64 earlier tiles per step, as the compaction.
#include "device_common.hpp"
#include "internal.hpp"

namespace rs {

namespace {

constexpr int kScanBlock = 1024;
constexpr int kScanQuads = 8;                                   // 16-byte vectors per thread
constexpr int kScanTile = kScanBlock * kScanQuads * 4;          // 32768 elements
constexpr uint64_t kScanAggregate = 1ull << 32;                 // the tile's own sum is ready
constexpr uint64_t kScanPrefix = 2ull << 32;                    // the inclusive prefix is ready

__device__ __forceinline__ uint64_t load_state64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_state64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of all tiles before `tile` (modulo 2^32): wave 0 reads the states of
// 64 earlier tiles per step, waits until every one up to the nearest
// published prefix is ready, adds them and stops at that prefix; tile 0
// publishes its prefix at once, so the walk ends there at the latest.
__device__ uint32_t scan_look_back(uint64_t* states, uint32_t tile, uint32_t lane) {
    uint32_t excl = 0;
    int32_t newest = static_cast<int32_t>(tile) - 1;
    for (;;) {
        const int32_t t = newest - static_cast<int32_t>(lane);
        uint64_t st = (t >= 0) ? load_state64(&states[t]) : kScanPrefix;
        for (;;) {
            const uint64_t not_ready = ballot((st >> 32) == 0u);
            const uint64_t prefix = ballot((st & kScanPrefix) != 0u);
            const uint64_t upto = prefix ? (prefix & (~prefix + 1ull)) * 2ull - 1ull : ~0ull;
            if ((not_ready & upto) == 0ull) break;
            __builtin_amdgcn_s_sleep(1);
            if ((st >> 32) == 0u && t >= 0) st = load_state64(&states[t]);
        }
        const uint64_t prefix = ballot((st & kScanPrefix) != 0u);
        const uint64_t upto = prefix ? (prefix & (~prefix + 1ull)) * 2ull - 1ull : ~0ull;
        const uint32_t mine = ((upto >> lane) & 1ull) ? static_cast<uint32_t>(st) : 0u;
        excl += __shfl(wave_inclusive_sum(mine), kWave - 1, kWave);
        if (prefix) break;
        newest -= kWave;
    }
    return excl;
}

// ---------------------------------------------------------------------------
// Prefix sum.  Thread t of a tile holds the 16-byte vectors q * 1024 + t,
// q = 0..7, i.e. vector row q of the tile is the 4096 elements q*4096 ..;
// element order within the tile is (row, thread, element).  Each wave scans
// its share of every row; wave 0 then scans the 128 (row, wave) totals in
// that order, publishes the tile's sum, looks back and hands every wave its
// offsets.
//
// Software-pipelined over a block's tiles: the next tile is taken during the
// look-back and its loads are issued before this tile's stores.  One
// counter tracks a wave's loads and stores together and in order, so a
// wait for loads issued after the stores would also wait for the stores to
// drain; issued before them, the next tile's data arrives while the stores
// are still in flight.  The per-tile LDS words are double-buffered by the
// parity of the block's tile count, so a wave that runs ahead to the next
// tile never overwrites words a slower wave still reads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void scan_load_tile(__amdgpu_buffer_rsrc_t in_rsrc, uint32_t base, bool full,
                                               uint32_t tid, uint32_t (&x)[kScanQuads][4]) {
#pragma unroll
    for (int q = 0; q < kScanQuads; ++q) {
        const uint32_t e0 = base + (q * kScanBlock + tid) * 4;
        if (full) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(in_rsrc, static_cast<int>(e0 * 4u), 0, 2);
            x[q][0] = v.x;
            x[q][1] = v.y;
            x[q][2] = v.z;
            x[q][3] = v.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)   // past n: 0 (the descriptor returns 0 there)
                x[q][e] = __builtin_amdgcn_raw_buffer_load_b32(in_rsrc, static_cast<int>((e0 + e) * 4u), 0, 2);
        }
    }
}

template <bool INCLUSIVE>
__global__ __launch_bounds__(kScanBlock) void scan_kernel(const uint32_t* __restrict__ in,
                                                          uint32_t* __restrict__ out, uint32_t n,
                                                          uint32_t tiles, uint64_t* __restrict__ states,
                                                          uint32_t* __restrict__ sched, uint32_t groups,
                                                          uint32_t chunk_log2) {
    constexpr int WAVES = kScanBlock / kWave;
    constexpr int PARTS = kScanQuads * WAVES;          // (row, wave) totals, row-major
    static_assert(PARTS % kWave == 0, "wave 0 scans the totals in lane-sized groups");
    __shared__ uint32_t s_part[2][PARTS];              // totals, then exclusive offsets in the tile
    __shared__ uint32_t s_tile[2];                     // [1]: the first tile; [it & 1]: the tile taken in iteration it
    __shared__ uint32_t s_excl[2];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;
    const uint32_t group = blockIdx.x % groups;
    const __amdgpu_buffer_rsrc_t in_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(in), 0, static_cast<int>(n * 4u), kBufferWord3);
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(out, 0, static_cast<int>(n * 4u), kBufferWord3);

    if (tid == 0) s_tile[1] = next_chunked_tile(sched, groups, chunk_log2, group, tiles);
    __syncthreads();
    uint32_t tile = s_tile[1];
    if (tile >= tiles) return;   // uniform
    uint32_t x[kScanQuads][4];
    scan_load_tile(in_rsrc, tile * kScanTile, n - tile * kScanTile >= static_cast<uint32_t>(kScanTile), tid, x);

    for (uint32_t it = 0;; ++it) {
        const uint32_t buf = it & 1u;
        const uint32_t base = tile * kScanTile;
        const bool full = n - base >= static_cast<uint32_t>(kScanTile);

        // inclusive sums inside each vector, the vectors' totals scanned over the wave
        uint32_t wave_excl[kScanQuads];
#pragma unroll
        for (int q = 0; q < kScanQuads; ++q) {
            x[q][1] += x[q][0];
            x[q][2] += x[q][1];
            x[q][3] += x[q][2];
            const uint32_t inc = wave_inclusive_sum(x[q][3]);
            wave_excl[q] = inc - x[q][3];
            if (lane == kWave - 1) s_part[buf][q * WAVES + wave] = inc;
        }
        __syncthreads();

        if (wave == 0) {
            // the next tile, in flight during the scan of the totals and the look-back
            const uint32_t next = (tid == 0) ? next_chunked_tile(sched, groups, chunk_log2, group, tiles) : 0u;
            // exclusive offsets of the (row, wave) parts inside the tile
            uint32_t carry = 0;
#pragma unroll
            for (int g = 0; g < PARTS / kWave; ++g) {
                const uint32_t v = s_part[buf][g * kWave + lane];
                const uint32_t inc = wave_inclusive_sum(v);
                s_part[buf][g * kWave + lane] = carry + inc - v;
                carry += __shfl(inc, kWave - 1, kWave);
            }
            const uint32_t tile_total = carry;
            uint32_t excl = 0;
            if (lane == 0)
                store_state64(&states[tile], (tile == 0 ? kScanPrefix : kScanAggregate) | tile_total);
            if (tile > 0) {
                excl = scan_look_back(states, tile, lane);
                if (lane == 0) store_state64(&states[tile], kScanPrefix | static_cast<uint32_t>(excl + tile_total));
            }
            if (lane == 0) {
                s_excl[buf] = excl;
                s_tile[buf] = next;
            }
        }
        __syncthreads();
        const uint32_t excl = s_excl[buf];
        const uint32_t next = s_tile[buf];

        // this tile's sums stay in x_out; x takes the next tile's loads
        uint32_t x_out[kScanQuads][4];
#pragma unroll
        for (int q = 0; q < kScanQuads; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) x_out[q][e] = x[q][e];
        if (next < tiles)   // uniform
            scan_load_tile(in_rsrc, next * kScanTile, n - next * kScanTile >= static_cast<uint32_t>(kScanTile), tid, x);

#pragma unroll
        for (int q = 0; q < kScanQuads; ++q) {
            const uint32_t off = excl + s_part[buf][q * WAVES + wave] + wave_excl[q];
            u32x4 v;
            // x_out[q][e] holds the inclusive sum of the vector's elements 0..e
            if (INCLUSIVE) {
                v.x = off + x_out[q][0];
                v.y = off + x_out[q][1];
                v.z = off + x_out[q][2];
                v.w = off + x_out[q][3];
            } else {
                v.x = off;
                v.y = off + x_out[q][0];
                v.z = off + x_out[q][1];
                v.w = off + x_out[q][2];
            }
            const uint32_t e0 = base + (q * kScanBlock + tid) * 4;
            if (full) {
                __builtin_amdgcn_raw_buffer_store_b128(v, out_rsrc, static_cast<int>(e0 * 4u), 0, 0);
            } else {   // stores past n are dropped by the descriptor
                __builtin_amdgcn_raw_buffer_store_b32(v.x, out_rsrc, static_cast<int>(e0 * 4u), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(v.y, out_rsrc, static_cast<int>((e0 + 1) * 4u), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(v.z, out_rsrc, static_cast<int>((e0 + 2) * 4u), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(v.w, out_rsrc, static_cast<int>((e0 + 3) * 4u), 0, 0);
            }
        }
        if (next >= tiles) break;   // uniform
        tile = next;
    }
}

// ---------------------------------------------------------------------------
// Select / partition.
// ---------------------------------------------------------------------------

// The predicate `x OP threshold` as three comparisons combined by masks:
// keep = (lt & want_lt) | (eq & want_eq) | (gt & want_gt) | (unordered &
// want_unordered), the masks set from OP on the host.  Floats compare as
// IEEE values (a NaN is unordered with everything: only != keeps it).
struct Predicate {
    uint32_t threshold;                       // bit pattern of the threshold
    uint32_t want_lt, want_eq, want_gt, want_un;
};

template <int TYPE>
__device__ __forceinline__ uint32_t keeps(uint32_t u, const Predicate& p) {
    uint32_t lt, eq, gt, un = 0u;
    if constexpr (TYPE == RS_KEY_F32) {
        const float a = __uint_as_float(u), b = __uint_as_float(p.threshold);
        lt = a < b;
        eq = a == b;
        gt = a > b;
        un = !(lt | eq | gt);
    } else if constexpr (TYPE == RS_KEY_I32) {
        const int32_t a = static_cast<int32_t>(u), b = static_cast<int32_t>(p.threshold);
        lt = a < b;
        eq = a == b;
        gt = a > b;
    } else {
        lt = u < p.threshold;
        eq = u == p.threshold;
        gt = u > p.threshold;
    }
    return (lt & p.want_lt) | (eq & p.want_eq) | (gt & p.want_gt) | (un & p.want_un);
}

constexpr int kSelBlock = 1024;

// Writes out[first .. first + count) from s_src[0 .. count): 4-byte stores
// up to the first 16-byte boundary of out, 16-byte stores after it, 4-byte
// stores for the rest (out is 16-byte aligned).
__device__ __forceinline__ void store_span(const uint32_t* s_src, __amdgpu_buffer_rsrc_t out,
                                           uint32_t first, uint32_t count, uint32_t tid) {
    uint32_t head = (4u - (first & 3u)) & 3u;
    if (head > count) head = count;
    const uint32_t quads = (count - head) / 4u;
    const uint32_t tail = head + quads * 4u;
    if (tid < head)
        __builtin_amdgcn_raw_buffer_store_b32(s_src[tid], out, static_cast<int>((first + tid) * 4u), 0, 0);
    for (uint32_t q = tid; q < quads; q += kSelBlock) {
        const uint32_t i = head + 4u * q;
        u32x4 v;
        v.x = s_src[i];
        v.y = s_src[i + 1];
        v.z = s_src[i + 2];
        v.w = s_src[i + 3];
        __builtin_amdgcn_raw_buffer_store_b128(v, out, static_cast<int>((first + i) * 4u), 0, 0);
    }
    if (tid < count - tail)
        __builtin_amdgcn_raw_buffer_store_b32(s_src[tail + tid], out,
                                              static_cast<int>((first + tail + tid) * 4u), 0, 0);
}

struct SelectArgs {
    const uint32_t* in;
    uint32_t* out;
    const uint32_t* vals_in;
    uint32_t* vals_out;
    uint32_t* d_count;
    const uint32_t* kept_total;   // partition: the kept count of the whole input
    uint32_t n, tiles;
    uint32_t* states;
    uint32_t* sched;
    uint32_t groups, chunk_log2;
    Predicate pred;
};

// Tile = 1024 threads x ROWS rows of 16-byte vectors (wave w's row j is the
// 256 consecutive elements at w * 64 * ROWS * 4 + 256 j; lane l holds four).
// In-wave rank of the kept elements with four ballots per row, tile count
// published, wave 0 looks back, kept elements (and values) compacted in LDS
// and stored as one run; PARTITION: then the rejected ones, compacted the
// same way, stored as one run at kept_total + rejected elements before.
template <int TYPE, bool PARTITION, bool PAIRS>
__global__ __launch_bounds__(kSelBlock) void select_kernel(SelectArgs a) {
    constexpr int ROWS = PAIRS ? 4 : 8;
    constexpr int WAVES = kSelBlock / kWave;
    constexpr int WAVE_ELEMS = kWave * ROWS * 4;
    constexpr int TILE = WAVES * WAVE_ELEMS;
    __shared__ uint32_t s_keys[TILE];
    __shared__ uint32_t s_vals[PAIRS ? TILE : 1];
    __shared__ uint32_t s_wave_count[WAVES];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_excl;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;
    const uint32_t group = blockIdx.x % a.groups;
    const uint32_t n = a.n;
    const __amdgpu_buffer_rsrc_t in_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(a.in), 0, static_cast<int>(n * 4u), kBufferWord3);
    const __amdgpu_buffer_rsrc_t vin_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(PAIRS ? a.vals_in : a.in), 0, static_cast<int>(n * 4u), kBufferWord3);
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.out, 0, static_cast<int>(n * 4u), kBufferWord3);
    const __amdgpu_buffer_rsrc_t vout_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        PAIRS ? a.vals_out : a.out, 0, static_cast<int>(n * 4u), kBufferWord3);
    const uint32_t kept_total = PARTITION ? *a.kept_total : 0u;

    for (;;) {
        if (tid == 0) s_tile = next_chunked_tile(a.sched, a.groups, a.chunk_log2, group, a.tiles);
        __syncthreads();
        const uint32_t tile = s_tile;
        if (tile >= a.tiles) break;   // uniform
        const uint32_t tile_base = tile * TILE;
        const uint32_t valid = (n - tile_base < static_cast<uint32_t>(TILE)) ? n - tile_base : TILE;
        const bool full = valid == static_cast<uint32_t>(TILE);

        uint32_t x[ROWS][4];
        uint32_t v[PAIRS ? ROWS : 1][4];
        uint32_t inside[ROWS][4];   // 1 for elements below n
        const uint32_t wave_first = tile_base + wave * WAVE_ELEMS;
#pragma unroll
        for (int j = 0; j < ROWS; ++j) {
            const uint32_t e0 = wave_first + j * (kWave * 4) + lane * 4;
            if (full) {
                const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(in_rsrc, static_cast<int>(e0 * 4u), 0, 2);
                x[j][0] = q.x;
                x[j][1] = q.y;
                x[j][2] = q.z;
                x[j][3] = q.w;
                if constexpr (PAIRS) {
                    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(vin_rsrc, static_cast<int>(e0 * 4u), 0, 2);
                    v[j][0] = w.x;
                    v[j][1] = w.y;
                    v[j][2] = w.z;
                    v[j][3] = w.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[j][e] = __builtin_amdgcn_raw_buffer_load_b32(in_rsrc, static_cast<int>((e0 + e) * 4u), 0, 2);
                    if constexpr (PAIRS)
                        v[j][e] = __builtin_amdgcn_raw_buffer_load_b32(vin_rsrc, static_cast<int>((e0 + e) * 4u), 0, 2);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) inside[j][e] = (e0 + e < n) ? 1u : 0u;
        }

        // exclusive kept count inside the wave: rows before, lanes before, elements before
        uint32_t pos[ROWS][4];   // rank among the wave's kept elements, or among its rejected ones
        uint32_t kp_bits = 0;    // bit 4j + e: element (j, e) is kept
        uint32_t wave_total = 0;
#pragma unroll
        for (int j = 0; j < ROWS; ++j) {
            uint32_t lanes_before = 0, row_total = 0, in_lane = 0;
            uint32_t kp[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kp[e] = keeps<TYPE>(x[j][e], a.pred) & inside[j][e];
                const uint64_t vote = ballot(kp[e] != 0u);
                lanes_before += count_below(vote);
                row_total += static_cast<uint32_t>(__popcll(vote));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t kept_before = wave_total + lanes_before + in_lane;
                // element index inside the wave minus kept before it = rejected before it
                pos[j][e] = kp[e] ? kept_before : (j * (kWave * 4) + lane * 4 + e) - kept_before;
                kp_bits |= kp[e] << (4 * j + e);
                in_lane += kp[e];
            }
            wave_total += row_total;
        }
        if (lane == 0) s_wave_count[wave] = wave_total;
        __syncthreads();

        uint32_t wave_off = 0, tile_count = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const uint32_t c = s_wave_count[w];
            if (w < static_cast<int>(wave)) wave_off += c;
            tile_count += c;
        }
        if (tid == 0)
            store_state(&a.states[tile], (tile == 0 ? kStatePrefix : kStateAggregate) | tile_count);

        // kept elements (and values) compacted in LDS in input order
#pragma unroll
        for (int j = 0; j < ROWS; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((kp_bits >> (4 * j + e)) & 1u) {
                    s_keys[wave_off + pos[j][e]] = x[j][e];
                    if constexpr (PAIRS) s_vals[wave_off + pos[j][e]] = v[j][e];
                }

        if (wave == 0) {
            uint32_t excl = 0;
            if (tile > 0) {
                int32_t newest = static_cast<int32_t>(tile) - 1;
                for (;;) {
                    const int32_t t = newest - static_cast<int32_t>(lane);
                    uint32_t st = (t >= 0) ? load_state(&a.states[t]) : kStatePrefix;
                    for (;;) {
                        const uint64_t not_ready = ballot((st & ~kStateCountMask) == 0u);
                        const uint64_t prefix = ballot((st & kStatePrefix) != 0u);
                        const uint64_t upto = prefix ? (prefix & (~prefix + 1ull)) * 2ull - 1ull : ~0ull;
                        if ((not_ready & upto) == 0ull) break;
                        __builtin_amdgcn_s_sleep(1);
                        if ((st & ~kStateCountMask) == 0u && t >= 0) st = load_state(&a.states[t]);
                    }
                    const uint64_t prefix = ballot((st & kStatePrefix) != 0u);
                    const uint64_t upto = prefix ? (prefix & (~prefix + 1ull)) * 2ull - 1ull : ~0ull;
                    const uint32_t mine = ((upto >> lane) & 1ull) ? (st & kStateCountMask) : 0u;
                    excl += __shfl(wave_inclusive_sum(mine), kWave - 1, kWave);
                    if (prefix) break;
                    newest -= kWave;
                }
                if (lane == 0) store_state(&a.states[tile], kStatePrefix | (excl + tile_count));
            }
            if (lane == 0) s_excl = excl;
        }
        __syncthreads();

        const uint32_t excl = s_excl;
        store_span(s_keys, out_rsrc, excl, tile_count, tid);
        if constexpr (PAIRS) store_span(s_vals, vout_rsrc, excl, tile_count, tid);
        if (tid == 0 && tile == a.tiles - 1) *a.d_count = excl + tile_count;

        if constexpr (PARTITION) {
            // rejected elements: compacted in LDS the same way, stored after every kept one
            __syncthreads();   // the kept run has been read from LDS
            const uint32_t wave_rej_off = wave * WAVE_ELEMS - wave_off;   // rejected in earlier waves
#pragma unroll
            for (int j = 0; j < ROWS; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!((kp_bits >> (4 * j + e)) & 1u) && inside[j][e]) {
                        s_keys[wave_rej_off + pos[j][e]] = x[j][e];
                        if constexpr (PAIRS) s_vals[wave_rej_off + pos[j][e]] = v[j][e];
                    }
            __syncthreads();
            const uint32_t rejected = valid - tile_count;
            const uint32_t first = kept_total + (tile_base - excl);
            store_span(s_keys, out_rsrc, first, rejected, tid);
            if constexpr (PAIRS) store_span(s_vals, vout_rsrc, first, rejected, tid);
        }
        // LDS is rewritten only after the next loop-top barrier
    }
}

// Kept elements of the whole input (partition's first launch): one atomic
// add per block into *total (zeroed beforehand).
template <int TYPE>
__global__ __launch_bounds__(kSelBlock) void count_kept_kernel(const uint32_t* __restrict__ in,
                                                               uint32_t n, Predicate pred,
                                                               uint32_t* __restrict__ total) {
    __shared__ uint32_t s_sum[kSelBlock / kWave];
    const uint32_t tid = threadIdx.x;
    const uint32_t nvec = n / 4;
    const u32x4* in4 = reinterpret_cast<const u32x4*>(in);
    uint32_t c = 0;
    // one contiguous chunk of 16-byte vectors per block, four rows of the
    // block in flight at a time (nvec < 2^28, so no index below wraps)
    constexpr int kInFlight = 4;
    const uint32_t per_block = (nvec + gridDim.x - 1) / gridDim.x;
    const uint32_t begin = blockIdx.x * per_block;
    const uint32_t end = (begin + per_block < nvec) ? begin + per_block : nvec;
    uint32_t i = begin + tid;
    for (; i + (kInFlight - 1) * kSelBlock < end; i += kInFlight * kSelBlock) {
        u32x4 q[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) q[u] = __builtin_nontemporal_load(&in4[i + u * kSelBlock]);
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            c += keeps<TYPE>(q[u].x, pred) + keeps<TYPE>(q[u].y, pred) + keeps<TYPE>(q[u].z, pred) +
                 keeps<TYPE>(q[u].w, pred);
    }
    for (; i < end; i += kSelBlock) {
        const u32x4 q = __builtin_nontemporal_load(&in4[i]);
        c += keeps<TYPE>(q.x, pred) + keeps<TYPE>(q.y, pred) + keeps<TYPE>(q.z, pred) + keeps<TYPE>(q.w, pred);
    }
    if (blockIdx.x == 0 && tid < n - nvec * 4) c += keeps<TYPE>(in[nvec * 4 + tid], pred);
    c = __shfl(wave_inclusive_sum(c), kWave - 1, kWave);
    if ((tid & (kWave - 1)) == 0) s_sum[tid / kWave] = c;
    __syncthreads();
    if (tid == 0) {
        uint32_t s = 0;
        for (int w = 0; w < kSelBlock / kWave; ++w) s += s_sum[w];
        if (s) fetch_add_agent(total, s);
    }
}

// Temp layouts: [tile counters, 256 B][kept total, 256 B][states]
struct ScanLayout {
    size_t sched, total, states, bytes;
    uint32_t tiles;
};

ScanLayout scan_layout(uint64_t n, uint32_t tile, size_t state_bytes) {
    ScanLayout L{};
    L.tiles = static_cast<uint32_t>((n + tile - 1) / tile);
    L.sched = 0;
    L.total = 256;
    L.states = 512;
    L.bytes = 512 + (static_cast<size_t>(L.tiles) * state_bytes + 255) / 256 * 256;
    return L;
}

uint32_t select_tile(bool pairs) { return pairs ? 16384u : 32768u; }

template <typename K>
uint32_t resident_of(K kernel) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 1024, 0) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    return static_cast<uint32_t>(per_cu) * static_cast<uint32_t>(device_cus());
}

Predicate make_predicate(int op, uint32_t threshold_bits) {
    Predicate p{threshold_bits, 0u, 0u, 0u, 0u};
    switch (op) {
    case RS_OP_LT: p.want_lt = 1u; break;
    case RS_OP_LE: p.want_lt = p.want_eq = 1u; break;
    case RS_OP_GT: p.want_gt = 1u; break;
    case RS_OP_GE: p.want_gt = p.want_eq = 1u; break;
    case RS_OP_EQ: p.want_eq = 1u; break;
    default: p.want_lt = p.want_gt = p.want_un = 1u; break;   // !=
    }
    return p;
}

template <int TYPE, bool PARTITION, bool PAIRS>
hipError_t launch_select_t(const SelectArgs& a, hipStream_t s) {
    auto kern = select_kernel<TYPE, PARTITION, PAIRS>;
    static const uint32_t resident = resident_of(kern);   // one-time init
    // 16-tile chunks with values (16384-element tiles: twice the tiles, longer
    // look-back chains; 2^28 partition's select 0.96-0.97 -> 0.90-0.91 ms),
    // 32 without (32768-element tiles, as the compaction)
    const TileGrid g = tile_grid(a.tiles, resident, PAIRS ? kPassChunk : kStreamChunk);
    SelectArgs b = a;
    b.groups = g.groups;
    b.chunk_log2 = g.chunk_log2;
    kern<<<dim3(g.grid), kSelBlock, 0, s>>>(b);
    return hipGetLastError();
}

template <int TYPE>
hipError_t launch_select_type(bool partition, bool pairs, const SelectArgs& a, hipStream_t s) {
    if (partition) {
        if (pairs) return launch_select_t<TYPE, true, true>(a, s);
        return launch_select_t<TYPE, true, false>(a, s);
    }
    if (pairs) return launch_select_t<TYPE, false, true>(a, s);
    return launch_select_t<TYPE, false, false>(a, s);
}

}  // namespace

size_t scan_temp_bytes(uint64_t n) { return scan_layout(n, kScanTile, 8).bytes; }

hipError_t launch_scan(const uint32_t* in, uint32_t* out, uint32_t n, bool inclusive, void* temp,
                       hipStream_t stream) {
    const ScanLayout L = scan_layout(n, kScanTile, 8);
    char* base = static_cast<char*>(temp);
    uint32_t* sched = reinterpret_cast<uint32_t*>(base + L.sched);
    uint64_t* states = reinterpret_cast<uint64_t*>(base + L.states);
    hipError_t e = launch_fill_zero(sched, L.bytes / 4, stream, RS_KERNEL_SCAN_INIT);
    if (e != hipSuccess) return e;
    auto kern = inclusive ? scan_kernel<true> : scan_kernel<false>;
    static const uint32_t resident = resident_of(scan_kernel<false>);   // same shape either way
    const TileGrid g = tile_grid(L.tiles, resident, kStreamChunk);
    timing_before(stream, RS_KERNEL_SCAN);
    kern<<<dim3(g.grid), kScanBlock, 0, stream>>>(in, out, n, L.tiles, states, sched, g.groups, g.chunk_log2);
    e = hipGetLastError();
    timing_after(stream);
    return e;
}

size_t select_temp_bytes(uint64_t n, bool pairs) { return scan_layout(n, select_tile(pairs), 4).bytes; }

hipError_t launch_select(int key_type, int op, uint32_t threshold_bits, const uint32_t* in,
                         uint32_t* out, const uint32_t* vals_in, uint32_t* vals_out,
                         uint32_t* d_count, uint32_t n, bool partition, void* temp,
                         hipStream_t stream) {
    const bool pairs = vals_in != nullptr;
    const ScanLayout L = scan_layout(n, select_tile(pairs), 4);
    char* base = static_cast<char*>(temp);
    SelectArgs a{};
    a.in = in;
    a.out = out;
    a.vals_in = vals_in;
    a.vals_out = vals_out;
    a.d_count = d_count;
    a.kept_total = reinterpret_cast<uint32_t*>(base + L.total);
    a.n = n;
    a.tiles = L.tiles;
    a.states = reinterpret_cast<uint32_t*>(base + L.states);
    a.sched = reinterpret_cast<uint32_t*>(base + L.sched);
    a.pred = make_predicate(op, threshold_bits);
    hipError_t e = launch_fill_zero(a.sched, L.bytes / 4, stream, RS_KERNEL_SELECT_INIT);
    if (e != hipSuccess) return e;
    if (partition) {
        int grid = static_cast<int>((n / 4 + kSelBlock * 8 - 1) / (kSelBlock * 8));
        if (grid < 1) grid = 1;
        if (grid > device_cus()) grid = device_cus();
        uint32_t* total = reinterpret_cast<uint32_t*>(base + L.total);
        timing_before(stream, RS_KERNEL_SELECT_COUNT);
        if (key_type == RS_KEY_F32) count_kept_kernel<RS_KEY_F32><<<grid, kSelBlock, 0, stream>>>(in, n, a.pred, total);
        else if (key_type == RS_KEY_I32) count_kept_kernel<RS_KEY_I32><<<grid, kSelBlock, 0, stream>>>(in, n, a.pred, total);
        else count_kept_kernel<RS_KEY_U32><<<grid, kSelBlock, 0, stream>>>(in, n, a.pred, total);
        e = hipGetLastError();
        timing_after(stream);
        if (e != hipSuccess) return e;
    }
    timing_before(stream, RS_KERNEL_SELECT);
    if (key_type == RS_KEY_F32) e = launch_select_type<RS_KEY_F32>(partition, pairs, a, stream);
    else if (key_type == RS_KEY_I32) e = launch_select_type<RS_KEY_I32>(partition, pairs, a, stream);
    else e = launch_select_type<RS_KEY_U32>(partition, pairs, a, stream);
    timing_after(stream);
    return e;
}

}  // namespace rs
