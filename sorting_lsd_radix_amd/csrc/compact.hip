// compact.hip -- single-pass stream compaction of positive floats for gfx950.
//
// out[0..k) = the x > 0 of the input in order, out[k..n) = +0.0f, count = k
// ("CUDA 算子笔记 3", section Stream Compaction: predicate, exclusive scan of
// the predicate, scatter; and its decoupled look-back method, where each tile
// publishes its own count, then walks back over earlier tiles' counts until it
// meets a published inclusive prefix, with a whole wave probing earlier tiles
// at once).
//
// gfx950 mapping:
//  * tile = 1024 threads x 32 floats (32768), loaded as eight 16-byte vectors
//    per lane; within a wave, row j covers 256 consecutive floats (lane l
//    holds 4 of them), so the in-tile exclusive count is: rows before + lanes
//    before (four ballots and mbcnt) + elements before in the lane.  Large
//    tiles keep the number of tiles in flight, and so the look-back walk,
//    short;
//  * the predicate is taken on bits: (u - 1) < 0x7F800000 is exactly
//    x > 0.0f for IEEE binary32 including subnormals, so no flush-to-zero
//    mode can change it;
//  * kept values are compacted in LDS and stored as one contiguous run; the
//    rejected count of the tile is written as one contiguous run of zeros at
//    the far end, so the whole output is written exactly once;
//  * wave 0 looks back over 64 earlier tiles per step (agent-scope loads).
#include "device_common.hpp"
#include "internal.hpp"

namespace rs {

namespace {

constexpr int kCompBlock = 1024;
constexpr int kCompRows = 8;                               // 16-byte vectors per lane
constexpr int kCompWaveElems = kWave * kCompRows * 4;      // 2048 floats per wave
constexpr int kCompTile = (kCompBlock / kWave) * kCompWaveElems;

__device__ __forceinline__ uint32_t keep_positive(uint32_t u) {
    return (u - 1u) < 0x7F800000u ? 1u : 0u;
}

__global__ __launch_bounds__(kCompBlock) void compact_kernel(const uint32_t* __restrict__ in,
                                                             uint32_t* __restrict__ out,
                                                             uint32_t* __restrict__ d_count,
                                                             uint32_t n, uint32_t tiles,
                                                             uint32_t* __restrict__ states,
                                                             uint32_t* __restrict__ tile_counter) {
    constexpr int WAVES = kCompBlock / kWave;
    __shared__ uint32_t s_out[kCompTile];
    __shared__ uint32_t s_wave_count[WAVES];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_excl;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;

    if (tid == 0) s_tile = fetch_add_agent(tile_counter, 1u);
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint32_t tile_base = tile * kCompTile;
    const uint32_t valid = (n - tile_base < static_cast<uint32_t>(kCompTile)) ? n - tile_base
                                                                            : kCompTile;

    // ---- load four rows of 256 floats per wave --------------------------------
    uint32_t x[kCompRows][4];
    const uint32_t wave_first = tile_base + wave * kCompWaveElems;
#pragma unroll
    for (int j = 0; j < kCompRows; ++j) {
        const uint32_t e0 = wave_first + j * (kWave * 4) + lane * 4;
        if (e0 + 3 < n) {
            const uint4 q = *reinterpret_cast<const uint4*>(in + e0);
            x[j][0] = q.x;
            x[j][1] = q.y;
            x[j][2] = q.z;
            x[j][3] = q.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[j][e] = (e0 + e < n) ? in[e0 + e] : 0u;  // 0 is not kept
        }
    }

    // ---- exclusive count of kept elements inside the wave ---------------------
    uint32_t pos[kCompRows][4];
    uint32_t wave_total = 0;
#pragma unroll
    for (int j = 0; j < kCompRows; ++j) {
        uint32_t lanes_before = 0, row_total = 0, in_lane = 0;
        uint32_t kp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kp[e] = keep_positive(x[j][e]);
            const uint64_t vote = ballot(kp[e] != 0u);
            lanes_before += count_below(vote);
            row_total += static_cast<uint32_t>(__popcll(vote));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pos[j][e] = kp[e] ? wave_total + lanes_before + in_lane : 0xFFFFFFFFu;
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
        store_state(&states[tile], (tile == 0 ? kStatePrefix : kStateAggregate) | tile_count);

    // ---- compact the kept values of the tile in LDS ---------------------------
#pragma unroll
    for (int j = 0; j < kCompRows; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (pos[j][e] != 0xFFFFFFFFu) s_out[wave_off + pos[j][e]] = x[j][e];

    // ---- look back: kept elements in all earlier tiles -----------------------
    if (wave == 0) {
        uint32_t excl = 0;
        if (tile > 0) {
            int32_t newest = static_cast<int32_t>(tile) - 1;   // probed by lane 0
            for (;;) {
                const int32_t t = newest - static_cast<int32_t>(lane);
                uint32_t s = (t >= 0) ? load_state(&states[t]) : kStatePrefix;
                // wait until the lanes up to the nearest published prefix are ready
                for (;;) {
                    const uint64_t not_ready = ballot((s & ~kStateCountMask) == 0u);
                    const uint64_t prefix = ballot((s & kStatePrefix) != 0u);
                    const uint64_t upto = prefix ? (prefix & (~prefix + 1ull)) * 2ull - 1ull : ~0ull;
                    if ((not_ready & upto) == 0ull) break;
                    __builtin_amdgcn_s_sleep(1);
                    if ((s & ~kStateCountMask) == 0u && t >= 0) s = load_state(&states[t]);
                }
                const uint64_t prefix = ballot((s & kStatePrefix) != 0u);
                const uint64_t upto = prefix ? (prefix & (~prefix + 1ull)) * 2ull - 1ull : ~0ull;
                const uint32_t mine = ((upto >> lane) & 1ull) ? (s & kStateCountMask) : 0u;
                excl += __shfl(wave_inclusive_sum(mine), kWave - 1, kWave);
                if (prefix) break;
                newest -= kWave;
            }
            if (lane == 0) store_state(&states[tile], kStatePrefix | (excl + tile_count));
        }
        if (lane == 0) s_excl = excl;
    }
    __syncthreads();

    // ---- contiguous stores: kept run, then this tile's share of the zero tail --
    const uint32_t excl = s_excl;
    // (the index checks always pass for consistent counts; they guard the stores)
    for (uint32_t i = tid; i < tile_count; i += kCompBlock)
        if (excl + i < n) out[excl + i] = s_out[i];
    const uint32_t rejected_before = tile_base - excl;
    const uint32_t rejected = valid - tile_count;
    const uint32_t zero_first = n - rejected_before - rejected;
    for (uint32_t i = tid; i < rejected; i += kCompBlock)
        if (zero_first + i < n) out[zero_first + i] = 0u;
    if (tid == 0 && tile == tiles - 1) *d_count = excl + tile_count;
}

// Temp layout: [counter u32, padded to 256 B][states: tiles u32]
struct CompactLayout {
    size_t counter, states, total;
    uint32_t tiles;
};

CompactLayout compact_layout(uint64_t n) {
    CompactLayout L{};
    L.tiles = static_cast<uint32_t>((n + kCompTile - 1) / kCompTile);
    L.counter = 0;
    L.states = 256;
    L.total = 256 + (static_cast<size_t>(L.tiles) * 4 + 255) / 256 * 256;
    return L;
}

}  // namespace

size_t compact_temp_bytes(uint64_t n) { return compact_layout(n).total; }

hipError_t launch_compact(const float* in, float* out, uint32_t* d_count, uint32_t n, void* temp,
                          hipStream_t stream) {
    const CompactLayout L = compact_layout(n);
    char* base = static_cast<char*>(temp);
    uint32_t* counter = reinterpret_cast<uint32_t*>(base + L.counter);
    uint32_t* states = reinterpret_cast<uint32_t*>(base + L.states);
    hipError_t e = launch_fill_zero(counter, L.total / 4, stream, RS_KERNEL_COMPACT_INIT);
    if (e != hipSuccess) return e;
    timing_before(stream, RS_KERNEL_COMPACT);
    compact_kernel<<<dim3(L.tiles), kCompBlock, 0, stream>>>(
        reinterpret_cast<const uint32_t*>(in), reinterpret_cast<uint32_t*>(out), d_count, n,
        L.tiles, states, counter);
    e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace rs
