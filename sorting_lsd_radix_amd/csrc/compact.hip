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
//  * wave 0 looks back over 64 earlier tiles per step (agent-scope loads);
//  * persistent blocks take tiles from the XCD-chunked scheduler, so the
//    output runs of neighbouring tiles meet in one XCD's L2.
#include <mutex>

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

// Writes out[first .. first + count): the values s_src[0 .. count) (or zeros
// when s_src is null), with 4-byte stores up to the first 16-byte boundary,
// 16-byte stores after it (thread t writes quad t, t + 1024, ...) and 4-byte
// stores for the last count mod 4 elements.  `out` is 16-byte aligned.
__device__ __forceinline__ void store_run(const uint32_t* s_src, __amdgpu_buffer_rsrc_t out,
                                          uint32_t first, uint32_t count, uint32_t tid) {
    uint32_t head = (4u - (first & 3u)) & 3u;
    if (head > count) head = count;
    const uint32_t quads = (count - head) / 4u;
    const uint32_t tail = head + quads * 4u;
    if (tid < head)
        __builtin_amdgcn_raw_buffer_store_b32(s_src ? s_src[tid] : 0u, out,
                                              static_cast<int>((first + tid) * 4u), 0, 0);
    for (uint32_t q = tid; q < quads; q += kCompBlock) {
        const uint32_t i = head + 4u * q;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (s_src) {
            v.x = s_src[i];
            v.y = s_src[i + 1];
            v.z = s_src[i + 2];
            v.w = s_src[i + 3];
        }
        __builtin_amdgcn_raw_buffer_store_b128(v, out, static_cast<int>((first + i) * 4u), 0, 0);
    }
    if (tid < count - tail)
        __builtin_amdgcn_raw_buffer_store_b32(s_src ? s_src[tail + tid] : 0u, out,
                                              static_cast<int>((first + tail + tid) * 4u), 0, 0);
}

// Persistent: each block loops over the tiles the chunked scheduler hands it.
__global__ __launch_bounds__(kCompBlock) void compact_kernel(const uint32_t* __restrict__ in,
                                                             uint32_t* __restrict__ out,
                                                             uint32_t* __restrict__ d_count,
                                                             uint32_t n, uint32_t tiles,
                                                             uint32_t* __restrict__ states,
                                                             uint32_t* __restrict__ sched,
                                                             uint32_t groups, uint32_t chunk_log2) {
    constexpr int WAVES = kCompBlock / kWave;
    __shared__ uint32_t s_out[kCompTile];
    __shared__ uint32_t s_wave_count[WAVES];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_excl;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;
    const uint32_t group = blockIdx.x % groups;
    // stores through a descriptor of n elements: an index past the end (never
    // reached for consistent counts) is dropped by the hardware
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(out, 0, static_cast<int>(n * 4u), kBufferWord3);

    for (;;) {
        // the previous tile's readers of s_tile, s_out and s_excl all passed a
        // barrier since
        if (tid == 0) s_tile = next_chunked_tile(sched, groups, chunk_log2, group, tiles);
        __syncthreads();
        const uint32_t tile = s_tile;
        if (tile >= tiles) break;   // uniform: no tiles left
        const uint32_t tile_base = tile * kCompTile;
        const uint32_t valid = (n - tile_base < static_cast<uint32_t>(kCompTile)) ? n - tile_base
                                                                                : kCompTile;

        // ---- load eight rows of 256 floats per wave --------------------------------
        uint32_t x[kCompRows][4];
        const uint32_t wave_first = tile_base + wave * kCompWaveElems;
        if (valid == static_cast<uint32_t>(kCompTile)) {
            // a full tile: streaming 16-byte loads, each float read once
            const u32x4* p = reinterpret_cast<const u32x4*>(in + wave_first) + lane;
#pragma unroll
            for (int j = 0; j < kCompRows; ++j) {
                const u32x4 q = __builtin_nontemporal_load(p + j * kWave);
                x[j][0] = q.x;
                x[j][1] = q.y;
                x[j][2] = q.z;
                x[j][3] = q.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kCompRows; ++j) {
                const uint32_t e0 = wave_first + j * (kWave * 4) + lane * 4;
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
                    uint32_t st = (t >= 0) ? load_state(&states[t]) : kStatePrefix;
                    // wait until the lanes up to the nearest published prefix are ready
                    for (;;) {
                        const uint64_t not_ready = ballot((st & ~kStateCountMask) == 0u);
                        const uint64_t prefix = ballot((st & kStatePrefix) != 0u);
                        const uint64_t upto = prefix ? (prefix & (~prefix + 1ull)) * 2ull - 1ull : ~0ull;
                        if ((not_ready & upto) == 0ull) break;
                        __builtin_amdgcn_s_sleep(1);
                        if ((st & ~kStateCountMask) == 0u && t >= 0) st = load_state(&states[t]);
                    }
                    const uint64_t prefix = ballot((st & kStatePrefix) != 0u);
                    const uint64_t upto = prefix ? (prefix & (~prefix + 1ull)) * 2ull - 1ull : ~0ull;
                    const uint32_t mine = ((upto >> lane) & 1ull) ? (st & kStateCountMask) : 0u;
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
        store_run(s_out, out_rsrc, excl, tile_count, tid);
        const uint32_t rejected_before = tile_base - excl;
        const uint32_t rejected = valid - tile_count;
        const uint32_t zero_first = n - rejected_before - rejected;
        store_run(nullptr, out_rsrc, zero_first, rejected, tid);
        if (tid == 0 && tile == tiles - 1) *d_count = excl + tile_count;
    }
}

// Temp layout: [tile counters: one u32 per group, padded to 256 B][states: tiles u32]
struct CompactLayout {
    size_t sched, states, total;
    uint32_t tiles;
};

CompactLayout compact_layout(uint64_t n) {
    CompactLayout L{};
    L.tiles = static_cast<uint32_t>((n + kCompTile - 1) / kCompTile);
    L.sched = 0;
    L.states = 256;
    L.total = 256 + (static_cast<size_t>(L.tiles) * 4 + 255) / 256 * 256;
    return L;
}

uint32_t compact_resident() {
    static const uint32_t resident = [] {   // thread-safe one-time init
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, compact_kernel, kCompBlock, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        return static_cast<uint32_t>(per_cu) * static_cast<uint32_t>(device_cus());
    }();
    return resident;
}

// ---- allocation-free variant -----------------------------------------------------
// The scratch of rs_compact_positive_f32_noalloc: a file-scope device array
// big enough for the tile counters and tile states of every accepted size
// (n < 2^30: 32768 tiles of 32768 elements).  Each device holds its own copy
// until the process ends; in host code `scratch` only names the symbol, so
// its device address is looked up once per device and kept.
constexpr size_t kStaticScratchBytes = 256 + (static_cast<size_t>(RS_MAX_N / kCompTile) * 4 + 255) / 256 * 256;
__device__ __align__(256) uint32_t scratch[kStaticScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on failure).
void* static_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

size_t compact_temp_bytes(uint64_t n) { return compact_layout(n).total; }

size_t compact_static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t launch_compact_static(const float* in, float* out, uint32_t* d_count, uint32_t n,
                                 hipStream_t stream) {
    if (compact_layout(n).total > kStaticScratchBytes) return hipErrorInvalidValue;
    void* ptr = static_scratch();
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    // the same kernels as launch_compact; the fill kernel clears the counters
    // and states the previous call left in the scratch
    return launch_compact(in, out, d_count, n, ptr, stream);
}

hipError_t launch_compact(const float* in, float* out, uint32_t* d_count, uint32_t n, void* temp,
                          hipStream_t stream) {
    const CompactLayout L = compact_layout(n);
    char* base = static_cast<char*>(temp);
    uint32_t* sched = reinterpret_cast<uint32_t*>(base + L.sched);
    uint32_t* states = reinterpret_cast<uint32_t*>(base + L.states);
    hipError_t e = launch_fill_zero(sched, L.total / 4, stream, RS_KERNEL_COMPACT_INIT);
    if (e != hipSuccess) return e;
    const TileGrid g = tile_grid(L.tiles, compact_resident(), kStreamChunk);
    timing_before(stream, RS_KERNEL_COMPACT);
    compact_kernel<<<dim3(g.grid), kCompBlock, 0, stream>>>(
        reinterpret_cast<const uint32_t*>(in), reinterpret_cast<uint32_t*>(out), d_count, n,
        L.tiles, states, sched, g.groups, g.chunk_log2);
    e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace rs
