// radix.hip -- stable LSD radix sort of 32-bit keys (and key-value pairs) for
// gfx950, one-sweep style with 8-bit digits.
//
// The method ("CUDA 算子笔记 3", section 一次处理多位): one read of the keys
// counts the digits of every pass (upsweep); then each pass places every key
// at  bucket start + same-digit keys in earlier tiles + stable rank inside its
// tile, where the middle term comes from a decoupled look-back over per-tile
// digit counts (same page, section on the decoupled look-back scan).  Each
// pass is a stable counting sort, which is what makes the LSD order correct
// ("WebGPU Unleashed", 4.1 래딕스 정렬; "第10章 并行模式：排序", 10.3).
//
// How it maps onto CDNA4:
//  * tile = BLOCK x ITEMS keys; a wave owns a contiguous run of 64 x ITEMS
//    keys, loaded as ITEMS coalesced 256-byte rows (lane l of row j holds
//    position j*64 + l), so rank order is (wave, row, lane) = input order;
//  * the in-wave stable rank uses eight ballots to find the lanes holding
//    the same digit, mbcnt to count the ones below, and a per-wave LDS
//    counter per digit updated by one lane per digit group (no LDS atomics,
//    one LDS write per distinct digit, so skewed inputs cost less, not more);
//  * the tile is re-laid out in LDS in digit order so that each digit's run
//    is written to HBM with consecutive addresses;
//  * tile ids come from an atomic counter, so a tile only ever waits on
//    tiles that are already running; state words are read and written at
//    agent scope because tiles on different XCDs sit behind different L2s.
#include "device_common.hpp"
#include "internal.hpp"

namespace rs {

namespace {

constexpr int kSortBlock = 512;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortBlock * kSortItems;

constexpr int kUpBlock = 256;
constexpr int kUpSub = 4;          // sub-histograms per digit (spreads LDS atomics)
constexpr int kMaxPasses = 4;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---------------------------------------------------------------------------
// Fill kernel: zeroes a u32 region (temp counters, bins and tile states).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, uint64_t words) {
    const uint64_t nvec = words / 4;
    uint4* p4 = reinterpret_cast<uint4*>(p);
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec;
         i += stride)
        p4[i] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0 && threadIdx.x < words - nvec * 4) p[nvec * 4 + threadIdx.x] = 0u;
}

// ---------------------------------------------------------------------------
// Upsweep: counts of every pass's digit over all keys, in one read.
// bins[p * 256 + d] += #keys with digit_p == d  (bins zeroed beforehand).
// ("CUDA 算子笔记 3", 一次处理多位, the first kernel; "第10章", 10.3 and 10.4
// on shared-memory histograms and spreading atomic contention.)
// ---------------------------------------------------------------------------
struct PassDigits {
    uint32_t shift[kMaxPasses];
    uint32_t mask[kMaxPasses];
    uint32_t passes;
};

template <bool FLIP>
__device__ __forceinline__ void count_key(uint32_t* s_hist, uint32_t key, const PassDigits& pd,
                                          uint32_t sub) {
    if (FLIP) key = float_to_sortable(key);
#pragma unroll
    for (int p = 0; p < kMaxPasses; ++p) {
        if (p < static_cast<int>(pd.passes)) {
            const uint32_t d = (key >> pd.shift[p]) & pd.mask[p];
            atomicAdd(&s_hist[(p * kRadix + d) * kUpSub + sub], 1u);
        }
    }
}

template <bool FLIP>
__global__ __launch_bounds__(kUpBlock) void upsweep_kernel(const uint32_t* __restrict__ keys,
                                                           uint32_t n, PassDigits pd,
                                                           uint32_t* __restrict__ bins) {
    __shared__ uint32_t s_hist[kMaxPasses * kRadix * kUpSub];
    for (int i = threadIdx.x; i < kMaxPasses * kRadix * kUpSub; i += kUpBlock) s_hist[i] = 0u;
    __syncthreads();

    const uint32_t sub = threadIdx.x % kUpSub;
    const uint32_t nvec = n / 4;
    const uint4* k4 = reinterpret_cast<const uint4*>(keys);
    const uint32_t stride = gridDim.x * kUpBlock;
    for (uint32_t i = blockIdx.x * kUpBlock + threadIdx.x; i < nvec; i += stride) {
        const uint4 q = k4[i];
        count_key<FLIP>(s_hist, q.x, pd, sub);
        count_key<FLIP>(s_hist, q.y, pd, sub);
        count_key<FLIP>(s_hist, q.z, pd, sub);
        count_key<FLIP>(s_hist, q.w, pd, sub);
    }
    if (blockIdx.x == 0 && threadIdx.x < n - nvec * 4)
        count_key<FLIP>(s_hist, keys[nvec * 4 + threadIdx.x], pd, sub);
    __syncthreads();

    for (uint32_t i = threadIdx.x; i < pd.passes * kRadix; i += kUpBlock) {
        uint32_t c = 0;
#pragma unroll
        for (int s = 0; s < kUpSub; ++s) c += s_hist[i * kUpSub + s];
        if (c) fetch_add_agent(&bins[i], c);
    }
}

// ---------------------------------------------------------------------------
// One-sweep pass: stable scatter of one 8-bit digit.
// ---------------------------------------------------------------------------

// Lanes of the wave whose digit equals this lane's (eight ballots).
__device__ __forceinline__ uint64_t lanes_with_same_digit(uint32_t d) {
    uint64_t peers = ~0ull;
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t vote = ballot(bit);
        peers &= bit ? vote : ~vote;
    }
    return peers;
}

template <int BLOCK, int ITEMS, bool PAIRS, bool FLIP_IN, bool FLIP_OUT>
__global__ __launch_bounds__(BLOCK) void onesweep_kernel(
    const uint32_t* __restrict__ src_keys, uint32_t* __restrict__ dst_keys,
    const uint32_t* __restrict__ src_vals, uint32_t* __restrict__ dst_vals, uint32_t n,
    uint32_t shift, uint32_t mask, const uint32_t* __restrict__ bins,
    uint32_t* __restrict__ states, uint32_t* __restrict__ next_states,
    uint32_t* __restrict__ tile_counter) {
    constexpr int WAVES = BLOCK / kWave;
    constexpr int TILE = BLOCK * ITEMS;
    static_assert(BLOCK >= kRadix && BLOCK % kWave == 0, "one thread per digit needed");

    __shared__ uint32_t s_keys[TILE];
    __shared__ uint32_t s_vals[PAIRS ? TILE : 1];
    __shared__ uint32_t s_off[WAVES * kRadix];   // per-wave digit counters, then offsets
    __shared__ uint32_t s_adjust[kRadix];
    __shared__ uint32_t s_wsum[2][kRadix / kWave];
    __shared__ uint32_t s_tile;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;

    if (tid == 0) s_tile = fetch_add_agent(tile_counter, 1u);
    for (uint32_t i = lane; i < kRadix; i += kWave) s_off[wave * kRadix + i] = 0u;
    // global digit count of this pass (thread d holds digit d)
    const uint32_t bin = (tid < kRadix) ? bins[tid] : 0u;
    __syncthreads();

    const uint32_t tile = s_tile;
    const uint32_t tile_base = tile * TILE;
    const uint32_t valid = (n - tile_base < static_cast<uint32_t>(TILE)) ? n - tile_base : TILE;
    const bool full = (valid == static_cast<uint32_t>(TILE));

    // ---- load: row j of wave w is 64 consecutive keys -------------------------
    uint32_t k[ITEMS];
    uint32_t v[PAIRS ? ITEMS : 1];
    const uint32_t first = tile_base + wave * (kWave * ITEMS) + lane;
    if (full) {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            k[j] = src_keys[first + j * kWave];
            if (PAIRS) v[j] = src_vals[first + j * kWave];
        }
    } else {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t idx = first + j * kWave;
            const bool in = idx < n;
            k[j] = in ? src_keys[idx] : 0u;
            if (PAIRS) v[j] = in ? src_vals[idx] : 0u;
        }
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        if (FLIP_IN) k[j] = float_to_sortable(k[j]);
        if (!full && first + j * kWave >= n) k[j] = 0xFFFFFFFFu;   // padding sorts last
    }

    // ---- stable rank inside the wave ------------------------------------------
    uint32_t rank[ITEMS];
    uint32_t* my_count = s_off + wave * kRadix;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t d = (k[j] >> shift) & mask;
        const uint64_t peers = lanes_with_same_digit(d);
        const uint32_t below = count_below(peers);
        const uint32_t before = my_count[d];
        if (below == 0) my_count[d] = before + static_cast<uint32_t>(__popcll(peers));
        rank[j] = before + below;
    }
    __syncthreads();

    // ---- per digit: offsets of each wave, tile count, scans -----------------
    uint32_t count = 0;
    if (tid < kRadix) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const uint32_t c = s_off[w * kRadix + tid];
            s_off[w * kRadix + tid] = count;
            count += c;
        }
    }
    // the padding of a partial tile sits in the last digit; it is not published
    const uint32_t pads = full ? 0u : static_cast<uint32_t>(TILE) - valid;
    const uint32_t real = (tid == mask) ? count - pads : count;
    if (tid < kRadix)
        store_state(&states[tile * kRadix + tid], (tile == 0 ? kStatePrefix : kStateAggregate) | real);

    uint32_t inc_c = 0, inc_b = 0;
    if (tid < kRadix) {
        inc_c = wave_inclusive_sum(count);
        inc_b = wave_inclusive_sum(bin);
        if (lane == kWave - 1) {
            s_wsum[0][wave] = inc_c;
            s_wsum[1][wave] = inc_b;
        }
    }
    __syncthreads();
    uint32_t local_start = 0, bin_start = 0;
    if (tid < kRadix) {
        uint32_t pc = 0, pb = 0;
#pragma unroll
        for (int w = 0; w < kRadix / kWave; ++w) {
            if (w < static_cast<int>(wave)) {
                pc += s_wsum[0][w];
                pb += s_wsum[1][w];
            }
        }
        local_start = pc + inc_c - count;
        bin_start = pb + inc_b - bin;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s_off[w * kRadix + tid] += local_start;
    }
    __syncthreads();

    // ---- re-lay the tile out in digit order in LDS -------------------------------
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t d = (k[j] >> shift) & mask;
        const uint32_t pos = s_off[wave * kRadix + d] + rank[j];
        s_keys[pos] = k[j];
        if (PAIRS) s_vals[pos] = v[j];
    }

    // ---- decoupled look-back: same-digit keys in all earlier tiles ------------
    if (tid < kRadix) {
        uint32_t excl = 0;
        if (tile > 0) {
            int32_t t = static_cast<int32_t>(tile) - 1;
            for (;;) {
                const uint32_t s = load_state(&states[static_cast<uint32_t>(t) * kRadix + tid]);
                if ((s & ~kStateCountMask) == 0u) {
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                excl += s & kStateCountMask;
                if (s & kStatePrefix) break;
                --t;
            }
            store_state(&states[tile * kRadix + tid], kStatePrefix | (excl + real));
        }
        s_adjust[tid] = bin_start + excl - local_start;
        if (next_states) next_states[tile * kRadix + tid] = 0u;
    }
    __syncthreads();

    // ---- scatter each digit run to consecutive addresses --------------------------
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const uint32_t i = r * BLOCK + tid;
        if (full || i < valid) {
            const uint32_t key = s_keys[i];
            const uint32_t dst = i + s_adjust[(key >> shift) & mask];
            if (dst < n) {   // always true for consistent counts; guards the store
                dst_keys[dst] = FLIP_OUT ? sortable_to_float(key) : key;
                if (PAIRS) dst_vals[dst] = s_vals[i];
            }
        }
    }
}

// Temp layout (every piece 256-byte aligned):
//   bins     [kMaxPasses][256] u32   global digit counts of each pass
//   counters [kMaxPasses]      u32   tile-id counters, padded to 256 B
//   states0  [tiles][256]      u32   look-back states of even passes
//   states1  [tiles][256]      u32   look-back states of odd passes (passes >= 2)
//   tmp_keys [n] u32, tmp_vals [n] u32   ping-pong buffers (passes >= 2)
// bins, counters and states0 are contiguous and cleared by one fill launch.
struct SortLayout {
    size_t bins, counters, states0, states1, tmp_keys, tmp_vals, total;
    uint64_t clear_words;
    uint32_t tiles;
};

SortLayout sort_layout(uint64_t n, bool pairs, int passes) {
    SortLayout L{};
    L.tiles = static_cast<uint32_t>((n + kSortTile - 1) / kSortTile);
    const size_t states_bytes = align_up(static_cast<size_t>(L.tiles) * kRadix * 4);
    size_t off = 0;
    L.bins = off;
    off += align_up(kMaxPasses * kRadix * 4);
    L.counters = off;
    off += align_up(kMaxPasses * 4);
    L.states0 = off;
    off += states_bytes;
    L.clear_words = off / 4;
    L.states1 = off;
    if (passes >= 2) off += states_bytes;
    L.tmp_keys = off;
    if (passes >= 2) off += align_up(n * 4);
    L.tmp_vals = off;
    if (passes >= 2 && pairs) off += align_up(n * 4);
    L.total = off;
    return L;
}

template <int BLOCK, int ITEMS, bool PAIRS>
hipError_t launch_pass(bool flip_in, bool flip_out, dim3 grid, hipStream_t s,
                       const uint32_t* sk, uint32_t* dk, const uint32_t* sv, uint32_t* dv,
                       uint32_t n, uint32_t shift, uint32_t mask, const uint32_t* bins,
                       uint32_t* states, uint32_t* next_states, uint32_t* counter) {
    if (flip_in && flip_out)
        onesweep_kernel<BLOCK, ITEMS, PAIRS, true, true><<<grid, BLOCK, 0, s>>>(
            sk, dk, sv, dv, n, shift, mask, bins, states, next_states, counter);
    else if (flip_in)
        onesweep_kernel<BLOCK, ITEMS, PAIRS, true, false><<<grid, BLOCK, 0, s>>>(
            sk, dk, sv, dv, n, shift, mask, bins, states, next_states, counter);
    else if (flip_out)
        onesweep_kernel<BLOCK, ITEMS, PAIRS, false, true><<<grid, BLOCK, 0, s>>>(
            sk, dk, sv, dv, n, shift, mask, bins, states, next_states, counter);
    else
        onesweep_kernel<BLOCK, ITEMS, PAIRS, false, false><<<grid, BLOCK, 0, s>>>(
            sk, dk, sv, dv, n, shift, mask, bins, states, next_states, counter);
    return hipGetLastError();
}

int upsweep_grid(uint32_t n) {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    const uint64_t vec_per_block = static_cast<uint64_t>(kUpBlock) * 16;   // >= 16 uint4 per thread
    uint64_t g = (static_cast<uint64_t>(n) / 4 + vec_per_block - 1) / vec_per_block;
    if (g < 1) g = 1;
    if (g > static_cast<uint64_t>(cus) * 2) g = static_cast<uint64_t>(cus) * 2;
    return static_cast<int>(g);
}

}  // namespace

uint32_t onesweep_tile_keys() { return kSortTile; }

size_t sort_temp_bytes(uint64_t n, bool pairs, int passes) {
    return sort_layout(n, pairs, passes).total;
}

hipError_t launch_fill_zero(uint32_t* p, uint64_t words, hipStream_t stream, int kernel_id) {
    if (words == 0) return hipSuccess;
    uint64_t blocks = (words / 4 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 2048) blocks = 2048;
    timing_before(stream, kernel_id);
    fill_zero_kernel<<<dim3(static_cast<uint32_t>(blocks)), 256, 0, stream>>>(p, words);
    hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

hipError_t launch_sort(const uint32_t* keys_in, uint32_t* keys_out, const uint32_t* vals_in,
                       uint32_t* vals_out, uint32_t n, int begin_bit, int end_bit, bool is_f32,
                       void* temp, hipStream_t stream) {
    const bool pairs = vals_in != nullptr;
    const int passes = (end_bit - begin_bit + kRadixBits - 1) / kRadixBits;
    const SortLayout L = sort_layout(n, pairs, passes);
    char* base = static_cast<char*>(temp);
    uint32_t* bins = reinterpret_cast<uint32_t*>(base + L.bins);
    uint32_t* counters = reinterpret_cast<uint32_t*>(base + L.counters);
    uint32_t* states[2] = {reinterpret_cast<uint32_t*>(base + L.states0),
                           reinterpret_cast<uint32_t*>(base + L.states1)};
    uint32_t* tmp_keys = reinterpret_cast<uint32_t*>(base + L.tmp_keys);
    uint32_t* tmp_vals = reinterpret_cast<uint32_t*>(base + L.tmp_vals);

    hipError_t e = launch_fill_zero(reinterpret_cast<uint32_t*>(base), L.clear_words, stream,
                                    RS_KERNEL_SORT_INIT);
    if (e != hipSuccess) return e;

    PassDigits pd{};
    pd.passes = static_cast<uint32_t>(passes);
    for (int p = 0; p < passes; ++p) {
        const int s = begin_bit + kRadixBits * p;
        const int w = (end_bit - s < kRadixBits) ? end_bit - s : kRadixBits;
        pd.shift[p] = static_cast<uint32_t>(s);
        pd.mask[p] = (1u << w) - 1u;
    }
    timing_before(stream, RS_KERNEL_UPSWEEP);
    if (is_f32)
        upsweep_kernel<true><<<upsweep_grid(n), kUpBlock, 0, stream>>>(keys_in, n, pd, bins);
    else
        upsweep_kernel<false><<<upsweep_grid(n), kUpBlock, 0, stream>>>(keys_in, n, pd, bins);
    e = hipGetLastError();
    timing_after(stream);
    if (e != hipSuccess) return e;

    const dim3 grid(L.tiles);
    const uint32_t* sk = keys_in;
    const uint32_t* sv = vals_in;
    for (int p = 0; p < passes; ++p) {
        const bool to_out = ((passes - 1 - p) % 2) == 0;
        uint32_t* dk = to_out ? keys_out : tmp_keys;
        uint32_t* dv = pairs ? (to_out ? vals_out : tmp_vals) : nullptr;
        uint32_t* next = (p + 1 < passes) ? states[(p + 1) & 1] : nullptr;
        const bool flip_in = is_f32 && p == 0;
        const bool flip_out = is_f32 && p == passes - 1;
        timing_before(stream, RS_KERNEL_ONESWEEP);
        if (pairs)
            e = launch_pass<kSortBlock, kSortItems, true>(flip_in, flip_out, grid, stream, sk, dk, sv,
                                                          dv, n, pd.shift[p], pd.mask[p],
                                                          bins + p * kRadix, states[p & 1], next,
                                                          counters + p);
        else
            e = launch_pass<kSortBlock, kSortItems, false>(flip_in, flip_out, grid, stream, sk, dk,
                                                           nullptr, nullptr, n, pd.shift[p],
                                                           pd.mask[p], bins + p * kRadix,
                                                           states[p & 1], next, counters + p);
        timing_after(stream);
        if (e != hipSuccess) return e;
        sk = dk;
        sv = dv;
    }
    return hipSuccess;
}

}  // namespace rs
