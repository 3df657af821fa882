// radix.hip -- stable LSD radix sort of 32- and 64-bit keys (and key-value
// pairs) for gfx950, one-sweep style with 8-bit digits.
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
//  * the stable rank inside a wave is one LDS atomic add per key on the
//    wave's counter of its digit, whose same-address lanes the hardware
//    serves in lane order (checked by a GPU test); while a digit is crowded
//    it is instead eight ballots that find the lanes holding the same digit,
//    mbcnt to count the ones below and one counter update per digit group
//    (one LDS write per distinct digit, so skewed inputs cost less);
//  * one upsweep block per CU counts every pass's digits into LDS
//    sub-histograms laid out so that the lanes of an access hit distinct
//    banks;
//  * the tile is re-laid out in LDS in digit order so that each digit's run
//    is written to HBM with consecutive addresses;
//  * tile ids come from one atomic counter per XCD group, each handing out
//    its interleaved chunks of consecutive tiles in order, so a tile only
//    waits on smaller tiles, which blocks of their groups take in turn
//    (next_chunked_tile states the residency this needs); state words are
//    read and written at agent scope because tiles on different XCDs sit
//    behind different L2s;
//  * every key type and direction is a sign-dependent XOR of the key's words
//    (KeyXform), applied on the first pass's load and undone on the last
//    pass's store; the passes in between move the transformed patterns
//    ("第10章 并行模式：排序", 八、习题: the float, descending and 64-bit
//    exercises);
//  * 64-bit keys take the same pass kernel with two words per key (8-byte
//    loads, LDS slots and stores); a two-key sort reads the major and minor
//    keys from two arrays in its first pass and writes them back to two
//    arrays in its last, with 64-bit keys in between (the multi-key exercise:
//    a stable LSD over the concatenated key).
#include "device_common.hpp"
#include "internal.hpp"

namespace rs {

namespace {

// Shapes of the one-sweep pass (threads per block x keys per thread).
// Every shape allows 4 waves per SIMD, i.e. 128 registers per lane: one
// 1024-thread block or two 512-thread blocks per CU.
constexpr int kPassWavesPerSimd = 4;
// Small sorts: 1024 x 16.
constexpr int kSortBlock = 1024;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortBlock * kSortItems;
// Passes of at most this many tiles (of the 1024-thread shapes) use the wide
// look-back: every earlier tile's count is read at once, in batches of
// kWideBatch per thread, instead of a walk one batch of tiles at a time.
constexpr uint32_t kWideMaxTiles = 256;
constexpr int kWideBatch = 8;
// The hybrid sort's top-digit pass: 8192-key tiles while they are at most
// kWideMaxTiles, so a small input spreads over twice as many CUs as with the
// 16384-key shape (measured faster at 2^20 pairs; 4096-key tiles were slower,
// their wide look-backs being longer); 16384-key tiles above that.
constexpr int kMsdItems = 8;
constexpr int kMsdTile = kSortBlock * kMsdItems;
// Large pair sorts: bigger tiles cut the per-tile work (scans, look-back,
// tile hand-out) per key.  24 keys and values per thread from the size that
// gives every CU a tile; 28 (32 spills) once there are at least 2^26 keys,
// below which the last round of tiles leaves too many CUs idle.
constexpr int kPairsBlock = 1024;
constexpr int kPairsItems = 24;
constexpr uint64_t kPairsLargeMinN = 256ull * kPairsBlock * kPairsItems;
constexpr int kPairsHugeItems = 28;
constexpr uint64_t kPairsHugeMinN = 1ull << 26;
// Large keys-only sorts: 32 keys per thread fit without values, and two
// 512-thread blocks share a CU, so one block ranks while the other waits on
// memory or on the look-back; used once every block (two per CU) has a tile.
constexpr int kKeysBlock = 512;
constexpr int kKeysItems = 32;
constexpr uint64_t kKeysLargeMinN = 512ull * kKeysBlock * kKeysItems;
// From 2^27 keys (16 tiles per CU) one 1024 x 32 block per CU is faster:
// half as many tiles in flight shorten every look-back walk.
constexpr int kKeysHugeBlock = 1024;
constexpr uint64_t kKeysHugeMinN = 1ull << 27;
// Up to this many keys the whole sort runs in one block, in LDS.
constexpr uint32_t kTileSortMax = 16384;
// Hybrid sorts of up to kHybridMaxN 4-byte keys: one pass on the top digit
// (MSD), then one workgroup per bucket sorts the lower digits in LDS, when
// no bucket holds more than kBucketCap keys (otherwise the LSD passes run).
constexpr uint32_t kHybridMaxN = 3u << 20;
constexpr int kBucketBlock = 1024;
constexpr int kBucketItems = 16;
constexpr uint32_t kBucketCap = kBucketBlock * kBucketItems;
static_assert(kHybridMaxN / kSortTile <= kWideMaxTiles, "the multi-pass fallback uses the wide look-back");
// Earlier tiles read per look-back batch.  A wave waits for every word of a
// batch that any of its lanes still needs, so small batches win: 2 measured
// best for the 16384-key tiles (8 is 2-4 % slower), 1 for the 24576-key pair
// tiles (1 % faster than 2 there, 1-2 % slower elsewhere).
constexpr int kSortLookback = 2;
constexpr int kPairsLookback = 1;
constexpr int kGroups = 8;             // XCDs
// Cache-policy operand of a buffer access: the non-temporal bit.
constexpr int kNonTemporal = 2;

constexpr int kUpBlock = 1024;   // many waves per CU hide the LDS atomics' latency
// Sub-histograms per digit, indexed by lane mod 32 and stored innermost, so
// the 32 lanes an LDS access serves together hit 32 different banks whatever
// their digits (128 KB for four passes: one block per CU).  8 sub-histograms
// (bank = lane mod 8 and two digit bits) took 14 % longer at 2^28 keys.
constexpr int kUpSub = 32;
constexpr int kMaxPasses = 4;        // 8-bit passes of a 32-bit key
constexpr int kMaxPasses64 = 8;      // ... of a 64-bit key
// 64-bit keys: eight passes' counts with 16 sub-histograms per digit (128 KB).
constexpr int kUpSub64 = 16;
// 64-bit keys: 1024 x 16 tiles (16384 keys, 128 KB of 8-byte LDS slots).
constexpr int kKey64Block = 1024;
constexpr int kKey64Items = 16;

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
    uint32_t shift[kMaxPasses64];
    uint32_t mask[kMaxPasses64];
    uint32_t width[kMaxPasses64];
    uint32_t passes;
    KeyXform xf;   // applied to each key before its digits are counted (XF kernels)
};

// PASSES digits of one key counted (one bit-field extract each; the pass
// count is a template argument, so no per-digit branch).
template <bool XF, int PASSES>
__device__ __forceinline__ void count_key(uint32_t* s_hist, uint32_t key, const PassDigits& pd,
                                          uint32_t sub) {
    if (XF) key = xform32(key, pd.xf);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const uint32_t d = __builtin_amdgcn_ubfe(key, pd.shift[p], pd.width[p]);
        atomicAdd(&s_hist[(p * kRadix + d) * kUpSub + sub], 1u);
    }
}

template <bool XF, int PASSES>
__device__ __forceinline__ void count_rows4(uint32_t* s_hist, const u32x4 (&q)[4], const PassDigits& pd,
                                            uint32_t sub) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        count_key<XF, PASSES>(s_hist, q[u].x, pd, sub);
        count_key<XF, PASSES>(s_hist, q[u].y, pd, sub);
        count_key<XF, PASSES>(s_hist, q[u].z, pd, sub);
        count_key<XF, PASSES>(s_hist, q[u].w, pd, sub);
    }
}

template <bool XF, int PASSES>
__global__ __launch_bounds__(kUpBlock) void upsweep_kernel(const uint32_t* __restrict__ keys,
                                                           uint32_t n, PassDigits pd,
                                                           uint32_t* __restrict__ bins) {
    __shared__ uint32_t s_hist[kMaxPasses * kRadix * kUpSub];
    for (int i = threadIdx.x; i < kMaxPasses * kRadix * kUpSub; i += kUpBlock) s_hist[i] = 0u;
    __syncthreads();

    // Each block reads one contiguous chunk of whole 16-byte vectors, four
    // rows of kUpBlock vectors at a time, with non-temporal loads (the keys
    // are not read again before the first pass evicts them anyway).
    const uint32_t sub = threadIdx.x % kUpSub;
    const uint32_t nvec = n / 4;
    const uint32_t per_block = (nvec + gridDim.x - 1) / gridDim.x;
    const uint32_t begin = blockIdx.x * per_block;
    const uint32_t end = (begin + per_block < nvec) ? begin + per_block : nvec;
    const u32x4* k4 = reinterpret_cast<const u32x4*>(keys);
    uint32_t i = begin + threadIdx.x;
    for (; i + 3 * kUpBlock < end; i += 4 * kUpBlock) {
        u32x4 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = __builtin_nontemporal_load(&k4[i + u * kUpBlock]);
        count_rows4<XF, PASSES>(s_hist, q, pd, sub);
    }
    for (; i < end; i += kUpBlock) {
        const u32x4 v = __builtin_nontemporal_load(&k4[i]);
        count_key<XF, PASSES>(s_hist, v.x, pd, sub);
        count_key<XF, PASSES>(s_hist, v.y, pd, sub);
        count_key<XF, PASSES>(s_hist, v.z, pd, sub);
        count_key<XF, PASSES>(s_hist, v.w, pd, sub);
    }
    if (blockIdx.x == 0 && threadIdx.x < n - nvec * 4)
        count_key<XF, PASSES>(s_hist, keys[nvec * 4 + threadIdx.x], pd, sub);
    __syncthreads();

    // Thread i sums bin i's sub-histograms starting at sub i mod 32, so the
    // lanes of one read hit different banks.
    for (uint32_t i = threadIdx.x; i < PASSES * kRadix; i += kUpBlock) {
        uint32_t c = 0;
#pragma unroll
        for (int s = 0; s < kUpSub; ++s) c += s_hist[i * kUpSub + ((i + s) % kUpSub)];
        if (c) fetch_add_agent(&bins[i], c);
    }
}

// Upsweep of 64-bit keys: up to eight passes' counts in one read.  The keys
// are one array of 8-byte keys, or (SOA) a low-word and a high-word array.
template <bool XF>
__device__ __forceinline__ void count_key64(uint32_t* s_hist, uint64_t key, const PassDigits& pd,
                                            uint32_t sub) {
    if (XF) key = xform64(key, pd.xf);
#pragma unroll
    for (int p = 0; p < kMaxPasses64; ++p) {
        if (p < static_cast<int>(pd.passes)) {
            const uint32_t d = static_cast<uint32_t>(key >> pd.shift[p]) & pd.mask[p];
            atomicAdd(&s_hist[(p * kRadix + d) * kUpSub64 + sub], 1u);
        }
    }
}

template <bool XF, bool SOA>
__global__ __launch_bounds__(kUpBlock) void upsweep64_kernel(const uint32_t* __restrict__ keys,
                                                             const uint32_t* __restrict__ keys_hi,
                                                             uint32_t n, PassDigits pd,
                                                             uint32_t* __restrict__ bins) {
    __shared__ uint32_t s_hist[kMaxPasses64 * kRadix * kUpSub64];
    for (int i = threadIdx.x; i < kMaxPasses64 * kRadix * kUpSub64; i += kUpBlock) s_hist[i] = 0u;
    __syncthreads();

    // one contiguous chunk of 16-byte vectors per block: two 8-byte keys per
    // vector, or four low words and four high words
    constexpr uint32_t PER_VEC = SOA ? 4u : 2u;
    const uint32_t sub = threadIdx.x % kUpSub64;
    const uint32_t nvec = n / PER_VEC;
    const uint32_t per_block = (nvec + gridDim.x - 1) / gridDim.x;
    const uint32_t begin = blockIdx.x * per_block;
    const uint32_t end = (begin + per_block < nvec) ? begin + per_block : nvec;
    const u32x4* k4 = reinterpret_cast<const u32x4*>(keys);
    const u32x4* h4 = reinterpret_cast<const u32x4*>(keys_hi);
    auto count_vec = [&](const u32x4& q, const u32x4& h) {
        if (SOA) {
            count_key64<XF>(s_hist, (static_cast<uint64_t>(h.x) << 32) | q.x, pd, sub);
            count_key64<XF>(s_hist, (static_cast<uint64_t>(h.y) << 32) | q.y, pd, sub);
            count_key64<XF>(s_hist, (static_cast<uint64_t>(h.z) << 32) | q.z, pd, sub);
            count_key64<XF>(s_hist, (static_cast<uint64_t>(h.w) << 32) | q.w, pd, sub);
        } else {
            count_key64<XF>(s_hist, (static_cast<uint64_t>(q.y) << 32) | q.x, pd, sub);
            count_key64<XF>(s_hist, (static_cast<uint64_t>(q.w) << 32) | q.z, pd, sub);
        }
    };
    // four rows of kUpBlock vectors in flight at a time, as the 4-byte upsweep
    uint32_t i = begin + threadIdx.x;
    for (; i + 3 * kUpBlock < end; i += 4 * kUpBlock) {
        u32x4 q[4], h[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            q[u] = __builtin_nontemporal_load(&k4[i + u * kUpBlock]);
            h[u] = SOA ? __builtin_nontemporal_load(&h4[i + u * kUpBlock]) : q[u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) count_vec(q[u], h[u]);
    }
    for (; i < end; i += kUpBlock) {
        const u32x4 q = __builtin_nontemporal_load(&k4[i]);
        count_vec(q, SOA ? __builtin_nontemporal_load(&h4[i]) : q);
    }
    if (blockIdx.x == 0 && threadIdx.x < n - nvec * PER_VEC) {
        const uint32_t j = nvec * PER_VEC + threadIdx.x;
        const uint64_t key = SOA ? (static_cast<uint64_t>(keys_hi[j]) << 32) | keys[j]
                                 : (static_cast<uint64_t>(keys[2 * j + 1]) << 32) | keys[2 * j];
        count_key64<XF>(s_hist, key, pd, sub);
    }
    __syncthreads();

    for (uint32_t i = threadIdx.x; i < pd.passes * kRadix; i += kUpBlock) {
        uint32_t c = 0;
#pragma unroll
        for (int s = 0; s < kUpSub64; ++s) c += s_hist[i * kUpSub64 + ((i + s) % kUpSub64)];
        if (c) fetch_add_agent(&bins[i], c);
    }
}

// ---------------------------------------------------------------------------
// One-sweep pass: stable scatter of one 8-bit digit.
// ---------------------------------------------------------------------------

// Lanes of the wave whose digit differs from this lane's (eight ballots).  For
// each bit, m is 0 or all ones (the bit sign-extended) and the ballot marks
// the lanes whose bit is set; lanes that differ from this one in that bit are
// vote ^ m.  The sets are OR-ed with one 3-input logic op per half (truth
// table A | (B ^ C) = 0xF6 in the A=0xF0, B=0xCC, C=0xAA convention).  The
// ballot is taken from m itself (one compare) through a small asm statement,
// which keeps the compiler from re-deriving the bit with a shift first.
__device__ __forceinline__ uint64_t lanes_with_other_digit(uint32_t d) {
    uint32_t diff_lo = 0u, diff_hi = 0u;
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
        const uint32_t m = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(d), b, 1));
        uint64_t vote;
        asm volatile("v_cmp_ne_u32_e64 %0, 0, %1" : "=s"(vote) : "v"(m));
        diff_lo = __builtin_amdgcn_bitop3_b32(diff_lo, static_cast<uint32_t>(vote), m, 0xF6);
        diff_hi = __builtin_amdgcn_bitop3_b32(diff_hi, static_cast<uint32_t>(vote >> 32), m, 0xF6);
    }
    return (static_cast<uint64_t>(diff_hi) << 32) | diff_lo;
}

// Ballot rank of one row: the wave's running count of digit d plus the lanes
// below this one that hold the same digit; the lowest lane of each digit group
// advances the wave's counter by the group's size.  LDS instructions of one
// wave execute in order, so the next row reads the advanced counters.
__device__ __forceinline__ uint32_t ballot_rank(uint32_t* my_count, uint32_t d, uint32_t lane) {
    const uint32_t before = my_count[d];
    const uint64_t others = lanes_with_other_digit(d);
    const uint32_t below = lane - count_below(others);      // same digit, lower lane
    const uint32_t group_size = kWave - static_cast<uint32_t>(__popcll(others));
    if (below == 0) my_count[d] = before + group_size;
    return before + below;
}

// Arguments of one digit pass.  Keys are u32 words, or 8-byte keys (two
// words, low first) for the 64-bit kernels; with soa_in (soa_out) the 64-bit
// keys are read from (written to) a low-word array src_keys (dst_keys) and a
// high-word array src_hi (dst_hi).
struct PassArgs {
    const uint32_t* src_keys;
    uint32_t* dst_keys;
    const uint32_t* src_vals;
    uint32_t* dst_vals;
    const uint32_t* src_hi;
    uint32_t* dst_hi;
    uint32_t soa_in, soa_out;
    KeyXform xin;              // applied to the keys as loaded (XF_IN kernels)
    KeyXform xout;             // applied to the keys as stored (XF_OUT kernels)
    uint32_t n, tiles, shift, width;   // digit = bits [shift, shift + width) of the key
    const uint32_t* bins;      // global digit counts of this pass
    uint32_t* states;          // look-back words of this pass, zeroed
    uint32_t* next_states;     // look-back words of the next pass, cleared here (or null)
    uint32_t* sched;           // tile counters of this pass (one per group), zeroed
    uint32_t groups;           // block groups = min(8, grid)
    uint32_t chunk_log2;       // tiles per chunk = 2^chunk_log2 (at most the blocks per group)
    uint32_t atomic_limit_log2;   // atomic rank while no digit holds more than 2^-this of the keys
    // Launch gate of the hybrid sort: 0 runs always; 1 runs only when no
    // count of gate_bins[0..255] exceeds gate_cap, 2 only when one does.
    uint32_t gate, gate_cap;
    const uint32_t* gate_bins;
    // Multi-pass launch (MULTI kernels: the hybrid sort's LSD fallback):
    // every pass of the sort in one launch.  Tiles are handed out in (pass,
    // tile) order from multi_counter[0]; multi_counter[1 + p] counts the
    // finished tiles of pass p, and a tile of pass p > 0 starts only when
    // every tile of pass p - 1 has finished.  Pass p reads m[p].src_*, writes
    // m[p].dst_*, uses bins + 256 p and the zeroed states m_states + p *
    // tiles * 256.
    uint32_t multi_passes;
    uint32_t* multi_counter;
    uint32_t* m_states;
    struct PassIo {
        const uint32_t* src_keys;
        uint32_t* dst_keys;
        const uint32_t* src_vals;
        uint32_t* dst_vals;
        uint32_t shift, width;
    } m[kMaxPasses];
};

// Loads the ITEMS keys of this lane for `tile`: row j of wave w is the 64
// consecutive keys at tile*TILE + w*64*ITEMS + j*64.  The loads go through a
// buffer descriptor of n elements, so a row past the end of a partial tile
// reads 0 without a branch or a clamp (the padding is applied afterwards;
// where the tile reaches past 2^30 keys such a row's byte offset wraps round
// 2^32 and reads keys from the start of the same buffer, which are replaced
// by the padding and never stored); they are non-temporal, since each key is
// read once per pass.  The row offsets fold into the instructions'
// immediate offsets.
template <int ITEMS, int TILE>
__device__ __forceinline__ void load_rows(const uint32_t* __restrict__ src, uint32_t tile,
                                          uint32_t n, uint32_t wave, uint32_t lane,
                                          uint32_t (&x)[ITEMS]) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(src), 0, static_cast<int>(n * 4u), kBufferWord3);
    const uint32_t first = (tile * TILE + wave * (kWave * ITEMS) + lane) * 4u;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
        x[j] = __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(first + j * kWave * 4), 0,
                                                    kNonTemporal);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The same rows of 8-byte keys: one 8-byte load per lane and row (a row is
// 512 consecutive bytes); n < 2^29 keeps every byte offset of the array
// below 2^32.
template <int ITEMS, int TILE>
__device__ __forceinline__ void load_rows64(const uint32_t* __restrict__ src, uint32_t tile,
                                            uint32_t n, uint32_t wave, uint32_t lane,
                                            uint64_t (&x)[ITEMS]) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(src), 0, static_cast<int>(n * 8u), kBufferWord3);
    const uint32_t first = (tile * TILE + wave * (kWave * ITEMS) + lane) * 8u;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(
            r, static_cast<int>(first + j * kWave * 8), 0, kNonTemporal);
        x[j] = (static_cast<uint64_t>(w.y) << 32) | w.x;
    }
}

// Digit of a key: bits [shift, shift + width) (a 64-bit key may straddle its words).
__device__ __forceinline__ uint32_t digit_of(uint32_t k, uint32_t shift, uint32_t width) {
    return __builtin_amdgcn_ubfe(k, shift, width);
}
__device__ __forceinline__ uint32_t digit_of(uint64_t k, uint32_t shift, uint32_t width) {
    return __builtin_amdgcn_ubfe(static_cast<uint32_t>(k >> shift), 0, width);
}

// One-sweep pass over one 8-bit digit.  Persistent: each block loops over the
// tiles the scheduler hands it.  Per tile: load, stable in-wave rank (LDS
// atomics or ballots), tile counts and scans, decoupled look-back, re-layout
// in digit order in LDS, scatter of each digit run.
// WIDE (passes of few tiles, 1024 threads): a tile publishes only its own
// counts, and its exclusive prefix is the sum of the counts of all earlier
// tiles, read by four threads per digit in parallel.  When a pass's tiles
// all start together (a small input), a walk that stops at the nearest
// published prefix can take up to about tile/4 dependent round trips for the
// last tiles, while the reads here are independent.  (At 64 tiles both forms
// measured the same; the wide one is what lets the hybrid sort's top-digit
// pass use 128 tiles of 8192 keys.)
template <int BLOCK, int ITEMS, int LOOKBACK, bool PAIRS, bool XF_IN, bool XF_OUT, bool KEY64,
          bool MULTI = false, bool WIDE = false>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(kPassWavesPerSimd)))
void onesweep_kernel(PassArgs a) {
    using Key = typename std::conditional<KEY64, uint64_t, uint32_t>::type;
    constexpr int WAVES = BLOCK / kWave;
    constexpr int TILE = BLOCK * ITEMS;
    constexpr int WAVE_KEYS = kWave * ITEMS;
    static_assert(BLOCK >= kRadix && BLOCK % kWave == 0, "one thread per digit needed");
    static_assert(TILE <= 32768, "16-bit positions");
    static_assert(ITEMS % 4 == 0, "digits are packed four per register");
    static_assert(!WIDE || BLOCK == 4 * kRadix, "the wide look-back uses four threads per digit");

    // One staging buffer: the keys in digit order, then the values in digit order.
    __shared__ Key s_buf[TILE];
    uint32_t* const s_vbuf = reinterpret_cast<uint32_t*>(s_buf);
    __shared__ uint32_t s_off[WAVES * kRadix];   // per-wave digit counters, then offsets
    __shared__ uint32_t s_adjust[kRadix];
    __shared__ uint32_t s_wsum[2][kRadix / kWave];
    __shared__ uint32_t s_next;
    __shared__ uint32_t s_crowded;   // a digit of this tile holds too many of its keys
    __shared__ uint32_t s_part[WIDE ? 3 * kRadix : 1];   // wide look-back: partial sums of threads 256..1023

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;
    // (the per-pass values below change between passes only in MULTI kernels)
    const uint32_t* __restrict__ src_keys = a.src_keys;
    uint32_t* __restrict__ dst_keys = a.dst_keys;
    const uint32_t* __restrict__ src_vals = a.src_vals;
    uint32_t* __restrict__ dst_vals = a.dst_vals;
    uint32_t* __restrict__ states = a.states;
    const uint32_t n = a.n, tiles = a.tiles;
    uint32_t shift = a.shift, width = a.width;
    uint32_t last_digit = (1u << width) - 1u;
    const uint32_t group = blockIdx.x % a.groups;
    uint32_t cur_pass = 0;
    bool xf_in = XF_IN, xf_out = XF_OUT;   // uniform
    if constexpr (MULTI) {
        src_keys = a.m[0].src_keys;
        dst_keys = a.m[0].dst_keys;
        src_vals = a.m[0].src_vals;
        dst_vals = a.m[0].dst_vals;
        states = a.m_states;
        shift = a.m[0].shift;
        width = a.m[0].width;
        last_digit = (1u << width) - 1u;
        xf_out = XF_OUT && a.multi_passes == 1;
    }

    // The first tile is taken while the counts load (a small sort's block
    // often has only this tile); a launch the gate stops leaves its counter
    // unused.
    if (tid == 0) {
        if constexpr (MULTI) s_next = fetch_add_agent(&a.multi_counter[0], 1u);
        else s_next = next_chunked_tile(a.sched, a.groups, a.chunk_log2, group, tiles);
    }
    // global digit count of this pass (thread d holds digit d), in flight
    // together with the gate's counts
    uint32_t bin = (tid < kRadix) ? a.bins[tid] : 0u;
    if (a.gate != 0) {   // uniform: a gated launch of the hybrid sort
        const uint32_t c = (tid < kRadix) ? a.gate_bins[tid] : 0u;
        const bool oversize = __syncthreads_or(c > a.gate_cap);
        if (oversize != (a.gate == 2)) return;
    }
    // Same-address LDS atomics serialise, so the atomic rank below is used
    // while no digit holds more than a share 2^-atomic_limit_log2 of the
    // pass's keys, and for a tile only if the block's previous tile had no
    // digit over that share of its keys (earlier passes gather equal keys
    // into runs, which then collide within a row); otherwise the ballot rank.
#ifdef RS_FORCE_BALLOT_RANK
    bool spread = false;   // build switch: ballot rank on every tile
#else
    bool spread = !__syncthreads_or((static_cast<uint64_t>(bin) << a.atomic_limit_log2) > n);
#endif
    bool atomic_rank = spread;   // uniform

    for (bool first_tile = true;; first_tile = false) {
        // After the first, a tile is taken only when the block can start on it
        // at once: the time from taking a tile to publishing its count delays
        // every later tile's look-back.
        if (tid == 0) {
            if (!first_tile) {
                if constexpr (MULTI) s_next = fetch_add_agent(&a.multi_counter[0], 1u);
                else s_next = next_chunked_tile(a.sched, a.groups, a.chunk_log2, group, tiles);
            }
            s_crowded = 0u;   // the previous tile's readers all passed a barrier since
        }
        // Only this wave reads and writes its counters during the rank, and the
        // previous tile's readers of s_off all passed a barrier since.
        for (uint32_t i = lane; i < kRadix; i += kWave) s_off[wave * kRadix + i] = 0u;
        __syncthreads();
        uint32_t tile = s_next;
        if constexpr (MULTI) {
            if (tile >= tiles * a.multi_passes) break;   // uniform: no tiles left
            const uint32_t p = tile / tiles;
            tile -= p * tiles;
            if (p != cur_pass) {   // uniform; a block's passes only increase
                // Every tile of pass p - 1 has been handed out (smaller ids) to
                // running blocks; wait until all of them have finished, then
                // take their stores in (agent-scope acquire after their release).
                if (tid == 0) {
                    while (load_state(&a.multi_counter[p]) < tiles) __builtin_amdgcn_s_sleep(2);
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                }
                cur_pass = p;
                src_keys = a.m[p].src_keys;
                dst_keys = a.m[p].dst_keys;
                src_vals = a.m[p].src_vals;
                dst_vals = a.m[p].dst_vals;
                states = a.m_states + static_cast<size_t>(p) * tiles * kRadix;
                shift = a.m[p].shift;
                width = a.m[p].width;
                last_digit = (1u << width) - 1u;
                xf_in = false;
                xf_out = XF_OUT && p + 1 == a.multi_passes;
                bin = (tid < kRadix) ? a.bins[p * kRadix + tid] : 0u;
#ifdef RS_FORCE_BALLOT_RANK
                spread = false;
                __syncthreads();
#else
                spread = !__syncthreads_or((static_cast<uint64_t>(bin) << 4) > n);
#endif
                atomic_rank = spread;
            }
        } else {
            if (tile >= tiles) break;   // uniform: no tiles left
        }
        Key k[ITEMS];
        if constexpr (KEY64) {
            if (a.soa_in) {
                uint32_t lo[ITEMS], hi[ITEMS];
                load_rows<ITEMS, TILE>(src_keys, tile, n, wave, lane, lo);
                load_rows<ITEMS, TILE>(a.src_hi, tile, n, wave, lane, hi);
#pragma unroll
                for (int j = 0; j < ITEMS; ++j) k[j] = (static_cast<uint64_t>(hi[j]) << 32) | lo[j];
            } else {
                load_rows64<ITEMS, TILE>(src_keys, tile, n, wave, lane, k);
            }
        } else {
            load_rows<ITEMS, TILE>(src_keys, tile, n, wave, lane, k);
        }
        const uint32_t tile_base = tile * TILE;
        const uint32_t valid = (n - tile_base < static_cast<uint32_t>(TILE)) ? n - tile_base : TILE;
        const bool full = (valid == static_cast<uint32_t>(TILE));
        const uint32_t first = tile_base + wave * WAVE_KEYS + lane;
        if (XF_IN && xf_in) {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                if constexpr (KEY64) k[j] = xform64(k[j], a.xin);
                else k[j] = xform32(k[j], a.xin);
            }
        }
        if (!full) {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j)
                if (first + j * kWave >= n) k[j] = ~static_cast<Key>(0);   // padding sorts last
        }

        // ---- stable rank inside the wave --------------------------------------
        // rank in the wave, later the position in the tile: 16 bits, two per register
        uint32_t pos[ITEMS / 2];
        uint32_t* my_count = s_off + wave * kRadix;
        if (atomic_rank) {
            // Atomic rank: one LDS atomic add per key on the wave's digit
            // counter.  On gfx950 the lanes of one ds_add_rtn_u32 that hit the
            // same address are served in lane order, so each lane gets the
            // counter plus the lanes below it with the same digit: the stable
            // rank.  This is observed behaviour, which a GPU test of the
            // hardware checks directly and every parity test depends on.
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const uint32_t d = digit_of(k[j], shift, width);
                const uint32_t slot = atomicAdd(&my_count[d], 1u);   // served in lane order
                if (j % 2 == 0) pos[j / 2] = slot;
                else pos[j / 2] |= slot << 16;
            }
        } else {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const uint32_t d = digit_of(k[j], shift, width);
                const uint32_t slot = ballot_rank(my_count, d, lane);
                if (j % 2 == 0) pos[j / 2] = slot;
                else pos[j / 2] |= slot << 16;
                // the slots are chained through the LDS counters anyway; keeping the
                // scheduler from interleaving them keeps register pressure low
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();

        // ---- per digit: offsets of each wave, tile count, scans -------------
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
        const uint32_t pads = static_cast<uint32_t>(TILE) - valid;
        const uint32_t real = (tid == last_digit) ? count - pads : count;
        if (tid < kRadix)
            store_state(&states[tile * kRadix + tid],
                        (tile == 0 && !WIDE ? kStatePrefix : kStateAggregate) | real);

        uint32_t inc_c = 0, inc_b = 0;
        if (tid < kRadix) {
            inc_c = PAIRS ? wave_inclusive_sum_shfl(count) : wave_inclusive_sum(count);
            inc_b = PAIRS ? wave_inclusive_sum_shfl(bin) : wave_inclusive_sum(bin);
            if (lane == kWave - 1) {
                s_wsum[0][wave] = inc_c;
                s_wsum[1][wave] = inc_b;
            }
        }
        if (tid < kRadix && (count << a.atomic_limit_log2) > static_cast<uint32_t>(TILE)) s_crowded = 1u;
        __syncthreads();
        atomic_rank = spread && s_crowded == 0u;   // for the next tile
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

        // First look-back batch: the states of this digit in the LOOKBACK tiles
        // before this one, loaded together so their latencies overlap each
        // other and the work below.
        uint32_t lb[LOOKBACK];
        // Wide look-back: thread (q, d) = (tid / 256, tid % 256) sums digit d's
        // counts of the tiles q, q + 4, q + 8, ... below this one, kWideBatch
        // of them per batch of loads; the first batch is in flight during the
        // re-layout.
        const uint32_t wd = tid % kRadix, wq = tid / kRadix;
        uint32_t wl[WIDE ? kWideBatch : 1];
        if constexpr (WIDE) {
#pragma unroll
            for (int b = 0; b < kWideBatch; ++b) {
                const uint32_t t = wq + 4u * b;
                wl[b] = (t < tile) ? load_state(&states[t * kRadix + wd]) : kStateAggregate;
            }
        }
        if (!WIDE && tid < kRadix && tile > 0) {
#pragma unroll
            for (int b = 0; b < LOOKBACK; ++b) {
                const int32_t t = static_cast<int32_t>(tile) - 1 - b;
                lb[b] = (t >= 0) ? load_state(&states[static_cast<uint32_t>(t) * kRadix + tid]) : 0u;
            }
        }

        // The values are loaded now; their latency overlaps the re-layout of
        // the keys and the look-back, and they do not hold registers during
        // the rank.
        uint32_t v[PAIRS ? ITEMS : 1];
        if constexpr (PAIRS) load_rows<ITEMS, TILE>(src_vals, tile, n, wave, lane, v);

        // ---- re-lay the keys out in digit order in LDS ---------------------------
        // Keys-only passes go in groups of RG rows: the group's digit-offset
        // reads are issued together, then its stores, so the reads' LDS
        // latencies overlap instead of each store waiting on its own read
        // (2^28 keys-only pass 0.501 -> 0.488 ms; pair passes, whose tiles
        // wait on memory, gained nothing and keep one row at a time).
        constexpr int RG = PAIRS ? 1 : (ITEMS % 8 == 0 ? 8 : 4);
#pragma unroll
        for (int g = 0; g < ITEMS; g += RG) {
            Key key[RG];
            uint32_t base[RG];
#pragma unroll
            for (int i = 0; i < RG; ++i) {
                // recompute the digit rather than keep the rank loop's LDS addresses
                // alive across the scans (an empty asm hides the reuse)
                key[i] = k[g + i];
                asm volatile("" : "+v"(key[i]));
                base[i] = s_off[wave * kRadix + digit_of(key[i], shift, width)];
            }
#pragma unroll
            for (int i = 0; i < RG; ++i) {
                const int j = g + i;
                // (the clamp never changes a consistent position; it keeps the store in the tile)
                const uint32_t sh = 16 * (j % 2);
                const uint32_t p = min(base[i] + ((pos[j / 2] >> sh) & 0xFFFFu), static_cast<uint32_t>(TILE - 1));
                pos[j / 2] = (pos[j / 2] & ~(0xFFFFu << sh)) | (p << sh);
                s_buf[p] = key[i];
            }
        }

        // ---- decoupled look-back: same-digit keys in all earlier tiles --------
        // Walk from the nearest earlier tile down, adding published tile counts
        // until the first published inclusive prefix; states are read in
        // batches of LOOKBACK tiles.  Tile 0 always publishes a prefix, so the
        // walk ends at tile 0 at the latest and never reads below it.
        if constexpr (WIDE) {
            // every earlier tile publishes its counts right after its rank,
            // which waits on nothing, and is taken by a running block
            // eventually (the scheduler's progress argument), so no wait here
            // is forever
            uint32_t part = 0;
            for (uint32_t first_t = wq;; first_t += 4u * kWideBatch) {
#pragma unroll
                for (int b = 0; b < kWideBatch; ++b) {
                    const uint32_t t = first_t + 4u * b;
                    uint32_t st = wl[b];
                    while ((st & ~kStateCountMask) == 0u) {   // (t < tile here: others hold a flag)
                        __builtin_amdgcn_s_sleep(1);
                        st = load_state(&states[t * kRadix + wd]);
                    }
                    if (t < tile) part += st & kStateCountMask;
                }
                const uint32_t next_t = first_t + 4u * kWideBatch;
                if (next_t >= tile) break;
#pragma unroll
                for (int b = 0; b < kWideBatch; ++b) {
                    const uint32_t t = next_t + 4u * b;
                    wl[b] = (t < tile) ? load_state(&states[t * kRadix + wd]) : kStateAggregate;
                }
            }
            if (wq > 0) s_part[(wq - 1) * kRadix + wd] = part;
            __syncthreads();
            if (tid < kRadix) {
                const uint32_t excl = part + s_part[tid] + s_part[kRadix + tid] + s_part[2 * kRadix + tid];
                s_adjust[tid] = bin_start + excl - local_start;
                if (a.next_states) a.next_states[tile * kRadix + tid] = 0u;
            }
        } else if (tid < kRadix) {
            uint32_t excl = 0;
            if (tile > 0) {
                int32_t nearest = static_cast<int32_t>(tile) - 1;   // tile of lb[0]
                bool done = false;
                for (;;) {
#pragma unroll
                    for (int b = 0; b < LOOKBACK; ++b) {
                        if (!done) {
                            const uint32_t t = static_cast<uint32_t>(nearest - b);
                            uint32_t st = lb[b];
                            while ((st & ~kStateCountMask) == 0u) {
                                __builtin_amdgcn_s_sleep(1);
                                st = load_state(&states[t * kRadix + tid]);
                            }
                            excl += st & kStateCountMask;
                            done = (st & kStatePrefix) != 0u;
                        }
                    }
                    if (done) break;
                    nearest -= LOOKBACK;
#pragma unroll
                    for (int b = 0; b < LOOKBACK; ++b) {
                        const int32_t t = nearest - b;
                        lb[b] = (t >= 0) ? load_state(&states[static_cast<uint32_t>(t) * kRadix + tid])
                                         : 0u;
                    }
                }
                store_state(&states[tile * kRadix + tid], kStatePrefix | (excl + real));
            }
            s_adjust[tid] = bin_start + excl - local_start;
            if (a.next_states) a.next_states[tile * kRadix + tid] = 0u;
        }
        __syncthreads();

        // ---- scatter each digit run to consecutive addresses ----------------------
        // Slot r of this thread is tile position r * BLOCK + tid; its digit is
        // kept (four per register) for the value scatter.  Stores go through
        // buffer descriptors whose size is n elements: the hardware drops a
        // store past the end, which is where every pad of a partial tile
        // lands (pads rank after the last real key of the last digit, whose
        // run ends at n), so no slot needs a branch and the LDS reads of all
        // slots can be in flight together.  A pad's destination can lie past
        // 2^30, where its byte offset would wrap round 2^32 back into the
        // buffer; it is clamped to n first (n * 4 < 2^32 is out of range).
        const bool soa_out = KEY64 && a.soa_out;   // uniform
        const uint32_t key_bytes = (KEY64 && !soa_out) ? 8u : 4u;
        const __amdgpu_buffer_rsrc_t out_keys = __builtin_amdgcn_make_buffer_rsrc(
            dst_keys, 0, static_cast<int>(n * key_bytes), kBufferWord3);
        const __amdgpu_buffer_rsrc_t out_hi = __builtin_amdgcn_make_buffer_rsrc(
            KEY64 ? a.dst_hi : dst_keys, 0, static_cast<int>(n * 4u), kBufferWord3);
        uint32_t digits[PAIRS ? ITEMS / 4 : 1];
#pragma unroll
        for (int r = 0; r < ITEMS; ++r) {
            const uint32_t i = r * BLOCK + tid;
            Key key = s_buf[i];
            const uint32_t d = digit_of(key, shift, width);
            if (PAIRS) {
                if (r % 4 == 0) digits[r / 4] = d;
                else digits[r / 4] |= d << (8 * (r % 4));
            }
            const uint32_t dst = min(i + s_adjust[d], n);
            if constexpr (KEY64) {
                if (XF_OUT && xf_out) key = xform64(key, a.xout);
                const uint32_t lo = static_cast<uint32_t>(key), hi = static_cast<uint32_t>(key >> 32);
                if (soa_out) {
                    __builtin_amdgcn_raw_buffer_store_b32(lo, out_keys, static_cast<int>(dst * 4u), 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(hi, out_hi, static_cast<int>(dst * 4u), 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, out_keys,
                                                          static_cast<int>(dst * 8u), 0, 0);
                }
            } else {
                __builtin_amdgcn_raw_buffer_store_b32((XF_OUT && xf_out) ? xform32(key, a.xout) : key,
                                                      out_keys, static_cast<int>(dst * 4u), 0, 0);
            }
            if (PAIRS && r % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // bounds live registers
        }
        if (PAIRS) {
            const __amdgpu_buffer_rsrc_t out_vals =
                __builtin_amdgcn_make_buffer_rsrc(dst_vals, 0, static_cast<int>(n * 4u), kBufferWord3);
            __syncthreads();   // every key has been read from the staging buffer
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) s_vbuf[(pos[j / 2] >> (16 * (j % 2))) & 0xFFFFu] = v[j];
            __syncthreads();
#pragma unroll
            for (int r = 0; r < ITEMS; ++r) {
                const uint32_t i = r * BLOCK + tid;
                const uint32_t d = (digits[r / 4] >> (8 * (r % 4))) & 0xFFu;
                const uint32_t dst = min(i + s_adjust[d], n);
                __builtin_amdgcn_raw_buffer_store_b32(s_vbuf[i], out_vals, static_cast<int>(dst * 4u), 0, 0);
            }
        }
        if constexpr (MULTI) {
            // this tile of pass cur_pass is done: every wave's stores have
            // completed, then one agent-scope release makes them visible to
            // the blocks that wait on the pass's count
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                fetch_add_agent(&a.multi_counter[1 + cur_pass], 1u);
            }
        }
        // the next iteration rewrites s_buf and s_adjust only after a barrier
    }
}

// ---------------------------------------------------------------------------
// One-block sort of n <= kTileSortMax keys (and values): every pass runs in
// LDS, with the same stable in-wave rank as the one-sweep pass and no global
// counts, look-back or temp storage.  Pass p re-lays the tile out in the
// order of digit p; that order is pass p + 1's input order, which is the LSD
// recurrence of "WebGPU Unleashed", 4.1 (each pass a stable counting sort).
// Pads (key 0xFFFFFFFF after the order transform) fill the tile past n;
// they carry the last digit of every pass and come after every real key in
// input order, so they stay at positions n.. in every pass and are never
// stored.  XF: keys are transformed on the way in (pd.xf) and back on the way
// out (xout).
// ---------------------------------------------------------------------------
template <int BLOCK, int ITEMS, bool PAIRS, bool XF>
__global__ __launch_bounds__(BLOCK) void tile_sort_kernel(const uint32_t* __restrict__ keys_in,
                                                          uint32_t* __restrict__ keys_out,
                                                          const uint32_t* __restrict__ vals_in,
                                                          uint32_t* __restrict__ vals_out,
                                                          uint32_t n, PassDigits pd, KeyXform xout) {
    constexpr int WAVES = BLOCK / kWave;
    constexpr int TILE = BLOCK * ITEMS;
    constexpr int WAVE_KEYS = kWave * ITEMS;
    static_assert(BLOCK >= kRadix && BLOCK % kWave == 0, "one thread per digit needed");
    static_assert(TILE <= 32768 && ITEMS % 2 == 0, "16-bit positions, two per register");

    // the tile in digit order: keys, or (PAIRS) key and value in one 8-byte
    // word, so each slot takes one LDS write and one read per pass
    __shared__ uint32_t s_keys[PAIRS ? 1 : TILE];
    __shared__ uint64_t s_kv[PAIRS ? TILE : 1];
    __shared__ uint32_t s_off[WAVES * kRadix];   // per-wave digit counters, then offsets
    __shared__ uint32_t s_wsum[kRadix / kWave];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;
    const uint32_t first = wave * WAVE_KEYS + lane;   // row j of this lane: first + 64 j

    uint32_t k[ITEMS];
    uint32_t v[PAIRS ? ITEMS : 1];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t i = first + j * kWave;
        if (i < n) {
            k[j] = XF ? xform32(keys_in[i], pd.xf) : keys_in[i];
            if constexpr (PAIRS) v[j] = vals_in[i];
        } else {
            k[j] = 0xFFFFFFFFu;
            if constexpr (PAIRS) v[j] = 0u;
        }
    }

    for (uint32_t p = 0; p < pd.passes; ++p) {
        const uint32_t shift = pd.shift[p], width = pd.width[p];
        // this wave's counters; their readers in the previous pass all passed a barrier since
        for (uint32_t i = lane; i < kRadix; i += kWave) s_off[wave * kRadix + i] = 0u;

        // Stable rank with one LDS atomic add per key (same-address lanes of
        // one instruction are served in lane order on gfx950, as in the
        // one-sweep pass; at these sizes the serialisation of crowded digits
        // costs little, so no ballot fallback unless the build forces it).
        uint32_t pos[ITEMS / 2];
        uint32_t* my_count = s_off + wave * kRadix;
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t d = __builtin_amdgcn_ubfe(k[j], shift, width);
#ifdef RS_FORCE_BALLOT_RANK
            const uint32_t slot = ballot_rank(my_count, d, lane);
#else
            const uint32_t slot = atomicAdd(&my_count[d], 1u);   // served in lane order
#endif
            if (j % 2 == 0) pos[j / 2] = slot;
            else pos[j / 2] |= slot << 16;
        }
        __syncthreads();

        // per digit: offsets of each wave, then the tile-wide exclusive scan
        uint32_t count = 0;
        if (tid < kRadix) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const uint32_t c = s_off[w * kRadix + tid];
                s_off[w * kRadix + tid] = count;
                count += c;
            }
            const uint32_t inc = wave_inclusive_sum(count);
            if (lane == kWave - 1) s_wsum[wave] = inc;
            count = inc - count;   // exclusive within this wave's 64 digits
        }
        __syncthreads();
        if (tid < kRadix) {
            uint32_t start = count;
#pragma unroll
            for (int w = 0; w < kRadix / kWave; ++w)
                if (w < static_cast<int>(wave)) start += s_wsum[w];
#pragma unroll
            for (int w = 0; w < WAVES; ++w) s_off[w * kRadix + tid] += start;
        }
        __syncthreads();

        // re-lay the tile out in digit order; read it back as the next input order
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t d = __builtin_amdgcn_ubfe(k[j], shift, width);
            const uint32_t q = (s_off[wave * kRadix + d] + ((pos[j / 2] >> (16 * (j % 2))) & 0xFFFFu)) &
                               (TILE - 1);
            if constexpr (PAIRS) s_kv[q] = (static_cast<uint64_t>(v[j]) << 32) | k[j];
            else s_keys[q] = k[j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            if constexpr (PAIRS) {
                const uint64_t kv = s_kv[first + j * kWave];
                k[j] = static_cast<uint32_t>(kv);
                v[j] = static_cast<uint32_t>(kv >> 32);
            } else {
                k[j] = s_keys[first + j * kWave];
            }
        }
        // the next pass writes the staging buffer only after two more barriers
    }

#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t i = first + j * kWave;
        if (i < n) {
            keys_out[i] = XF ? xform32(k[j], xout) : k[j];
            if constexpr (PAIRS) vals_out[i] = v[j];
        }
    }
}

// ---------------------------------------------------------------------------
// Bucket sort of the hybrid path ("第10章 并行模式：排序", 10.5, the mixed
// strategy: a radix pass on the high bits, then a sort of each bucket on
// its own).  The top digit's pass has already placed every key (transformed)
// in its bucket, stably; block b sorts bucket b by the lower digits in LDS
// with the same passes as the one-workgroup sort and writes it to its final
// place.  The bucket's c keys are spread over the 16 waves as rows = ceil(c /
// 1024) rows of 64 per wave, in input order (wave, row, lane); rows past
// that are not touched, and the pads of the last rows (key 0xFFFFFFFF) rank
// after every real key and are never stored.  The launch does nothing when a
// bucket holds more than cap keys (then the LSD passes run instead).
// ---------------------------------------------------------------------------
struct BucketArgs {
    const uint32_t* keys;        // bucketed (transformed) keys
    const uint32_t* vals;
    uint32_t* keys_out;
    uint32_t* vals_out;
    const uint32_t* top_bins;    // key counts of the buckets
    uint32_t cap;
    PassDigits pd;               // the digits below the top one
    KeyXform xout;               // inverse transform on the store (XF_OUT)
};

template <bool PAIRS, bool XF_OUT>
__global__ __launch_bounds__(kBucketBlock) void bucket_sort_kernel(BucketArgs a) {
    constexpr int BLOCK = kBucketBlock;
    constexpr int ITEMS = kBucketItems;
    constexpr int WAVES = BLOCK / kWave;
    constexpr int TILE = BLOCK * ITEMS;
    static_assert((TILE & (TILE - 1)) == 0, "positions are masked to the tile");

    // the tile in digit order: keys, or (PAIRS) key and value in one 8-byte
    // word, so each slot takes one LDS write and one read per pass
    __shared__ uint32_t s_keys[PAIRS ? 1 : TILE];
    __shared__ uint64_t s_kv[PAIRS ? TILE : 1];
    __shared__ uint32_t s_off[WAVES * kRadix];
    __shared__ uint32_t s_wsum[kRadix / kWave];
    __shared__ uint32_t s_count;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;
    const uint32_t b = blockIdx.x;

    // Thread d < 256 holds bucket d's count; one load serves the gate, the
    // bucket's start (the counts of the buckets below b, summed per wave) and
    // its size.
    const uint32_t cd = (tid < kRadix) ? a.top_bins[tid] : 0u;
    const uint32_t below = wave_inclusive_sum(tid < b ? cd : 0u);
    if (wave < kRadix / kWave && lane == kWave - 1) s_wsum[wave] = below;
    if (tid == b) s_count = cd;
    if (__syncthreads_or(cd > a.cap)) return;   // uniform: the LSD passes sort this input
    uint32_t start = 0;
#pragma unroll
    for (int w = 0; w < kRadix / kWave; ++w) start += s_wsum[w];
    const uint32_t c = s_count;
    if (c == 0) return;   // uniform
    const uint32_t rows = (c + BLOCK - 1) / BLOCK;
    const uint32_t first = wave * (kWave * rows) + lane;   // row j of this lane: first + 64 j

    uint32_t k[ITEMS];
    uint32_t v[PAIRS ? ITEMS : 1];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        if (j < static_cast<int>(rows)) {
            const uint32_t i = first + j * kWave;
            if (i < c) {
                k[j] = a.keys[start + i];
                if constexpr (PAIRS) v[j] = a.vals[start + i];
            } else {
                k[j] = 0xFFFFFFFFu;
                if constexpr (PAIRS) v[j] = 0u;
            }
        }
    }

    for (uint32_t p = 0; p < a.pd.passes; ++p) {
        const uint32_t shift = a.pd.shift[p], width = a.pd.width[p];
        for (uint32_t i = lane; i < kRadix; i += kWave) s_off[wave * kRadix + i] = 0u;
        uint32_t pos[ITEMS];
        uint32_t* my_count = s_off + wave * kRadix;
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            if (j < static_cast<int>(rows)) {
                const uint32_t d = __builtin_amdgcn_ubfe(k[j], shift, width);
#ifdef RS_FORCE_BALLOT_RANK
                pos[j] = ballot_rank(my_count, d, lane);
#else
                pos[j] = atomicAdd(&my_count[d], 1u);   // served in lane order
#endif
            }
        }
        __syncthreads();
        uint32_t count = 0;
        if (tid < kRadix) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const uint32_t cw = s_off[w * kRadix + tid];
                s_off[w * kRadix + tid] = count;
                count += cw;
            }
            const uint32_t inc = wave_inclusive_sum(count);
            if (lane == kWave - 1) s_wsum[wave] = inc;
            count = inc - count;
        }
        __syncthreads();
        if (tid < kRadix) {
            uint32_t st = count;
#pragma unroll
            for (int w = 0; w < kRadix / kWave; ++w)
                if (w < static_cast<int>(wave)) st += s_wsum[w];
#pragma unroll
            for (int w = 0; w < WAVES; ++w) s_off[w * kRadix + tid] += st;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            if (j < static_cast<int>(rows)) {
                const uint32_t d = __builtin_amdgcn_ubfe(k[j], shift, width);
                const uint32_t q = (s_off[wave * kRadix + d] + pos[j]) & (TILE - 1);
                if constexpr (PAIRS) s_kv[q] = (static_cast<uint64_t>(v[j]) << 32) | k[j];
                else s_keys[q] = k[j];
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            if (j < static_cast<int>(rows)) {
                if constexpr (PAIRS) {
                    const uint64_t kv = s_kv[first + j * kWave];
                    k[j] = static_cast<uint32_t>(kv);
                    v[j] = static_cast<uint32_t>(kv >> 32);
                } else {
                    k[j] = s_keys[first + j * kWave];
                }
            }
        }
        // the next pass writes the staging buffers only after two more barriers
    }

#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        if (j < static_cast<int>(rows)) {
            const uint32_t i = first + j * kWave;
            if (i < c) {
                a.keys_out[start + i] = XF_OUT ? xform32(k[j], a.xout) : k[j];
                if constexpr (PAIRS) a.vals_out[start + i] = v[j];
            }
        }
    }
}

// Temp layout (every piece 256-byte aligned):
//   bins     [P][256]   u32   global digit counts of each pass (P = 4, or 8 for 64-bit keys)
//   sched    [P][64]    u32   tile counters of each pass, one per group (next_chunked_tile)
//   states0  [tiles][256] u32 look-back states of even passes
//   states1  [tiles][256] u32 look-back states of odd passes (passes >= 2)
//   tmp_keys [n] keys, tmp_vals [n] u32   ping-pong buffers (passes >= 2)
//   tmp_keys2 [n] keys   second key buffer of a two-key sort (its outputs are
//                        two word arrays, so its passes ping-pong in temp)
// bins, sched and states0 are contiguous and cleared by one fill launch.
//   multi    [64]           u32   multi-pass counters, and states_m [4][tiles][256]:
//                                  the hybrid sort's fallback (sizes it can take)
struct SortLayout {
    size_t bins, sched, multi, states0, states_m, states1, tmp_keys, tmp_vals, tmp_keys2, total;
    uint64_t clear_words;
    uint32_t tiles;
    uint32_t msd_tiles;   // tiles of the hybrid sort's top-digit pass (states0 holds its states)
};

constexpr uint32_t kSchedWords = 64;           // per pass: kGroups counters, padded to 256 bytes
constexpr uint32_t kMaxResidentBlocks = 4096;  // cap on the blocks of one pass

enum class PassShape { kSmall, kPairsLarge, kPairsHuge, kKeysLarge, kKeysHuge, kKey64 };

PassShape pass_shape(uint64_t n, bool pairs, bool key64) {
    if (key64) return PassShape::kKey64;
    if (pairs) {
        if (n >= kPairsHugeMinN) return PassShape::kPairsHuge;
        return n >= kPairsLargeMinN ? PassShape::kPairsLarge : PassShape::kSmall;
    }
    if (n >= kKeysHugeMinN) return PassShape::kKeysHuge;
    return n >= kKeysLargeMinN ? PassShape::kKeysLarge : PassShape::kSmall;
}

// Keys per tile of the one-sweep pass.
uint64_t pass_tile_keys(uint64_t n, bool pairs, bool key64) {
    switch (pass_shape(n, pairs, key64)) {
    case PassShape::kPairsLarge: return static_cast<uint64_t>(kPairsBlock) * kPairsItems;
    case PassShape::kPairsHuge: return static_cast<uint64_t>(kPairsBlock) * kPairsHugeItems;
    case PassShape::kKeysLarge: return static_cast<uint64_t>(kKeysBlock) * kKeysItems;
    case PassShape::kKeysHuge: return static_cast<uint64_t>(kKeysHugeBlock) * kKeysItems;
    case PassShape::kKey64: return static_cast<uint64_t>(kKey64Block) * kKey64Items;
    default: return static_cast<uint64_t>(kSortTile);
    }
}

// Sizes the hybrid sort takes (4-byte keys; it also needs two or more passes).
bool hybrid_size(uint64_t n, const SortKind& kind) {
    return !kind.key64 && n > kTileSortMax && n <= kHybridMaxN;
}

// Keys per tile of the hybrid sort's top-digit pass.
uint32_t msd_tile_keys(uint64_t n) {
    return (n + kMsdTile - 1) / kMsdTile <= kWideMaxTiles ? static_cast<uint32_t>(kMsdTile)
                                                           : static_cast<uint32_t>(kSortTile);
}

SortLayout sort_layout(uint64_t n, bool pairs, const SortKind& kind) {
    SortLayout L{};
    const int max_passes = kind.key64 ? kMaxPasses64 : kMaxPasses;
    const size_t key_bytes = kind.key64 ? 8 : 4;
    const uint64_t tile_keys = pass_tile_keys(n, pairs, kind.key64);
    L.tiles = static_cast<uint32_t>((n + tile_keys - 1) / tile_keys);
    const size_t states_bytes = align_up(static_cast<size_t>(L.tiles) * kRadix * 4);
    L.msd_tiles = 0;
    size_t states0_bytes = states_bytes;
    if (hybrid_size(n, kind)) {
        const uint32_t mt = msd_tile_keys(n);
        L.msd_tiles = static_cast<uint32_t>((n + mt - 1) / mt);
        const size_t b = align_up(static_cast<size_t>(L.msd_tiles) * kRadix * 4);
        if (b > states0_bytes) states0_bytes = b;
    }
    size_t off = 0;
    L.bins = off;
    off += align_up(static_cast<size_t>(max_passes) * kRadix * 4);
    L.sched = off;
    off += static_cast<size_t>(max_passes) * kSchedWords * 4;
    L.multi = off;
    off += kSchedWords * 4;
    L.states0 = off;
    off += states0_bytes;
    L.states_m = off;
    if (hybrid_size(n, kind)) off += static_cast<size_t>(kMaxPasses) * states_bytes;
    L.clear_words = off / 4;
    L.states1 = off;
    off += states_bytes;   // every sort path has at least two passes' worth of states
    L.tmp_keys = off;
    off += align_up(n * key_bytes);
    L.tmp_vals = off;
    if (pairs) off += align_up(n * 4);
    L.tmp_keys2 = off;
    if (kind.soa) off += align_up(n * key_bytes);
    L.total = off;
    return L;
}

// Resident blocks of one pass kernel instance (occupancy x CUs), cached.
template <typename K>
uint32_t resident_blocks(K kernel, int block) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    uint32_t r = static_cast<uint32_t>(per_cu) * static_cast<uint32_t>(device_cus());
    return r < kMaxResidentBlocks ? r : kMaxResidentBlocks;
}

template <int BLOCK, int ITEMS, int LOOKBACK, bool PAIRS, bool XI, bool XO, bool KEY64, bool WIDE>
hipError_t launch_pass_t(const PassArgs& a, hipStream_t s) {
    auto kern = onesweep_kernel<BLOCK, ITEMS, LOOKBACK, PAIRS, XI, XO, KEY64, false, WIDE>;
    static const uint32_t resident = resident_blocks(kern, BLOCK);   // one-time init
    const TileGrid g = tile_grid(a.tiles, resident, kPassChunk);
    PassArgs b = a;
    b.groups = g.groups;
    b.chunk_log2 = g.chunk_log2;
    kern<<<dim3(g.grid), BLOCK, 0, s>>>(b);
    return hipGetLastError();
}

template <int BLOCK, int ITEMS, int LOOKBACK, bool PAIRS, bool KEY64 = false, bool WIDE = false>
hipError_t launch_pass_items(bool xf_in, bool xf_out, const PassArgs& a, hipStream_t s) {
    if (xf_in && xf_out) return launch_pass_t<BLOCK, ITEMS, LOOKBACK, PAIRS, true, true, KEY64, WIDE>(a, s);
    if (xf_in) return launch_pass_t<BLOCK, ITEMS, LOOKBACK, PAIRS, true, false, KEY64, WIDE>(a, s);
    if (xf_out) return launch_pass_t<BLOCK, ITEMS, LOOKBACK, PAIRS, false, true, KEY64, WIDE>(a, s);
    return launch_pass_t<BLOCK, ITEMS, LOOKBACK, PAIRS, false, false, KEY64, WIDE>(a, s);
}

// The hybrid sort's fallback: every LSD pass in one launch of the small shape
// (hybrid sizes have at most kHybridMaxN / kSortTile <= kWideMaxTiles tiles).
template <bool PAIRS, bool XF>
hipError_t launch_multi_t(const PassArgs& a, hipStream_t s) {
    auto kern = onesweep_kernel<kSortBlock, kSortItems, kSortLookback, PAIRS, XF, XF, false, true, true>;
    static const uint32_t resident = resident_blocks(kern, kSortBlock);   // one-time init
    const uint32_t grid = a.tiles < resident ? a.tiles : resident;
    PassArgs b = a;
    b.groups = 1;
    b.chunk_log2 = 0;
    kern<<<dim3(grid), kSortBlock, 0, s>>>(b);
    return hipGetLastError();
}

hipError_t launch_multi(bool pairs, bool xf, const PassArgs& a, hipStream_t s) {
    if (pairs) return xf ? launch_multi_t<true, true>(a, s) : launch_multi_t<true, false>(a, s);
    return xf ? launch_multi_t<false, true>(a, s) : launch_multi_t<false, false>(a, s);
}

template <bool PAIRS>
hipError_t launch_pass(bool xf_in, bool xf_out, bool key64, const PassArgs& a, hipStream_t s) {
    const PassShape shape = pass_shape(a.n, PAIRS, key64);
    if (shape == PassShape::kKey64)
        return launch_pass_items<kKey64Block, kKey64Items, kSortLookback, PAIRS, true>(xf_in, xf_out, a, s);
    if (shape != PassShape::kSmall) {
        if constexpr (PAIRS) {
            if (shape == PassShape::kPairsHuge)
                return launch_pass_items<kPairsBlock, kPairsHugeItems, kPairsLookback, true>(xf_in, xf_out, a,
                                                                                             s);
            return launch_pass_items<kPairsBlock, kPairsItems, kPairsLookback, true>(xf_in, xf_out, a, s);
        } else {
            if (shape == PassShape::kKeysHuge)
                return launch_pass_items<kKeysHugeBlock, kKeysItems, kSortLookback, false>(xf_in, xf_out, a, s);
            return launch_pass_items<kKeysBlock, kKeysItems, kSortLookback, false>(xf_in, xf_out, a, s);
        }
    }
    if (a.tiles <= kWideMaxTiles)
        return launch_pass_items<kSortBlock, kSortItems, kSortLookback, PAIRS, false, true>(xf_in, xf_out, a, s);
    return launch_pass_items<kSortBlock, kSortItems, kSortLookback, PAIRS>(xf_in, xf_out, a, s);
}

// The hybrid sort's top-digit pass (the wide look-back; the tile size is
// chosen by msd_tile_keys, and a.tiles is the tile count for it).
hipError_t launch_msd_pass(bool pairs, bool xf_in, const PassArgs& a, hipStream_t s) {
    if (msd_tile_keys(a.n) == static_cast<uint32_t>(kMsdTile)) {
        return pairs ? launch_pass_items<kSortBlock, kMsdItems, kSortLookback, true, false, true>(xf_in, false, a, s)
                     : launch_pass_items<kSortBlock, kMsdItems, kSortLookback, false, false, true>(xf_in, false, a, s);
    }
    return pairs ? launch_pass_items<kSortBlock, kSortItems, kSortLookback, true, false, true>(xf_in, false, a, s)
                 : launch_pass_items<kSortBlock, kSortItems, kSortLookback, false, false, true>(xf_in, false, a, s);
}

template <int BLOCK, int ITEMS, bool PAIRS>
void launch_tile_sort_t(const uint32_t* ki, uint32_t* ko, const uint32_t* vi, uint32_t* vo,
                        uint32_t n, const PassDigits& pd, bool xf, const KeyXform& xout,
                        hipStream_t s) {
    if (xf)
        tile_sort_kernel<BLOCK, ITEMS, PAIRS, true><<<1, BLOCK, 0, s>>>(ki, ko, vi, vo, n, pd, xout);
    else
        tile_sort_kernel<BLOCK, ITEMS, PAIRS, false><<<1, BLOCK, 0, s>>>(ki, ko, vi, vo, n, pd, xout);
}

// One block, the smallest tile shape that holds n keys.
template <bool PAIRS>
void launch_tile_sort(const uint32_t* ki, uint32_t* ko, const uint32_t* vi, uint32_t* vo,
                      uint32_t n, const PassDigits& pd, bool xf, const KeyXform& xout,
                      hipStream_t s) {
    if (n <= 256 * 4)
        launch_tile_sort_t<256, 4, PAIRS>(ki, ko, vi, vo, n, pd, xf, xout, s);
    else if (n <= 512 * 8)
        launch_tile_sort_t<512, 8, PAIRS>(ki, ko, vi, vo, n, pd, xf, xout, s);
    else
        launch_tile_sort_t<1024, 16, PAIRS>(ki, ko, vi, vo, n, pd, xf, xout, s);
}

int upsweep_grid(uint32_t n) {
    const int cus = device_cus();
    const uint64_t vec_per_block = static_cast<uint64_t>(kUpBlock) * 4;   // >= 4 uint4 per thread
    uint64_t g = (static_cast<uint64_t>(n) / 4 + vec_per_block - 1) / vec_per_block;
    if (g < 1) g = 1;
    if (g > static_cast<uint64_t>(cus)) g = static_cast<uint64_t>(cus);   // one 128 KB block per CU
    return static_cast<int>(g);
}

template <bool XF>
void launch_upsweep32(const uint32_t* keys, uint32_t n, const PassDigits& pd, uint32_t* bins, int grid,
                      hipStream_t s) {
    switch (pd.passes) {
    case 1: upsweep_kernel<XF, 1><<<grid, kUpBlock, 0, s>>>(keys, n, pd, bins); break;
    case 2: upsweep_kernel<XF, 2><<<grid, kUpBlock, 0, s>>>(keys, n, pd, bins); break;
    case 3: upsweep_kernel<XF, 3><<<grid, kUpBlock, 0, s>>>(keys, n, pd, bins); break;
    default: upsweep_kernel<XF, 4><<<grid, kUpBlock, 0, s>>>(keys, n, pd, bins); break;
    }
}

// Digit positions of every pass over [begin_bit, end_bit), and the forward transform.
PassDigits pass_digits(int begin_bit, int end_bit, const KeyXform& xf) {
    PassDigits pd{};
    const int passes = (end_bit - begin_bit + kRadixBits - 1) / kRadixBits;
    pd.passes = static_cast<uint32_t>(passes);
    for (int p = 0; p < passes; ++p) {
        const int s = begin_bit + kRadixBits * p;
        const int w = (end_bit - s < kRadixBits) ? end_bit - s : kRadixBits;
        pd.shift[p] = static_cast<uint32_t>(s);
        pd.mask[p] = (1u << w) - 1u;
        pd.width[p] = static_cast<uint32_t>(w);
    }
    pd.xf = xf;
    return pd;
}

hipError_t launch_upsweep(const SortIo& io, const SortKind& kind, const PassDigits& pd,
                          uint32_t* bins, hipStream_t stream) {
    const uint32_t n = io.n;
    const bool xf = kind.transforms;
    timing_before(stream, RS_KERNEL_UPSWEEP);
    const int grid = upsweep_grid(kind.key64 && !kind.soa ? 2 * n : n);
    if (kind.key64) {
        if (kind.soa) {
            if (xf) upsweep64_kernel<true, true><<<grid, kUpBlock, 0, stream>>>(io.keys_in, io.hi_in, n, pd, bins);
            else upsweep64_kernel<false, true><<<grid, kUpBlock, 0, stream>>>(io.keys_in, io.hi_in, n, pd, bins);
        } else {
            if (xf) upsweep64_kernel<true, false><<<grid, kUpBlock, 0, stream>>>(io.keys_in, nullptr, n, pd, bins);
            else upsweep64_kernel<false, false><<<grid, kUpBlock, 0, stream>>>(io.keys_in, nullptr, n, pd, bins);
        }
    } else {
        if (xf) launch_upsweep32<true>(io.keys_in, n, pd, bins, grid, stream);
        else launch_upsweep32<false>(io.keys_in, n, pd, bins, grid, stream);
    }
    const hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace

TileGrid tile_grid(uint32_t tiles, uint32_t resident, uint32_t max_chunk) {
    TileGrid g{};
    g.grid = tiles < resident ? tiles : resident;
    if (g.grid == 0) g.grid = 1;
    // every group needs a block; a chunk is the largest power of two not above
    // the blocks per group, capped
    g.groups = g.grid < static_cast<uint32_t>(kGroups) ? g.grid : static_cast<uint32_t>(kGroups);
    g.chunk_log2 = 0;
    while ((2u << g.chunk_log2) <= g.grid / g.groups && (2u << g.chunk_log2) <= max_chunk) ++g.chunk_log2;
    return g;
}

// CUs of the device current at the first call (thread-safe one-time init).
// Grids only size the persistent launches: any count is correct, since
// blocks take their tiles dynamically.
int device_cus() {
    static const int cus = [] {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        return c;
    }();
    return cus;
}

size_t sort_temp_bytes(uint64_t n, bool pairs, const SortKind& kind) {
    if (n <= kTileSortMax && !kind.key64) return kAlign;   // the one-block sort needs no temp storage
    return sort_layout(n, pairs, kind).total;
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

// Inverse of a forward transform: the same form, with the masks of the two
// signs swapped when the forward masks flip the sign bit (then the sign of
// the transformed word is the opposite of the key's).
KeyXform inverse_xform(const KeyXform& f) {
    if ((f.pos_hi >> 31) == 0) return f;
    return KeyXform{f.neg_hi, f.pos_hi, f.neg_lo, f.pos_lo};
}

hipError_t launch_digit_counts(const SortIo& io, const SortKind& kind, int begin_bit, int end_bit,
                               uint32_t* d_counts, hipStream_t stream) {
    const PassDigits pd = pass_digits(begin_bit, end_bit, kind.xf);
    hipError_t e = launch_fill_zero(d_counts, static_cast<uint64_t>(pd.passes) * kRadix, stream,
                                    RS_KERNEL_SORT_INIT);
    if (e != hipSuccess) return e;
    return launch_upsweep(io, kind, pd, d_counts, stream);
}

hipError_t launch_sort(const SortIo& io, const SortKind& kind, int begin_bit, int end_bit,
                       void* temp, hipStream_t stream) {
    const uint32_t n = io.n;
    const bool pairs = io.vals_in != nullptr;
    const PassDigits pd = pass_digits(begin_bit, end_bit, kind.xf);
    const int passes = static_cast<int>(pd.passes);
    const KeyXform xout = inverse_xform(kind.xf);
    if (n <= kTileSortMax && !kind.key64) {
        timing_before(stream, RS_KERNEL_TILE_SORT);
        if (pairs)
            launch_tile_sort<true>(io.keys_in, io.keys_out, io.vals_in, io.vals_out, n, pd, kind.transforms,
                                   xout, stream);
        else
            launch_tile_sort<false>(io.keys_in, io.keys_out, nullptr, nullptr, n, pd, kind.transforms, xout,
                                    stream);
        const hipError_t e = hipGetLastError();
        timing_after(stream);
        return e;
    }
    const SortLayout L = sort_layout(n, pairs, kind);
    char* base = static_cast<char*>(temp);
    uint32_t* bins = reinterpret_cast<uint32_t*>(base + L.bins);
    uint32_t* sched = reinterpret_cast<uint32_t*>(base + L.sched);
    uint32_t* states[2] = {reinterpret_cast<uint32_t*>(base + L.states0),
                           reinterpret_cast<uint32_t*>(base + L.states1)};
    uint32_t* tmp_keys = reinterpret_cast<uint32_t*>(base + L.tmp_keys);
    uint32_t* tmp_vals = reinterpret_cast<uint32_t*>(base + L.tmp_vals);
    uint32_t* tmp_keys2 = reinterpret_cast<uint32_t*>(base + L.tmp_keys2);

    hipError_t e = launch_fill_zero(reinterpret_cast<uint32_t*>(base), L.clear_words, stream,
                                    RS_KERNEL_SORT_INIT);
    if (e != hipSuccess) return e;
    e = launch_upsweep(io, kind, pd, bins, stream);
    if (e != hipSuccess) return e;

    // Hybrid sort of a small input: the top digit's pass into temp, then one
    // workgroup per bucket; both run only if no bucket of the top digit
    // holds more than kBucketCap keys, and the LSD passes (all in one
    // multi-pass launch) only if one does (every launch reads the same
    // counts, so exactly one path runs).
    const int top = passes - 1;
    const bool hybrid = hybrid_size(n, kind) && passes >= 2;
    if (hybrid) {
        PassArgs a{};
        a.src_keys = io.keys_in;
        a.src_vals = io.vals_in;
        a.dst_keys = tmp_keys;
        a.dst_vals = pairs ? tmp_vals : nullptr;
        a.n = n;
        a.tiles = L.msd_tiles;
        a.shift = pd.shift[top];
        a.width = pd.width[top];
        a.bins = bins + top * kRadix;
        a.states = states[0];
        a.next_states = nullptr;
        a.sched = sched + static_cast<size_t>(top) * kSchedWords;
        a.atomic_limit_log2 = 1u;   // input order, as a first pass
        a.xin = kind.xf;
        a.gate = 1u;
        a.gate_cap = kBucketCap;
        a.gate_bins = bins + top * kRadix;
        timing_before(stream, RS_KERNEL_ONESWEEP);
        e = launch_msd_pass(pairs, kind.transforms, a, stream);
        timing_after(stream);
        if (e != hipSuccess) return e;

        BucketArgs ba{};
        ba.keys = tmp_keys;
        ba.vals = pairs ? tmp_vals : nullptr;
        ba.keys_out = io.keys_out;
        ba.vals_out = io.vals_out;
        ba.top_bins = bins + top * kRadix;
        ba.cap = kBucketCap;
        ba.pd = pd;
        ba.pd.passes = static_cast<uint32_t>(top);
        ba.xout = xout;
        const dim3 grid(1u << pd.width[top]);
        timing_before(stream, RS_KERNEL_BUCKET_SORT);
        if (pairs) {
            if (kind.transforms) bucket_sort_kernel<true, true><<<grid, kBucketBlock, 0, stream>>>(ba);
            else bucket_sort_kernel<true, false><<<grid, kBucketBlock, 0, stream>>>(ba);
        } else {
            if (kind.transforms) bucket_sort_kernel<false, true><<<grid, kBucketBlock, 0, stream>>>(ba);
            else bucket_sort_kernel<false, false><<<grid, kBucketBlock, 0, stream>>>(ba);
        }
        e = hipGetLastError();
        timing_after(stream);
        if (e != hipSuccess) return e;
    }

    if (hybrid) {
        PassArgs a{};
        a.n = n;
        a.tiles = L.tiles;
        a.bins = bins;
        a.atomic_limit_log2 = 1u;   // pass 0 reads the input order
        a.xin = kind.xf;
        a.xout = xout;
        a.gate = 2u;
        a.gate_cap = kBucketCap;
        a.gate_bins = bins + top * kRadix;
        a.multi_passes = static_cast<uint32_t>(passes);
        a.multi_counter = reinterpret_cast<uint32_t*>(base + L.multi);
        a.m_states = reinterpret_cast<uint32_t*>(base + L.states_m);
        const uint32_t* sk = io.keys_in;
        const uint32_t* sv = io.vals_in;
        for (int p = 0; p < passes; ++p) {
            const bool to_out = ((passes - 1 - p) % 2) == 0;
            a.m[p].src_keys = sk;
            a.m[p].src_vals = sv;
            a.m[p].dst_keys = to_out ? io.keys_out : tmp_keys;
            a.m[p].dst_vals = pairs ? (to_out ? io.vals_out : tmp_vals) : nullptr;
            a.m[p].shift = pd.shift[p];
            a.m[p].width = pd.width[p];
            sk = a.m[p].dst_keys;
            sv = a.m[p].dst_vals;
        }
        timing_before(stream, RS_KERNEL_ONESWEEP);
        e = launch_multi(pairs, kind.transforms, a, stream);
        timing_after(stream);
        return e;
    }

    const uint32_t* sk = io.keys_in;
    const uint32_t* sv = io.vals_in;
    for (int p = 0; p < passes; ++p) {
        const bool last = p == passes - 1;
        const bool to_out = ((passes - 1 - p) % 2) == 0;
        PassArgs a{};
        a.src_keys = sk;
        a.src_vals = sv;
        a.dst_vals = pairs ? (to_out ? io.vals_out : tmp_vals) : nullptr;
        if (kind.soa) {
            // two-key sort: the first pass reads the two word arrays, the last
            // writes them; in between 8-byte keys ping-pong in temp
            a.soa_in = (p == 0);
            a.src_hi = io.hi_in;
            a.soa_out = last;
            a.dst_keys = last ? io.keys_out : ((p % 2 == 0) ? tmp_keys : tmp_keys2);
            a.dst_hi = io.hi_out;
        } else {
            a.dst_keys = to_out ? io.keys_out : tmp_keys;
        }
        a.n = n;
        a.tiles = L.tiles;
        a.shift = pd.shift[p];
        a.width = pd.width[p];
        a.bins = bins + p * kRadix;
        a.states = states[p & 1];
        a.next_states = (p + 1 < passes) ? states[(p + 1) & 1] : nullptr;
        a.sched = sched + static_cast<size_t>(p) * kSchedWords;
        // The first pass reads the input order, where earlier passes have not
        // gathered equal digits into runs, so its atomic rank pays off up to a
        // digit holding half of the keys (measured); later passes stop at 1/16.
        a.atomic_limit_log2 = (p == 0) ? 1u : 4u;
        a.xin = kind.xf;
        a.xout = xout;
        const bool xf_in = kind.transforms && p == 0;
        const bool xf_out = kind.transforms && last;
        timing_before(stream, RS_KERNEL_ONESWEEP);
        e = pairs ? launch_pass<true>(xf_in, xf_out, kind.key64, a, stream)
                  : launch_pass<false>(xf_in, xf_out, kind.key64, a, stream);
        timing_after(stream);
        if (e != hipSuccess) return e;
        sk = a.dst_keys;
        sv = a.dst_vals;
    }
    return hipSuccess;
}

}  // namespace rs
