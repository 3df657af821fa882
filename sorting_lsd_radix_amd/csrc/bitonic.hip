// bitonic.hip -- LDS bitonic sort of independent tiles of up to 1024 keys.
//
// Batcher's network ("第10章 并行模式：排序", 10.2 Bitonic Sort算法: bitonic
// sequences, half-cleaners, log2(N)(log2(N)+1)/2 compare-exchange steps of
// N/2 comparators each; "gpu排序__gpu", the one-block shared-memory version
// that pads to a power of two with the largest key).  The network is not
// stable (10.7), so each element is compared as the pair (field, position in
// the tile): all pairs are distinct, the network's result is unique and equals
// the stable order of the field.  Padding uses field 0xFFFFFFFF with positions
// past the tile, which sorts after every real element and is never stored.
#include "device_common.hpp"
#include "internal.hpp"

namespace rs {

namespace {

constexpr int kBitonicMax = 1024;
constexpr int kBitonicBlock = kBitonicMax / 2;   // one comparator per thread per step

__global__ __launch_bounds__(kBitonicBlock) void bitonic_tile_kernel(
    const uint32_t* __restrict__ keys_in, uint32_t* __restrict__ keys_out, uint32_t n,
    uint32_t tile, uint32_t span, uint32_t shift, uint32_t mask) {
    // s_item: (field << 32) | position; s_key: original key by position
    __shared__ uint64_t s_item[kBitonicMax];
    __shared__ uint32_t s_key[kBitonicMax];

    const uint32_t base = blockIdx.x * tile;
    const uint32_t len = (n - base < tile) ? n - base : tile;
    const uint32_t tid = threadIdx.x;

    for (uint32_t i = tid; i < span; i += kBitonicBlock) {
        if (i < len) {
            const uint32_t key = keys_in[base + i];
            s_key[i] = key;
            s_item[i] = (static_cast<uint64_t>((key >> shift) & mask) << 32) | i;
        } else {
            s_item[i] = (0xFFFFFFFFull << 32) | i;
        }
    }
    __syncthreads();

    // Step (k, j) pairs element a = 2*tid - (tid mod j) with a + j.  For
    // j <= 64 the 64 lanes of a wave touch only their own 128 elements, so
    // between two such steps the wave needs no block barrier: the LDS executes
    // one wave's instructions in order, and a wave-scope fence keeps the
    // compiler from moving the next step's reads above this step's writes.
    const uint32_t pairs = span / 2;
    for (uint32_t k = 2; k <= span; k <<= 1) {
        for (uint32_t j = k >> 1; j > 0; j >>= 1) {
            if (tid < pairs) {
                const uint32_t a = 2 * tid - (tid & (j - 1));
                const uint32_t b = a + j;
                const bool ascending = (a & k) == 0;
                const uint64_t xa = s_item[a];
                const uint64_t xb = s_item[b];
                if ((xa > xb) == ascending) {
                    s_item[a] = xb;
                    s_item[b] = xa;
                }
            }
            const uint32_t next_j = (j > 1) ? (j >> 1) : k;   // k == span ends the network
            if (j <= kWave && next_j <= kWave) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            } else {
                __syncthreads();
            }
        }
    }
    __syncthreads();

    for (uint32_t i = tid; i < len; i += kBitonicBlock)
        keys_out[base + i] = s_key[static_cast<uint32_t>(s_item[i])];
}

// Full-width keys (begin_bit 0, end_bit 32): equal fields are equal keys, so
// the network needs no positions and any order of equals is the stable one.
// 256 threads hold the padded 1024-key tile in registers, four keys each:
// element e = 4 * tid + r (wave w holds e in [256 w, 256 w + 256)).  Step
// (k, j) pairs e with e ^ j: for j = 1, 2 both are in one thread's
// registers; for j = 4 .. 128 the partner is lane ^ (j / 4) of the same wave
// (DPP quad permutes for 1 and 2, a row rotate for 8, swizzles for 4 and
// 16, a lane permute for 32); for j = 256, 512 it is in another wave, and
// the step goes through LDS between two block barriers.  Element e keeps the
// smaller of the pair when (e is the lower index) == (e & k == 0, the
// ascending half of its bitonic sequence), the larger otherwise.
constexpr int kBitonicRegThreads = 256;

template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane distance");
    if constexpr (M == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    else if constexpr (M == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    else if constexpr (M == 8) return __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
    else if constexpr (M == 4 || M == 16)   // swizzle, bitmask mode: lane ^ M within 32 lanes
        return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(x), 0x1F | (M << 10)));
    else return __shfl_xor(x, 32, kWave);
}

__device__ __forceinline__ uint32_t keep(uint32_t x, uint32_t y, uint32_t e, uint32_t j, uint32_t k) {
    const bool keep_min = ((e & j) == 0) == ((e & k) == 0);
    return keep_min ? min(x, y) : max(x, y);
}

template <int K, int J>
__device__ __forceinline__ void bitonic_step(uint32_t (&x)[4], uint32_t e0, uint32_t* s) {
    if constexpr (J >= 256) {
        __syncthreads();   // the previous exchange's reads are done
#pragma unroll
        for (int r = 0; r < 4; ++r) s[e0 + r] = x[r];
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = keep(x[r], s[(e0 + r) ^ J], e0 + r, J, K);
    } else if constexpr (J >= 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = keep(x[r], lane_xor<J / 4>(x[r]), e0 + r, J, K);
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if ((r & J) == 0) {
                const uint32_t a = x[r], b = x[r + J];
                const bool up = ((e0 + r) & K) == 0;
                x[r] = up ? min(a, b) : max(a, b);
                x[r + J] = up ? max(a, b) : min(a, b);
            }
        }
    }
}

template <int K, int J>
__device__ __forceinline__ void bitonic_merge(uint32_t (&x)[4], uint32_t e0, uint32_t* s) {
    bitonic_step<K, J>(x, e0, s);
    if constexpr (J > 1) bitonic_merge<K, J / 2>(x, e0, s);
}

template <int K>
__device__ __forceinline__ void bitonic_network(uint32_t (&x)[4], uint32_t e0, uint32_t* s) {
    bitonic_merge<K, K / 2>(x, e0, s);
    if constexpr (K < kBitonicMax) bitonic_network<K * 2>(x, e0, s);
}

__global__ __launch_bounds__(kBitonicRegThreads) void bitonic_tile_u32_kernel(
    const uint32_t* __restrict__ keys_in, uint32_t* __restrict__ keys_out, uint32_t n, uint32_t tile) {
    __shared__ uint32_t s_x[kBitonicMax];
    const uint32_t base = blockIdx.x * tile;
    const uint32_t len = (n - base < tile) ? n - base : tile;
    const uint32_t e0 = threadIdx.x * 4;
    uint32_t x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (e0 + r < len) ? keys_in[base + e0 + r] : 0xFFFFFFFFu;   // pads sort last
    bitonic_network<2>(x, e0, s_x);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (e0 + r < len) keys_out[base + e0 + r] = x[r];
}

}  // namespace

hipError_t launch_bitonic(const uint32_t* keys_in, uint32_t* keys_out, uint32_t n, uint32_t tile,
                          int begin_bit, int end_bit, hipStream_t stream) {
    uint32_t span = 1;
    while (span < tile) span <<= 1;
    if (span < 2) span = 2;
    const int width = end_bit - begin_bit;
    const uint32_t mask = (width >= 32) ? 0xFFFFFFFFu : ((1u << width) - 1u);
    const uint32_t shift = (width == 0) ? 0u : static_cast<uint32_t>(begin_bit);
    const uint32_t tiles = (n + tile - 1) / tile;
    timing_before(stream, RS_KERNEL_BITONIC);
    if (begin_bit == 0 && end_bit == 32)
        bitonic_tile_u32_kernel<<<dim3(tiles), kBitonicRegThreads, 0, stream>>>(keys_in, keys_out, n, tile);
    else
        bitonic_tile_kernel<<<dim3(tiles), kBitonicBlock, 0, stream>>>(keys_in, keys_out, n, tile, span,
                                                                       shift, mask);
    hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace rs
