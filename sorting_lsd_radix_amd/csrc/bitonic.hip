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
    bitonic_tile_kernel<<<dim3(tiles), kBitonicBlock, 0, stream>>>(keys_in, keys_out, n, tile, span,
                                                                   shift, mask);
    hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace rs
