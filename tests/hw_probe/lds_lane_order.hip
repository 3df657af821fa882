// lds_lane_order.hip -- test infrastructure (not part of the library).
//
// Checks the hardware property the large keys-only sort pass relies on: when
// several lanes of one wave's LDS atomic add (ds_add_rtn_u32) hit the same
// address, the values returned follow lane order, so lane L receives the
// counter's old value plus the number of lower lanes with the same address.
// Each probe row draws one 8-bit "digit" per lane from a seeded hash, reads
// the wave's counter for it, computes the lane-order rank with a shuffle
// loop, then performs the atomic add and compares.  Every address stays in
// the block's LDS counters and no loop waits on another wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// mode 0: uniform digits; 1: 8 values; 2: all equal; 3: 80 % one digit;
// 4: half the lanes on digits 32 apart (same LDS bank), half uniform
__device__ __forceinline__ uint32_t probe_digit(uint32_t h, uint32_t mode) {
    switch (mode) {
    case 0: return h & 255u;
    case 1: return h & 7u;
    case 2: return 5u;
    case 3: return (h % 100u < 80u) ? 3u : (h >> 8) & 255u;
    default: return (h & 1u) ? 32u * ((h >> 1) & 7u) : (h >> 4) & 255u;
    }
}

__global__ __launch_bounds__(1024) void lane_order_kernel(uint32_t seed, uint32_t mode, uint32_t rows,
                                                          unsigned long long* mismatches) {
    __shared__ uint32_t counters[16 * 256];
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    for (uint32_t i = lane; i < 256u; i += 64u) counters[wave * 256u + i] = 0u;
    __builtin_amdgcn_wave_barrier();
    uint32_t bad = 0;
    for (uint32_t row = 0; row < rows; ++row) {
        const uint32_t h = mix32(seed * 2654435761u + blockIdx.x * 7919u + tid * 131u + row * 977u);
        const uint32_t d = probe_digit(h, mode);
        uint32_t below = 0;
        for (int l = 0; l < 64; ++l) {
            // every lane takes part in every shuffle (a lane left out would not supply its digit)
            const uint32_t dl = static_cast<uint32_t>(__shfl(static_cast<int>(d), l, 64));
            if (static_cast<uint32_t>(l) < lane && dl == d) ++below;
        }
        const uint32_t before = counters[wave * 256u + d];
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        const uint32_t got = atomicAdd(&counters[wave * 256u + d], 1u);
        if (got != before + below) ++bad;
        __builtin_amdgcn_wave_barrier();
    }
    if (bad) atomicAdd(mismatches, static_cast<unsigned long long>(bad));
}

}  // namespace

// Runs `blocks` blocks of 1024 threads for each of `seeds` seeds in one mode
// and returns the number of lanes whose atomic result broke lane order, or
// -1 on a HIP error.  Synchronises the device.
extern "C" long long probe_lds_lane_order(int mode, int seeds, int blocks, int rows) {
    unsigned long long* d_bad = nullptr;
    if (hipMalloc(&d_bad, sizeof(unsigned long long)) != hipSuccess) return -1;
    long long result = -1;
    if (hipMemset(d_bad, 0, sizeof(unsigned long long)) == hipSuccess) {
        for (int s = 0; s < seeds; ++s)
            lane_order_kernel<<<blocks, 1024>>>(static_cast<uint32_t>(s + 1 + 1000 * mode),
                                                static_cast<uint32_t>(mode), static_cast<uint32_t>(rows),
                                                d_bad);
        unsigned long long h_bad = 0;
        if (hipGetLastError() == hipSuccess && hipDeviceSynchronize() == hipSuccess &&
            hipMemcpy(&h_bad, d_bad, sizeof(h_bad), hipMemcpyDeviceToHost) == hipSuccess)
            result = static_cast<long long>(h_bad);
    }
    (void)hipFree(d_bad);
    return result;
}
