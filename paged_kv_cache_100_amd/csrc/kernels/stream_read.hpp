// Plain streaming read and copy of a buffer with 16-byte accesses.  Not part
// of the attention method: they calibrate the HBM byte counters (launches of
// known size) and give the achievable bandwidth to compare the decode kernel
// against.
#pragma once

#include "common.hpp"

namespace pkv {

constexpr int kStreamThreads = 256;
constexpr int kStreamBlocksMax = 16384;

// Streaming read in the decode kernels' access pattern: one wave per SIMD
// (grid = waves W), non-temporal 16-byte loads, kStreamLoads per lane per
// step (16 KiB per wave at 16 loads, the size of a bf16 decode chunk), two
// steps in flight.  Steps are dealt round-robin (wave w reads steps w, w + W,
// ...), so at any moment the waves read one contiguous span of W steps that
// covers every HBM channel, as the decode's scattered blocks do; contiguous
// per-wave shares would start every wave at the same offset modulo the
// channel interleave.  The bandwidth it reaches is the ceiling the decode's
// K/V stream is compared with.
constexpr int kStreamLoads = 16;

__device__ __forceinline__ u32x4 xor_all(const u32x4 (&v)[kStreamLoads])
{
    u32x4 a = v[0];
#pragma unroll
    for (int u = 1; u < kStreamLoads; ++u)
        a ^= v[u];
    return a;
}

__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void stream_read_kernel(const u32x4 *src, int64_t n16, u32x4 *sink)
{
    constexpr int64_t kStep = (int64_t)kStreamLoads * kWave;     // 16-byte units per step
    const int64_t W = gridDim.x;
    const int64_t steps = n16 / kStep;
    const int lane = threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    u32x4 a[kStreamLoads], b[kStreamLoads];
    auto load = [&](u32x4 (&v)[kStreamLoads], int64_t step) {
#pragma unroll
        for (int u = 0; u < kStreamLoads; ++u)
            v[u] = __builtin_nontemporal_load(src + step * kStep + u * kWave + lane);
    };
    int64_t k = blockIdx.x;
    if (k < steps) {
        load(a, k);
        // Steady state: the next step's loads are issued before this one's
        // are consumed.
        for (; k + 2 * W < steps; k += 2 * W) {
            load(b, k + W);
            acc ^= xor_all(a);
            load(a, k + 2 * W);
            acc ^= xor_all(b);
        }
        if (k + W < steps) {
            load(b, k + W);
            acc ^= xor_all(a);
            acc ^= xor_all(b);
        } else {
            acc ^= xor_all(a);
        }
    }
    for (int64_t i = steps * kStep + (int64_t)blockIdx.x * kWave + lane; i < n16; i += W * kWave)
        acc ^= __builtin_nontemporal_load(src + i);
    // A store the compiler cannot prove dead keeps every load alive; for real
    // data it practically never fires.
    if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0xF39CC060u &&
        acc[3] == 0x5CEDC834u)
        sink[blockIdx.x] = acc;
}

// Plain copy with 16-byte loads and stores: a launch that reads and writes a
// known number of bytes, to scale the HBM read and write counters.
__global__ __launch_bounds__(kStreamThreads) void stream_copy_kernel(const u32x4 *src, u32x4 *dst,
                                                                     int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

}  // namespace pkv
