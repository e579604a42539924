// Plain streaming read and copy of a buffer with 16-byte accesses.  Not part
// of the attention method: they calibrate the HBM byte counters (launches of
// known size) and give the achievable bandwidth to compare the decode kernel
// against.
#pragma once

#include "common.hpp"

namespace pkv {

constexpr int kStreamThreads = 256;
constexpr int kStreamBlocksMax = 16384;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4 *src, int64_t n16,
                                                                     u32x4 *sink)
{
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride)
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
