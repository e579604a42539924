// Plain streaming read of a buffer with 16-byte loads.  Not part of the
// attention method: it calibrates the HBM byte counters (a launch of known
// size) and gives the achievable read bandwidth to compare the decode kernel
// against.
#pragma once

#include "common.hpp"

namespace pkv {

constexpr int kStreamThreads = 256;
constexpr int kStreamBlocksMax = 4096;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4 *src, int64_t n16,
                                                                     u32x4 *sink)
{
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride)
        acc ^= src[i];
    // A store the compiler cannot prove dead keeps every load alive; for real
    // data it practically never fires.
    if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0xF39CC060u &&
        acc[3] == 0x5CEDC834u)
        sink[blockIdx.x] = acc;
}

}  // namespace pkv
