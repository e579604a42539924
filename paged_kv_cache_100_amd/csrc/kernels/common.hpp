// Shared device types for the paged-KV kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlockSize = 16;   // tokens per cache block
constexpr int kWave = 64;        // CDNA wavefront width

// 16-byte global load / store of raw bits.
__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// 16-byte load with the non-temporal hint: data read once (the KV cache
// stream) should not displace reusable lines from the caches.
__device__ __forceinline__ u32x4 load16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void store16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

}  // namespace pkv
