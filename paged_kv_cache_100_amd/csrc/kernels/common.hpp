// Shared device types for the paged-KV kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// Load of a value that is the same for every lane and does not change while
// the kernel runs (context lengths, block-table entries): through the
// constant address space it becomes a scalar-unit load, which neither waits
// for nor holds up the wave's vector-memory (K/V) loads.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int32_t scalar_load(const int32_t *p) { return *(const const_i32 *)p; }

// Device-coherent 32-bit accesses (agent-scope relaxed atomics: written
// through to, and read from, the level every XCD shares) for data one wave
// hands to a wave of another XCD inside one launch.
__device__ __forceinline__ void store_coherent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float *p, f32x4 v)
{
#pragma unroll
    for (int e = 0; e < 4; ++e)
        store_coherent(p + e, v[e]);
}
__device__ __forceinline__ float load_coherent(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Maximum of scores, NaN-propagating (IEEE maximum): gfx950 has it as one
// three-operand instruction that needs no canonicalised inputs, where fmaxf
// (maxNum) costs an extra canonicalising max per operand that the compiler
// cannot prove canonical (matrix-core results, lane exchanges).  Masked
// positions are -inf, so a NaN here is a NaN score, which spoils its column
// either way.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max8(const float (&x)[8])
{
    return vmax(vmax(vmax(vmax(x[0], x[1]), x[2]), vmax(vmax(x[3], x[4]), x[5])),
                vmax(x[6], x[7]));
}

// Lane-pair reductions across the four 16-lane rows with VALU permutes
// (no LDS round trip): max / sum of v over lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float max_over_rows(float v)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_rows(float v)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace pkv
