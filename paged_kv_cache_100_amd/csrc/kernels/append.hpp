// Slot-mapped append of one decode step's K/V rows into the paged cache.
//
// The step's new token computes only its own key and value and stores them
// next to the cached ones ("Week 11. Inference", step 2; the KV-cache class of
// the "Optimización de la inferencia" lesson, Build-It step 1, writes the new
// rows at the next position).  In the paged cache the "next position" of a
// token is its slot, physical_block * 16 + offset, resolved by the caller.
//
// One wave per (token, KV head).  Lane l moves head dims 2l and 2l + 1 of the
// key row (one 4-byte store each; the wave writes the row's 2H bytes
// contiguously) and head dims l + 64j of the value.  Value tiles are stored
// transposed ([H][16]), so a token's value elements are 2 bytes in each of H
// rows of 32 bytes: one store instruction of the wave writes 64 consecutive
// rows, four elements in each 128-byte line it touches -- the most one token
// puts in a line (a thread per 8 dims, storing down its rows, put one).  The
// decode that follows reads the lines the append wrote more slowly the more
// of them are freshly written; keys and values go out with non-temporal
// stores, which send them toward memory at once.
#pragma once

#include "common.hpp"

namespace pkv {

struct AppendParams {
    const uint16_t *k;             // [T][K][H]
    const uint16_t *v;             // [T][K][H]
    const int64_t *slot_mapping;   // [T]
    uint16_t *key_cache;           // [num_blocks][K][BS][H]
    uint16_t *value_cache;         // [num_blocks][K][H][BS]
    int32_t num_tokens;
    int32_t num_kv_heads;
    int64_t num_slots;             // num_blocks * BS
};

// Makes the row loads complete before the slot test: left alone, the
// compiler moves them behind it and the thread waits for two memory round
// trips (slot, then rows) instead of one.
__device__ __forceinline__ void keep_loaded(uint32_t a, uint32_t b)
{
    asm volatile("" : : "v"(a), "v"(b));
}

// (token * K + head) of this wave: the grid is 4-wave workgroups.
__device__ __forceinline__ uint64_t append_row()
{
    return (uint64_t)blockIdx.x * 4 + threadIdx.x / kWave;
}

template <int H, int BS = kBlockSize>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p)
{
    constexpr int kVals = H / kWave;                 // value dims per lane
    const uint64_t row = append_row();
    if (row >= (uint64_t)p.num_tokens * p.num_kv_heads)
        return;
    const int lane = threadIdx.x % kWave;
    const int g = (int)(row % (uint64_t)p.num_kv_heads);
    const uint64_t i = row / (uint64_t)p.num_kv_heads;
    const bool key_lane = 2 * lane < H;

    // The rows' loads do not depend on the slot: issue them all together.
    const uint16_t *krow = p.k + row * H;
    const uint16_t *vrow = p.v + row * H;
    const uint32_t kk = key_lane ? *reinterpret_cast<const uint32_t *>(krow + 2 * lane) : 0u;
    uint16_t vv[kVals];
#pragma unroll
    for (int j = 0; j < kVals; ++j)
        vv[j] = vrow[lane + kWave * j];
    const int64_t slot = p.slot_mapping[i];
    keep_loaded(kk, (uint32_t)vv[0] | ((uint32_t)vv[kVals - 1] << 16));
    if (slot < 0 || slot >= p.num_slots)
        return;                                    // padding or outside the pool
    const int64_t blk = slot / BS;
    const int off = (int)(slot % BS);
    const int64_t tile = blk * p.num_kv_heads + g; // (block, head) tile index

    if (key_lane)
        __builtin_nontemporal_store(
            kk, reinterpret_cast<uint32_t *>(p.key_cache + (tile * BS + off) * H + 2 * lane));
    uint16_t *dst = p.value_cache + tile * H * BS + off;
#pragma unroll
    for (int j = 0; j < kVals; ++j)
        __builtin_nontemporal_store(vv[j], dst + (lane + kWave * j) * BS);
}

// ---------------------------------------------------------------- FP8 ----
//
// Append into OCP FP8 E4M3 pools (one scale per pool): each bf16 value x is
// stored as the code nearest to x * inv (inv = 1/scale in fp32, one fp32
// multiply), after that product is clamped to +-448 (the largest finite
// code); ties go to the even code, NaN stores 0xFF.  The hardware conversion
// rounds to nearest even; the clamp keeps it from producing the NaN code for
// finite values, and NaN is forced to 0xFF explicitly.
struct AppendFp8Params {
    const uint16_t *k;             // [T][K][H] bf16
    const uint16_t *v;             // [T][K][H] bf16
    const int64_t *slot_mapping;   // [T]
    uint8_t *key_cache;            // [num_blocks][K][16][H] E4M3
    uint8_t *value_cache;          // [num_blocks][K][H][16] E4M3
    float k_inv;                   // fp32(1 / k_scale)
    float v_inv;                   // fp32(1 / v_scale)
    int32_t num_tokens;
    int32_t num_kv_heads;
    int64_t num_slots;
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// Codes of the two bf16 values packed in `word` (low half first), as the
// low 16 bits of the result.
__device__ __forceinline__ uint32_t quantize_pair(uint32_t word, float inv)
{
    float y0 = bf16_bits_to_float(word & 0xFFFFu) * inv;
    float y1 = bf16_bits_to_float(word >> 16) * inv;
    const uint32_t nan_bytes = (y0 != y0 ? 0x00FFu : 0u) | (y1 != y1 ? 0xFF00u : 0u);
    y0 = y0 > 448.0f ? 448.0f : (y0 < -448.0f ? -448.0f : y0);
    y1 = y1 > 448.0f ? 448.0f : (y1 < -448.0f ? -448.0f : y1);
    const uint32_t codes = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false) & 0xFFFFu;
    return codes | nan_bytes;
}

// The lane layout of append_kernel; key codes go out two per lane (2-byte
// stores, the row's H bytes contiguously), value codes one byte per store.
template <int H, int BS = kBlockSize>
__global__ __launch_bounds__(256) void append_fp8_kernel(AppendFp8Params p)
{
    constexpr int kVals = H / kWave;
    const uint64_t row = append_row();
    if (row >= (uint64_t)p.num_tokens * p.num_kv_heads)
        return;
    const int lane = threadIdx.x % kWave;
    const int g = (int)(row % (uint64_t)p.num_kv_heads);
    const uint64_t i = row / (uint64_t)p.num_kv_heads;
    const bool key_lane = 2 * lane < H;

    const uint16_t *krow = p.k + row * H;
    const uint16_t *vrow = p.v + row * H;
    const uint32_t kk = key_lane ? *reinterpret_cast<const uint32_t *>(krow + 2 * lane) : 0u;
    uint16_t vv[kVals];
#pragma unroll
    for (int j = 0; j < kVals; ++j)
        vv[j] = vrow[lane + kWave * j];
    const int64_t slot = p.slot_mapping[i];
    keep_loaded(kk, (uint32_t)vv[0] | ((uint32_t)vv[kVals - 1] << 16));
    if (slot < 0 || slot >= p.num_slots)
        return;
    const int64_t blk = slot / BS;
    const int off = (int)(slot % BS);
    const int64_t tile = blk * p.num_kv_heads + g;

    if (key_lane)
        *reinterpret_cast<uint16_t *>(p.key_cache + (tile * BS + off) * H + 2 * lane) =
            (uint16_t)quantize_pair(kk, p.k_inv);
    uint8_t *dst = p.value_cache + tile * H * BS + off;
#pragma unroll
    for (int j = 0; j < kVals; ++j)
        __builtin_nontemporal_store((uint8_t)quantize_pair(vv[j], p.v_inv),
                                    dst + (lane + kWave * j) * BS);
}

}  // namespace pkv
