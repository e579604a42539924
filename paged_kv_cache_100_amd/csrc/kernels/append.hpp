// Slot-mapped append of one decode step's K/V rows into the paged cache.
//
// The step's new token computes only its own key and value and stores them
// next to the cached ones ("Week 11. Inference", step 2; the KV-cache class of
// the "Optimización de la inferencia" lesson, Build-It step 1, writes the new
// rows at the next position).  In the paged cache the "next position" of a
// token is its slot, physical_block * 16 + offset, resolved by the caller.
//
// One thread moves 8 consecutive head-dim values (16 bytes) of one (token,
// KV head): a single 16-byte store for the key row, and eight 2-byte stores
// down the value tile's columns (value tiles are stored transposed, [H][16]),
// so a token dirties every 128-byte line of its value tile (32 at H = 128).
// The decode that follows reads those lines more slowly the more of them the
// append wrote (its key rows, two lines per token, cost next to nothing);
// writing the value elements with non-temporal stores sends them toward
// memory at once and takes part of that cost off the decode.
#pragma once

#include "common.hpp"

namespace pkv {

struct AppendParams {
    const uint16_t *k;             // [T][K][H]
    const uint16_t *v;             // [T][K][H]
    const int64_t *slot_mapping;   // [T]
    uint16_t *key_cache;           // [num_blocks][K][16][H]
    uint16_t *value_cache;         // [num_blocks][K][H][16]
    int32_t num_tokens;
    int32_t num_kv_heads;
    int64_t num_slots;             // num_blocks * 16
};

// Makes the two row loads complete before the slot test: left alone, the
// compiler moves them behind it and the thread waits for two memory round
// trips (slot, then rows) instead of one.
__device__ __forceinline__ void keep_loaded(const u32x4 &a, const u32x4 &b)
{
    asm volatile("" : : "v"(a), "v"(b));
}

template <int H>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p)
{
    constexpr int kChunks = H / 8;   // 16-byte pieces per row
    // The host guarantees T * K * H / 8 < 2^31: 32-bit index arithmetic.
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t total = (uint32_t)p.num_tokens * p.num_kv_heads * kChunks;
    if (gid >= total)
        return;
    const int c = (int)(gid % kChunks);
    const uint32_t row = gid / kChunks;            // token * K + head
    const int g = (int)(row % (uint32_t)p.num_kv_heads);
    const uint32_t i = row / (uint32_t)p.num_kv_heads;

    // The rows' loads do not depend on the slot: issue all three together.
    const int64_t src = (int64_t)row * H + 8 * c;
    const u32x4 kk = load16(p.k + src);
    const u32x4 vv = load16(p.v + src);
    const int64_t slot = p.slot_mapping[i];
    keep_loaded(kk, vv);
    if (slot < 0 || slot >= p.num_slots)
        return;                                    // padding or outside the pool
    const int64_t blk = slot / kBlockSize;
    const int off = (int)(slot % kBlockSize);
    const int64_t tile = blk * p.num_kv_heads + g; // (block, head) tile index

    store16(p.key_cache + (tile * kBlockSize + off) * H + 8 * c, kk);
    uint16_t *dst = p.value_cache + (tile * H + 8 * c) * kBlockSize + off;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t word = vv[e >> 1];
        __builtin_nontemporal_store((uint16_t)((e & 1) ? (word >> 16) : (word & 0xFFFFu)),
                                    dst + e * kBlockSize);
    }
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

// Eight bf16 values (16 bytes) -> eight codes (8 bytes, same order).
__device__ __forceinline__ u32x2 quantize8(u32x4 x, float inv)
{
    u32x2 r;
    r[0] = quantize_pair(x[0], inv) | (quantize_pair(x[1], inv) << 16);
    r[1] = quantize_pair(x[2], inv) | (quantize_pair(x[3], inv) << 16);
    return r;
}

template <int H>
__global__ __launch_bounds__(256) void append_fp8_kernel(AppendFp8Params p)
{
    constexpr int kChunks = H / 8;   // 8-value pieces per row
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t total = (uint32_t)p.num_tokens * p.num_kv_heads * kChunks;
    if (gid >= total)
        return;
    const int c = (int)(gid % kChunks);
    const uint32_t row = gid / kChunks;
    const int g = (int)(row % (uint32_t)p.num_kv_heads);
    const uint32_t i = row / (uint32_t)p.num_kv_heads;

    const int64_t src = (int64_t)row * H + 8 * c;
    const u32x4 kk = load16(p.k + src);
    const u32x4 vv = load16(p.v + src);
    const int64_t slot = p.slot_mapping[i];
    keep_loaded(kk, vv);
    if (slot < 0 || slot >= p.num_slots)
        return;
    const int64_t blk = slot / kBlockSize;
    const int off = (int)(slot % kBlockSize);
    const int64_t tile = blk * p.num_kv_heads + g;

    const u32x2 kq = quantize8(kk, p.k_inv);
    *reinterpret_cast<u32x2 *>(p.key_cache + (tile * kBlockSize + off) * H + 8 * c) = kq;

    const u32x2 vq = quantize8(vv, p.v_inv);
    uint8_t *dst = p.value_cache + (tile * H + 8 * c) * kBlockSize + off;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        __builtin_nontemporal_store((uint8_t)(vq[e >> 2] >> (8 * (e & 3))), dst + e * kBlockSize);
}

}  // namespace pkv
