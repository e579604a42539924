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
// down the value tile's columns (value tiles are stored transposed, [H][16]).
// The step moves at most a few hundred KiB, so the strided value stores cost
// nothing measurable next to the attention that follows.
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

template <int H>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p)
{
    constexpr int kChunks = H / 8;   // 16-byte pieces per row
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)p.num_tokens * p.num_kv_heads * kChunks;
    if (gid >= total)
        return;
    const int c = (int)(gid % kChunks);
    const int64_t row = gid / kChunks;             // token * K + head
    const int g = (int)(row % p.num_kv_heads);
    const int64_t i = row / p.num_kv_heads;

    const int64_t slot = p.slot_mapping[i];
    if (slot < 0 || slot >= p.num_slots)
        return;                                    // padding or outside the pool
    const int64_t blk = slot / kBlockSize;
    const int off = (int)(slot % kBlockSize);
    const int64_t tile = blk * p.num_kv_heads + g; // (block, head) tile index

    const int64_t src = row * H + 8 * c;
    store16(p.key_cache + (tile * kBlockSize + off) * H + 8 * c, load16(p.k + src));

    const u32x4 vv = load16(p.v + src);
    uint16_t *dst = p.value_cache + (tile * H + 8 * c) * kBlockSize + off;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t word = vv[e >> 1];
        dst[e * kBlockSize] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xFFFFu));
    }
}

}  // namespace pkv
