// Shared-prefix-aware decode and the copy-on-write block copy.
//
// Sequences that share a prompt prefix point their block tables at the same
// physical blocks ("CS336 Lecture 10: Inference", part 6: shared prefix
// blocks, copied on write).  Plain decode reads those blocks once per sharer.
// Here a prefix group -- its members listed by the caller -- reads its shared
// span once: the span is cut into partitions of P tokens, and for each one a
// wave's matrix-core tiles take as columns the (member, query head) pairs of
// a KV head's group, so every load of a shared key or value serves all the
// members the wave carries (up to four tiles, 64 pairs, per wave; more
// members take more waves, placed on one XCD at consecutive slots so their
// repeated reads meet in its L2).  Each member gets the partition's partial
// (m, l, o) over its own shared positions; the token-balanced per-sequence
// waves take the rest of every context, and their merge folds the prefix
// partials in with the log-sum-exp rule.  The result is plain attention:
// paging and sharing only change where the blocks are read from.
//
// Member b of group g shares positions 0 .. S_b - 1 (shared_span: the
// group's prefix, b's and the lead's contexts, rounded down to a chunk); the
// group's partitions cover the lead's span, and b's columns are masked from
// S_b on.  Partials go to row ((b * K + kvh) * prefix_parts + p) * G + g' of
// d.part_o / d.part_ml, so a partition's G rows are contiguous.  Every S_b
// is stored in d.shared_tokens (0 outside a group) for the merge: by the first
// ceil(B / 64) group waves for batches the per-sequence waves scan themselves
// (they compute S_b too), else by a small kernel before the per-sequence ones,
// which read it.  The group waves run in the token-balanced kernel's grid,
// after its persistent waves: the dispatcher places them as those finish, so
// they fill the idle SIMDs of its tail.
#pragma once

#include "decode_multi.hpp"

namespace pkv {

// One thread per sequence: d.shared_tokens[b] = S_b.
__global__ __launch_bounds__(kWave) void prefix_spans_kernel(DecodeParams d)
{
    const int b = (int)blockIdx.x * kWave + (int)threadIdx.x;
    if (b < d.num_seqs)
        d.shared_tokens[b] = prefix_shared_tokens(d, b);
}

// Group wave L (XCD-aware as in decode_multi_kernel): items =
// (group * K + kvh) * prefix_parts + partition, d.col_groups waves each.
// prefix_parts: partitions per member row, ceil(max shared span / P), with
// d.part = P.  q_lds: kTiles * (H / 32) * 64 16-byte slots of LDS.
// store_spans: waves L < ceil(B / 64) store S_b of sequences 64 L + lane.
template <class Fmt, int H, int kTiles, int BS = kBlockSize>
__device__ __forceinline__ void prefix_group_wave(const DecodeParams &d, int prefix_parts, int L,
                                                  u32x4 *q_lds, bool store_spans)
{
    const int lane = (int)threadIdx.x % kWave;
    if (store_spans && (int64_t)L * kWave < d.num_seqs) {
        const int b = L * kWave + lane;
        if (b < d.num_seqs)
            d.shared_tokens[b] = prefix_shared_tokens(d, b);
    }
    const int xcd = L % kXcds;
    const int j = L / kXcds;
    const int cg = j % d.col_groups;
    const int64_t item = (int64_t)(j / d.col_groups) * kXcds + xcd;
    if (item >= (int64_t)d.num_groups * d.num_kv_heads * prefix_parts)
        return;
    const int part_idx = (int)(item % prefix_parts);
    const int kvh = (int)((item / prefix_parts) % d.num_kv_heads);
    const int grp = (int)(item / ((int64_t)prefix_parts * d.num_kv_heads));
    const int col = lane & 15;
    const int quad = lane >> 4;
    const int G = d.group;
    const int32_t *members = d.group_members + (int64_t)grp * d.max_members;

    const int lead = members[0];
    if (lead < 0 || lead >= d.num_seqs)
        return;
    // The partition's block ids (read before its length is known: as many as
    // a partition holds, within the table row), then the partition's
    // positions within the lead's shared span.
    const int start = part_idx * d.part;
    const int32_t *table = d.block_tables + (int64_t)lead * d.max_blocks + start / BS;
    int my_id = 0;
    if (lane < d.part / BS && start / BS + lane < d.max_blocks)
        my_id = clamp_block(table[lane], d.num_blocks);
    const int prefix = d.prefix_tokens[grp];
    const int ctx_lead = min(max(d.context_lens[lead], 0), d.max_ctx);
    const int span = shared_span(d, prefix, ctx_lead, ctx_lead);
    if (start >= span)
        return;
    const int end = min(start + d.part, span);
    const int n_blocks = (end - start) / BS;

    // Column t of this lane: member m, head g; lim: the end of the member's
    // shared positions (a multiple of the chunk).  Only the member's sequence
    // (-1 for a column with nothing to attend) stays live across the chunk
    // loop; the head within the group is recomputed where it is needed.
    auto head_of = [&](int t, int lane_id) {
        const int c = 16 * (kTiles * cg + t) + (lane_id & 15);
        return c - (c / G) * G;
    };
    int mcol[kTiles];
    int lim[kTiles];
    bool short_col = false;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const int c = 16 * (kTiles * cg + t) + col;
        const int m = c / G;
        const int mb = m < d.max_members ? members[m] : -1;
        const bool in_group = mb >= 0 && mb < d.num_seqs && d.seq_group[mb] == grp;
        const int own =
            in_group ? shared_span(d, prefix, min(max(d.context_lens[mb], 0), d.max_ctx), ctx_lead)
                     : 0;
        const bool live = own > start;
        mcol[t] = live ? mb : -1;
        lim[t] = live ? min(own, end) : end;
        short_col |= live && own < end;
    }
    const bool mask = __builtin_amdgcn_ballot_w64(short_col) != 0;

#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const int64_t qrow =
            (int64_t)(mcol[t] >= 0 ? mcol[t] : lead) * d.num_heads + kvh * G + head_of(t, lane);
        const uint16_t *qr = d.q + qrow * H;
#pragma unroll
        for (int s = 0; s < H / 32; ++s) {
            u32x4 raw = load16(qr + Fmt::dim_offset(s, quad));
            if (mcol[t] < 0)
                raw = u32x4{0u, 0u, 0u, 0u};
            q_lds[(t * (H / 32) + s) * kWave + lane] = raw ^ d.q_sign;
        }
    }

    const int64_t tile_elems = (int64_t)BS * H;
    const int64_t block_elems = (int64_t)d.num_kv_heads * tile_elems;
    using Elem = typename Fmt::Elem;
    using Regs = typename Fmt::template Regs<H>;
    const Elem *kbase = static_cast<const Elem *>(d.key_cache) + kvh * tile_elems;
    const Elem *vbase = static_cast<const Elem *>(d.value_cache) + kvh * tile_elems;
    auto issue = [&](Regs &r, int ci) {
        const int k0 = (kChunk / BS) * ci;
        const int id0 = __builtin_amdgcn_readlane(my_id, k0);
        const int id1 = (BS == 16 && k0 + 1 < n_blocks) ? __builtin_amdgcn_readlane(my_id, k0 + 1)
                                                        : id0;
        const uint64_t o0 = (uint64_t)id0 * block_elems, o1 = (uint64_t)id1 * block_elems;
        Fmt::template load<H, BS>(r, kbase + o0, kbase + key_hi<BS, H>(o1), vbase + o0,
                                  vbase + value_hi<BS>(o1), col, quad);
    };

    float m[kTiles], l[kTiles];
    f32x4 acc[kTiles][H / 16];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        m[t] = -INFINITY;
        l[t] = 0.f;
#pragma unroll
        for (int c = 0; c < H / 16; ++c)
            acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Every position of the partition is a cached token; a member whose
    // shared span ends inside the partition has its later positions masked
    // (whole chunks: spans are multiples of the chunk).
    auto attend = [&](Regs &r, int ci) {
        int opaque = lane;
        asm volatile("" : "+v"(opaque));
        auto qfrag = [&](int t, int s) {
            return as_bf16x8(q_lds[(t * (H / 32) + s) * kWave + opaque]);
        };
        attend_chunk_multi<Fmt, H, kTiles, true>(r, qfrag, start + kChunk * ci + 8 * quad, lim,
                                                 end - start - kChunk * ci, quad, d.scale_log2,
                                                 m, l, acc, mask);
    };
    constexpr int kRing = multi_ring_depth<Fmt, kTiles>();
    Regs ring[kRing];
    run_ring<kRing>((end - start) / kChunk, ring, issue, attend);

    int opaque = lane;
    asm volatile("" : "+v"(opaque));
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const float lt = sum_over_rows(l[t]);
        if (mcol[t] < 0)
            continue;
        const int64_t prow =
            (((int64_t)mcol[t] * d.num_kv_heads + kvh) * prefix_parts + part_idx) * G +
            head_of(t, opaque);
        float *o = d.part_o + prow * H;
#pragma unroll
        for (int c = 0; c < H / 16; ++c)
            *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = acc[t][c] * d.out_scale;
        if (quad == 0) {
            d.part_ml[2 * prow] = m[t];
            d.part_ml[2 * prow + 1] = lt;
        }
    }
}

// ----------------------------------------------------- copy-on-write copy --

struct CopyBlocksParams {
    uint8_t *key_cache;
    uint8_t *value_cache;
    const int32_t *src;
    const int32_t *dst;
    int64_t block_bytes;   // K * block_size * H * element size, a multiple of 16
    int64_t num_blocks;
};

constexpr int kCopyThreads = 256;

// blockIdx.y = pair, blockIdx.x = slice of the block: 16-byte loads and
// stores of both pools.  Pairs with an id outside [0, num_blocks) are skipped.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyBlocksParams p)
{
    const int s = p.src[blockIdx.y];
    const int t = p.dst[blockIdx.y];
    if (s < 0 || t < 0 || s >= p.num_blocks || t >= p.num_blocks || s == t)
        return;
    const int64_t stride = (int64_t)gridDim.x * kCopyThreads * 16;
    for (int64_t off = ((int64_t)blockIdx.x * kCopyThreads + threadIdx.x) * 16;
         off < p.block_bytes; off += stride) {
        const u32x4 k = load16(p.key_cache + s * p.block_bytes + off);
        const u32x4 v = load16(p.value_cache + s * p.block_bytes + off);
        store16(p.key_cache + t * p.block_bytes + off, k);
        store16(p.value_cache + t * p.block_bytes + off, v);
    }
}

}  // namespace pkv
