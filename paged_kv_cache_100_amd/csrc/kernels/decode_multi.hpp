// Decode attention for several query tokens per sequence: the Q tokens of a
// speculative-decoding verification pass (the lesson's speculative-decoding
// section: the target model checks all draft tokens in one forward pass),
// already appended to the cache like a single decode token.
//
// What is computed: query token i (0 <= i < Q) of sequence b sits at position
// ctx - Q + i and, under the lesson's Build-It step 2 mask for seq_len_q > 1
// (an upper triangle anchored at the bottom-right corner of the score
// matrix), attends positions 0 .. ctx - Q + i -- what decoding the tokens one
// after another would have computed.  A query that sees no position gets
// zeros.  q and out are [B][Q][N][H].
//
// Work decomposition: as in decode.hpp, a wave per (partition, KV head,
// sequence), but the columns of the matrix-core tiles are now the Q * G
// (query token, query head) pairs of the KV head's group: column c = 16t + col
// of tile t is query token c / G, head c % G.  One wave carries all of a KV
// head's pairs, up to four tiles (64 columns); its key and value registers
// serve every tile, so the cache is read once however many tokens are
// verified.  The load ring gets shallower as tiles are added (their
// accumulators take its registers).  Each tile column keeps its own running
// maximum and sum.
//
// Masking: each score is checked against its own column's limit and value
// elements at or past ctx are zeroed, in every chunk (the checks only bite in
// the last one or two chunks of a sequence; a single code path keeps the
// loop small enough for the registers); an all-masked column's state stays
// finite (reference maximum 0 while the column has seen no position).
#pragma once

#include "decode.hpp"

namespace pkv {

constexpr int kMaxQueryTiles = 4;   // Q * G <= 64
constexpr int kBufferFlags = 0x00020000;   // word 3 of a raw buffer resource (gfx9)
constexpr int kCoherentAux = 16;           // cache policy: system-coherence bit (sc1)
constexpr int kTilesPerWave = 4;
constexpr int kXcds = 8;            // MI355X: workgroups are dealt to 8 XCDs in turn

// Chunk buffers per wave for kTiles tiles: bf16 4, 3, 3, 2; FP8 5, 4, 3, 2.
// These fit gfx950's 256 vector registers without spilling only because the
// per-column output rows are recomputed after the chunk loop and, from four
// tiles on, FP8 value codes are widened anew for every tile
// (KvFp8::value_fresh): holding the widened values of all eight value tiles
// across the tile loop takes 32 more registers than the kernel has.
template <class Fmt, int kTiles>
constexpr int multi_ring_depth()
{
    return kTiles == 1 ? Fmt::kRing
                       : kTiles == 2 ? Fmt::kRing - 1 : kTiles == 3 ? 3 : 2;
}

// One 32-token chunk for kTiles column tiles.  tok0 is the position of this
// lane's first token (chunk start + 8 * quad); column t of this lane sees
// positions below lim[t]; vrem = ctx - chunk start.  qf(t, s) yields the
// lane's query operand.  kMasked: the chunk may hold positions some column
// does not see; mask_scores (uniform) says whether it does, and value
// elements at or past ctx are zeroed in place, once for all tiles, in the
// chunk that holds the end of the context (both only near a sequence's end,
// so the other chunks pay for neither).
template <class Fmt, int H, int kTiles, bool kMasked, class QFrag>
__device__ __forceinline__ void attend_chunk_multi(typename Fmt::template Regs<H> &r,
                                                   QFrag &&qf, int tok0,
                                                   const int (&lim)[kTiles], int vrem, int quad,
                                                   float scale_log2, float (&m)[kTiles],
                                                   float (&l)[kTiles],
                                                   f32x4 (&acc)[kTiles][H / 16],
                                                   bool mask_scores = true)
{
    if (kMasked && vrem < kChunk)
        Fmt::template zero_values<H>(r, min(max(vrem - 8 * quad, 0), 8));
    // One tile at a time (scores, softmax, P.V), so only one tile's P is live.
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < H / 32; ++s) {
            const bf16x8 q = qf(t, s);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Fmt::key(r, 0, s), q, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Fmt::key(r, 1, s), q, s1, 0, 0, 0);
        }
        // Raw scores: the scale (never negative) goes on after the maximum
        // and into the exponent's argument, as in attend_chunk.
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = s0[i];
            x[4 + i] = s1[i];
        }
        if (kMasked && mask_scores) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (tok0 + e >= lim[t])
                    x[e] = -INFINITY;
        }
        float mx = max8(x);
        mx = max_over_rows(mx) * scale_log2;
        const float m_new = vmax(m[t], mx);
        // A column that has seen no position yet keeps m = -inf; exponentials
        // are then taken against 0 (all of them are 0).
        const float m_ref = (kMasked && m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m[t] - m_ref);
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], scale_log2, -m_ref));
        float psum = p[0];
#pragma unroll
        for (int e = 1; e < 8; ++e)
            psum += p[e];
        bf16x8 p_hi, p_lo;
        split_bf16(p, p_hi, p_lo);
        l[t] = l[t] * alpha + psum;
        m[t] = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int c = 0; c < H / 16; ++c)
                acc[t][c] *= alpha;
        }
#pragma unroll
        for (int c = 0; c < H / 16; ++c) {
            const bf16x8 vv = as_bf16x8(kTiles >= 4 ? Fmt::value_fresh(r, c) : Fmt::value(r, c));
            acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, p_hi, acc[t][c], 0, 0, 0);
            acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, p_lo, acc[t][c], 0, 0, 0);
        }
    }
}

// Grid: one dimension of kXcds * col_groups * ceil(items / kXcds) waves.
// Workgroup id L -> XCD L % 8, slot j = L / 8 on it; column group j % CG of
// item (j / CG) * 8 + L % 8; item = (b * K + kvh) * parts + partition.
template <class Fmt, int H, int kTiles, bool kSplit, int BS = kBlockSize>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_multi_kernel(DecodeParams p)
{
    const int L = blockIdx.x;
    const int xcd = L % kXcds;
    const int j = L / kXcds;
    const int cg = j % p.col_groups;
    const int64_t item = (int64_t)(j / p.col_groups) * kXcds + xcd;
    if (item >= (int64_t)p.num_parts * p.num_kv_heads * p.num_seqs)
        return;
    const int part_idx = (int)(item % p.num_parts);
    const int kvh = (int)((item / p.num_parts) % p.num_kv_heads);
    const int b = (int)(item / ((int64_t)p.num_parts * p.num_kv_heads));
    const int lane = threadIdx.x;
    const int col = lane & 15;
    const int quad = lane >> 4;
    const int Q = p.num_queries;
    const int G = p.group;

    const int start = part_idx * p.part;
    const int first_block = start / BS;
    const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks + first_block;

    const int ctx = min(max(p.context_lens[b], 0), p.max_ctx);

    // Column t of this lane: query token i, head g; its output row in
    // [B][Q][N] and the positions it sees.  The rows are recomputed where
    // they are used (from an index the compiler cannot see through), so
    // that they hold no registers across the chunk loop.
    auto out_row = [&](int t, int lane_id) -> int64_t {
        const int c = 16 * (kTiles * cg + t) + (lane_id & 15);
        const bool lv = c < Q * G;
        const int i = lv ? c / G : 0;
        const int g = lv ? c - i * G : 0;
        return ((int64_t)b * Q + i) * p.num_heads + kvh * G + g;
    };
    auto opaque_lane = [&]() {
        int v = lane;
        asm volatile("" : "+v"(v));
        return v;
    };
    bool live[kTiles];
    int lim[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const int c = 16 * (kTiles * cg + t) + col;
        live[t] = c < Q * G;
        lim[t] = live[t] ? ctx - Q + c / G + 1 : ctx;
    }

    // Two partitions merged in this kernel: a sequence whose context fits the
    // first partition is finished by that partition's wave alone.
    // (Four tiles keep the merge kernel: their registers leave no room for it.)
    constexpr bool kPairMerge = kSplit && kTiles < kMaxQueryTiles;
    const bool pair = kPairMerge && p.pair_tags != nullptr;
    if (start >= ctx) {
        if ((!kSplit || pair) && part_idx == 0) {   // empty sequence: zeros
#pragma unroll
            for (int t = 0; t < kTiles; ++t) {
                if (!live[t])
                    continue;
                float *o = p.out + out_row(t, lane) * H;
#pragma unroll
                for (int c = 0; c < H / 16; ++c)
                    *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        return;
    }
    const int end = min(start + p.part, ctx);
    const int n_blocks = (end - 1) / BS - first_block + 1;
    const int n_chunks = (end - start + kChunk - 1) / kChunk;

    // The query fragments live in this wave's LDS (each lane reads back only
    // what it wrote): registers go to the accumulators and the chunk ring.
    __shared__ u32x4 q_lds[kTiles * (H / 32) * kWave];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const uint16_t *qrow = p.q + out_row(t, lane) * H;
#pragma unroll
        for (int s = 0; s < H / 32; ++s) {
            u32x4 raw = load16(qrow + Fmt::dim_offset(s, quad));
            if (!live[t])
                raw = u32x4{0u, 0u, 0u, 0u};
            q_lds[(t * (H / 32) + s) * kWave + lane] = raw ^ p.q_sign;
        }
    }

    constexpr uint32_t tile_elems = BS * H;
    const uint32_t block_elems = (uint32_t)p.num_kv_heads * tile_elems;   // < 2^31
    const uint32_t id_lim = id_bound(p.num_blocks);
    using Elem = typename Fmt::Elem;
    using Regs = typename Fmt::template Regs<H>;
    const Elem *kbase = static_cast<const Elem *>(p.key_cache) + (uint64_t)kvh * tile_elems;
    const Elem *vbase = static_cast<const Elem *>(p.value_cache) + (uint64_t)kvh * tile_elems;

    // A chunk's two block ids are loaded one chunk ahead (load_chunk_ids), so
    // a partition may span any number of blocks.
    ChunkIds ids = load_chunk_ids<BS>(table, 0, n_blocks);
    auto issue = [&](Regs &r, int ci) {
        const uint64_t o0 = block_offset(ids.raw0, id_lim, block_elems);
        const uint64_t o1 = block_offset(ids.raw1, id_lim, block_elems);
        Fmt::template load<H, BS>(r, kbase + o0, kbase + key_hi<BS, H>(o1), vbase + o0,
                                  vbase + value_hi<BS>(o1), col, quad);
        if (ci + 1 < n_chunks)
            ids = load_chunk_ids<BS>(table, ci + 1, n_blocks);
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

    // Query token 0 sees positions below ctx - Q + 1: chunks wholly below
    // that need no score mask.
    const int lim_min = ctx - Q + 1;
    auto attend = [&](Regs &r, int ci) {
        // An index the compiler cannot see through, so that the LDS reads stay
        // inside the loop instead of being hoisted back into registers.
        int opaque = lane;
        asm volatile("" : "+v"(opaque));
        auto qfrag = [&](int t, int s) {
            return as_bf16x8(q_lds[(t * (H / 32) + s) * kWave + opaque]);
        };
        const int c0 = start + kChunk * ci;
        attend_chunk_multi<Fmt, H, kTiles, true>(r, qfrag, c0 + 8 * quad, lim, ctx - c0, quad,
                                                 p.scale_log2, m, l, acc,
                                                 c0 + kChunk > lim_min);
    };

    constexpr int kRing = multi_ring_depth<Fmt, kTiles>();
    Regs ring[kRing];
    run_ring<kRing>(n_chunks, ring, issue, attend);

    const bool single = !kSplit || (pair && ctx <= p.part);   // this wave finishes its rows
    // Pair partials of this sequence: a buffer over its Q * N rows of two
    // partitions, so that 16-byte accesses can carry the coherence bit.
    const int64_t pair_base = (int64_t)b * Q * p.num_heads * 2 * H;   // in floats
    const __amdgpu_buffer_rsrc_t pair_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        p.part_o + (pair ? pair_base : 0), 0, Q * p.num_heads * 2 * H * 4, kBufferFlags);
    float lts[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const float lt = sum_over_rows(l[t]);
        lts[t] = lt;
        if (!live[t])
            continue;
        if (single && !pair) {
            const float inv = lt > 0.f ? p.out_scale / lt : 0.f;
            float *o = p.out + out_row(t, opaque_lane()) * H;
#pragma unroll
            for (int c = 0; c < H / 16; ++c)
                *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = acc[t][c] * inv;
        } else if (single) {
            // One partition of a two-partition call: the merge's arithmetic on
            // a single partial (weight 1), so that the result is the one the
            // merge kernel would give.
            const float inv = lt > 0.f ? 1.0f / lt : 0.f;
            float *o = p.out + out_row(t, opaque_lane()) * H;
#pragma unroll
            for (int c = 0; c < H / 16; ++c)
                *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = (acc[t][c] * p.out_scale) * inv;
        } else if (!pair) {
            const int64_t slot = out_row(t, opaque_lane()) * p.num_parts + part_idx;
            float *o = p.part_o + slot * H;
#pragma unroll
            for (int c = 0; c < H / 16; ++c)
                *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = acc[t][c] * p.out_scale;
            if (quad == 0) {
                p.part_ml[2 * slot] = m[t];
                p.part_ml[2 * slot + 1] = lt;
            }
        } else {
            // Read by the other partition's wave, possibly on another XCD:
            // device-coherent 16-byte stores (system-coherence bit).
            const int64_t slot = out_row(t, opaque_lane()) * 2 + part_idx;
            const int off = (int)((slot * H - pair_base) * 4);
#pragma unroll
            for (int c = 0; c < H / 16; ++c)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, acc[t][c] * p.out_scale), pair_rsrc,
                    off + (16 * c + 4 * quad) * 4, 0, kCoherentAux);
            if (quad == 0) {
                store_coherent(p.part_ml + 2 * slot, m[t]);
                store_coherent(p.part_ml + 2 * slot + 1, lt);
            }
        }
    }
    if constexpr (!kPairMerge)
        return;
    if (!pair || single)
        return;
    // Two partitions: once this wave's partial is stored, it swaps the call's
    // tag into the (sequence, KV head) slot.  Finding the tag already there
    // means the other wave's partial is stored: this wave merges both, in
    // partition order with merge_parts_kernel's arithmetic (so the result
    // does not depend on which wave merges), reading the other partial with
    // device-coherent loads.  Nothing waits on the other wave, and the tags
    // need no clearing: every call brings a new value.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint64_t seen = 0;
    if (lane == 0)
        seen = __hip_atomic_exchange(p.pair_tags + ((int64_t)b * p.num_kv_heads + kvh) *
                                                       p.col_groups + cg, p.epoch,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)seen);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(seen >> 32));
    if ((((uint64_t)hi << 32) | lo) != p.epoch)
        return;                           // first to finish: the other wave merges
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        if (!live[t])
            continue;
        const int64_t row = out_row(t, opaque_lane());
        const int64_t other = row * 2 + (1 - part_idx);
        const float mo = load_coherent(p.part_ml + 2 * other);
        const float lo_ = load_coherent(p.part_ml + 2 * other + 1);
        f32x4 oo[H / 16];
        const int ooff = (int)((other * H - pair_base) * 4);
#pragma unroll
        for (int c = 0; c < H / 16; ++c)
            oo[c] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           pair_rsrc, ooff + (16 * c + 4 * quad) * 4, 0, kCoherentAux));
        // partition 0 first, as merge_parts_kernel takes them
        const bool own_first = part_idx == 0;
        const float m0 = own_first ? m[t] : mo, m1 = own_first ? mo : m[t];
        const float l0 = own_first ? lts[t] : lo_, l1 = own_first ? lo_ : lts[t];
        float nb = -INFINITY;
        const bool u0 = m0 > -INFINITY, u1 = m1 > -INFINITY;
        nb = u0 ? fmaxf(nb, m0) : nb;
        nb = u1 ? fmaxf(nb, m1) : nb;
        const float w0 = u0 ? __builtin_amdgcn_exp2f(m0 - nb) : 0.f;
        const float w1 = u1 ? __builtin_amdgcn_exp2f(m1 - nb) : 0.f;
        float den = 0.f;
        den += u0 ? w0 * l0 : 0.f;
        den += u1 ? w1 * l1 : 0.f;
        const float inv = den > 0.f ? 1.0f / den : 0.f;
        float *o = p.out + row * H;
#pragma unroll
        for (int c = 0; c < H / 16; ++c) {
            const f32x4 own = acc[t][c] * p.out_scale;
            const f32x4 o0 = own_first ? own : oo[c], o1 = own_first ? oo[c] : own;
            f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
            num += u0 ? w0 * o0 : f32x4{0.f, 0.f, 0.f, 0.f};
            num += u1 ? w1 * o1 : f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = num * inv;
        }
    }
}

}  // namespace pkv
