// Decode-phase attention over the paged KV cache, for gfx950 (CDNA4).
//
// What is computed (the attention-with-cache step of the "Optimización de la
// inferencia" lesson, in the paged form of its PagedAttention section and of
// "CS336 Lecture 10: Inference", parts 3 and 6): for every sequence b and
// query head n = kvh * G + g,
//     out[b][n] = sum_t softmax_t(scale * q[b][n] . k_t) v_t
// over the sequence's cached positions t < ctx_b, where position t lives in
// physical block block_tables[b][t / 16] at offset t % 16, and all G query
// heads of a group read the same KV head kvh.
//
// Work decomposition.  One wavefront owns one (partition, KV head, sequence):
// the G query heads of the group are the 16 columns of the matrix-core tiles
// (G <= 16; unused columns compute on zero queries and are never stored), so
// every key and value byte of the group is loaded from HBM exactly once.
// The wave walks its partition 32 tokens (two cache blocks) at a time:
//
//   scores   S^T[32 x 16] = K_chunk[32 x H] . Q^T[H x 16]
//            two v_mfma_f32_16x16x32_bf16 tiles per 32 k-values of H; each
//            lane's A operand is 16 contiguous bytes of one key row, loaded
//            straight from HBM into registers.
//   softmax  online (running maximum m and sum l per query column, in log2
//            units so one v_exp_f32 serves each score); the column maximum of
//            a chunk is reduced across the four lane quads with two
//            cross-lane shuffles.
//   P.V      O^T[H x 16] += V^T[H x 32] . P^T[32 x 16], one tile per 16
//            values of H.  The value tile is stored transposed ([H][16] per
//            block), so each lane's A operand is again 16 contiguous bytes.
//            P (in [0, 1]) is carried as p_hi + p_lo, both bf16, so the
//            product keeps ~16 significant bits (relative error <= 2^-17)
//            while V stays in bf16 with no conversion work.
//
// Row order inside a score tile is permuted so that the 4 scores a lane holds
// in each of the two S^T tiles are 8 *consecutive* tokens -- exactly the 8
// consecutive P^T values that lane must supply to the P.V tile: tile a, row
// m holds token 8*(m/4) + 4*a + m%4.  No data moves between the two
// products.
//
// Split-K ("FlashDecoding", named in "CS336 Lecture 10: Inference", part 6):
// the context is cut into partitions of `part` tokens.  With one partition
// the kernel normalises and writes `out` itself.  With several, each wave
// writes its partial (m, l, unnormalised o) and merge_kernel combines them:
//     M = max_j m_j,  out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j.
//
// Masking.  Scores of positions >= ctx become -inf, and value elements of
// those positions are zeroed before the matrix product (block tails may hold
// anything, NaN included); a block past the sequence's last block is never
// addressed (its table entry is not read).
#pragma once

#include "kv_format.hpp"

namespace pkv {

constexpr int kChunk = 32;   // tokens per inner step (two cache blocks)

struct DecodeParams {
    float *out;                   // [B][N][H]
    float *part_o;                // [B][N][P][H]   (split only; prefix pieces:
                                  //                 [B][K][pieces][G][H])
    float *part_ml;               // [B][N][P][2]   (likewise, pairs (m, l))
    const uint16_t *q;            // [B][N][H] bf16
    const void *key_cache;        // [num_blocks][K][16][H]  (Fmt::Elem)
    const void *value_cache;      // [num_blocks][K][H][16]  (Fmt::Elem)
    const int32_t *block_tables;  // [B][max_blocks]
    const int32_t *context_lens;  // [B]
    float scale_log2;             // |scale| * log2(e) (times k_scale for FP8 pools),
                                  // at least FLT_MIN
    uint32_t q_sign;              // 0x80008000 when the scale is negative (the
                                  // query's signs are flipped on load), else 0
    float out_scale;              // factor on every written o: 1, or v_scale for FP8 pools
    int32_t num_heads;            // N
    int32_t num_kv_heads;         // K
    int32_t group;                // G = N / K
    int32_t max_blocks;
    int32_t max_ctx;
    int32_t part;                 // tokens per partition (multiple of 32)
    int32_t num_parts;            // P
    int32_t num_queries;          // Q query tokens per sequence (1 for plain decode)
    int32_t col_groups;           // multi-query / prefix: waves per work item
    int32_t num_seqs;             // B
    int64_t num_blocks;
    // Prefix-aware decode only (else null / 0): sharers of a prompt prefix.
    const int32_t *seq_group;     // [B]: prefix group of each sequence, -1 = none
    const int32_t *group_members; // [num_groups][max_members], -1 = unused
    const int32_t *prefix_tokens; // [num_groups]: shared positions 0 .. prefix_tokens - 1
    int32_t num_groups;
    int32_t max_members;
    int32_t max_prefix;           // cap on every shared span (whole partitions the
                                  // workspace holds partials for)
    int32_t *shared_tokens;       // [B]: S_b, written by the group kernel; null = none
    int32_t window;               // sliding window: attend the last `window` positions; 0 = all
    // Multi-query calls of exactly two partitions: per (sequence, KV head)
    // tags through which the two partition waves find which of them finishes
    // second (that one merges both partials); null = merge_parts_kernel merges.
    uint64_t *pair_tags = nullptr;
    uint64_t epoch = 0;           // this call's tag value (never 0)
    // Tokens per cache block (16 or 32).  The host picks the kernels built
    // for it; the kernels take it as a template parameter, not from here.
    int32_t block_size = kBlockSize;
};

// First position a sequence of ctx tokens attends (sliding window), else 0.
__device__ __forceinline__ int window_start(const DecodeParams &d, int ctx)
{
    return d.window > 0 ? max(ctx - d.window, 0) : 0;
}

// Shared-prefix decode: sequence b's positions 0 .. S_b - 1 are read by its
// prefix group's kernel (once for all members), the rest by b's own waves.
// S_b = min(prefix_tokens[g], ctx_b, ctx_lead, max_prefix) rounded down to a
// whole chunk, lead being the group's first member, whose block table holds
// the shared block ids; 0 when b belongs to no group.  The group kernel
// computes it (shared_span, from its group's values) and stores it in
// d.shared_tokens for the per-sequence waves and the merge.
__device__ __forceinline__ int shared_span(const DecodeParams &d, int prefix_tokens, int ctx_b,
                                           int ctx_lead)
{
    const int span = min(min(min(prefix_tokens, ctx_b), ctx_lead), d.max_prefix);
    return max(span, 0) / kChunk * kChunk;
}

__device__ __forceinline__ int prefix_shared_tokens(const DecodeParams &d, int b)
{
    const int g = d.seq_group[b];
    if (g < 0 || g >= d.num_groups)
        return 0;
    const int lead = d.group_members[(int64_t)g * d.max_members];
    if (lead < 0 || lead >= d.num_seqs)
        return 0;
    return shared_span(d, d.prefix_tokens[g], min(max(d.context_lens[b], 0), d.max_ctx),
                       min(max(d.context_lens[lead], 0), d.max_ctx));
}

// S_b as the per-sequence side reads it (0 when no group kernel ran, and for
// indices past the batch).  The load depends on nothing loaded before it, so
// it shares a memory round trip with the context length.
__device__ __forceinline__ int stored_shared_tokens(const DecodeParams &d, int b)
{
    return (d.shared_tokens && b < d.num_seqs) ? d.shared_tokens[b] : 0;
}

__device__ __forceinline__ int clamp_block(int id, int64_t num_blocks)
{
    return (id >= 0 && (int64_t)id < num_blocks) ? id : 0;
}

// The two block ids of one 32-token chunk, as loaded.  Both go out together
// through the scalar unit, and the kernels clamp and use them only when the
// chunk's K/V loads are issued, a whole chunk of work later: a use right
// after the load would stall the wave for the table's round trip.  A chunk
// of one block loads its first id twice, so the second address stays inside
// the sequence's blocks.
struct ChunkIds {
    int raw0, raw1;
};
// The block ids of chunk jj (32 tokens) from a table row of nblk entries:
// two 16-token blocks, or one 32-token block (then raw1 = raw0).
template <int BS = kBlockSize>
__device__ __forceinline__ ChunkIds load_chunk_ids(const int32_t *row, int jj, int nblk)
{
    static_assert(BS == 16 || BS == 32, "16- or 32-token blocks");
    if constexpr (BS == 32) {
        const int id = scalar_load(row + jj);
        return ChunkIds{id, id};
    } else {
        const int e = 2 * jj;   // e < nblk
        return ChunkIds{scalar_load(row + e), scalar_load(row + min(e + 1, nblk - 1))};
    }
}

// Element offsets, from a chunk's block offsets o0 / o1 (each the start of a
// (block, KV head) tile), of its second 16 tokens in the key and value
// tiles: the second block's tile with 16-token blocks; with 32-token blocks
// the same tile, 16 key rows further and 16 elements into every value row.
template <int BS, int H>
__device__ __forceinline__ uint64_t key_hi(uint64_t o1)
{
    return BS == 32 ? o1 + 16 * H : o1;
}
template <int BS>
__device__ __forceinline__ uint64_t value_hi(uint64_t o1)
{
    return BS == 32 ? o1 + 16 : o1;
}

// clamp_block's bound as an unsigned 32-bit value: ids are int32, so
// min(num_blocks, 2^31) admits exactly the same ids, and a negative id, seen
// unsigned, is at least 2^31.
__device__ __forceinline__ uint32_t id_bound(int64_t num_blocks)
{
    return (uint32_t)min(max(num_blocks, (int64_t)0), (int64_t)1 << 31);
}

// Element offset of the block with id `raw` (block 0 if raw is outside
// [0, num_blocks)) in a pool of block_elems = K * BS * H elements per block.
// The host keeps K * BS * H below 2^31, so one 32 x 32-bit product serves.
__device__ __forceinline__ uint64_t block_offset(int raw, uint32_t bound, uint32_t block_elems)
{
    const uint32_t id = (uint32_t)raw < bound ? (uint32_t)raw : 0u;
    return ((uint64_t)__umulhi(id, block_elems) << 32) | (id * block_elems);
}

// `qf(s)` yields the lane's query operand for k-step s (from registers or LDS).
// kTail: a chunk with masked positions -- those at or past `rem` (the end of
// the context: their values are zeroed too) and those before `head` (the
// start of a sliding window: valid cached tokens, only their scores are
// masked).
template <class Fmt, int H, bool kTail, class QFrag>
__device__ __forceinline__ void attend_chunk(const typename Fmt::template Regs<H> &r, QFrag &&qf,
                                             int rem, int head, int quad,
                                             float scale_log2, float &m, float &l,
                                             f32x4 (&acc)[H / 16])
{
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < H / 32; ++s) {
        const bf16x8 q = qf(s);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Fmt::key(r, 0, s), q, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Fmt::key(r, 1, s), q, s1, 0, 0, 0);
    }
    // Lane (col, quad) now holds the scores of tokens 8quad + e, e = 0..7.
    // The softmax scale (never negative) goes on after the maximum, and into
    // the exponent's argument with one fused multiply-add.
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = s0[i];
        x[4 + i] = s1[i];
    }
    u32x4 vmask = {~0u, ~0u, ~0u, ~0u};
    if (kTail) {   // rem - head < 32 tokens valid
        const int valid = min(max(rem - 8 * quad, 0), 8);
        const int skip = min(max(head - 8 * quad, 0), 8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e >= valid || e < skip)
                x[e] = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            vmask[w] = (2 * w < valid ? 0x0000FFFFu : 0u) | (2 * w + 1 < valid ? 0xFFFF0000u : 0u);
    }
    float mx = max8(x);
    mx = max_over_rows(mx) * scale_log2;
    const float m_new = vmax(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);   // 0 on the first chunk

    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], scale_log2, -m_new));
    float psum = p[0];
#pragma unroll
    for (int e = 1; e < 8; ++e)
        psum += p[e];
    bf16x8 p_hi, p_lo;
    split_bf16(p, p_hi, p_lo);
    l = l * alpha + psum;
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int c = 0; c < H / 16; ++c)
            acc[c] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < H / 16; ++c) {
        const u32x4 vbits = Fmt::value(r, c);
        const bf16x8 vv = as_bf16x8(kTail ? (vbits & vmask) : vbits);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, p_hi, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, p_lo, acc[c], 0, 0, 0);
    }
}

// Register ring: a kernel keeps Fmt::kRing chunk buffers per wave, so
// kRing - 1 chunks are in flight while one is computed.  One wave per SIMD
// owns up to 512 registers: four 64-register bf16 chunks, or five
// 32-register FP8 chunks, fit next to the accumulators.

// Runs chunks 0 .. total-1 (total >= 1) through a ring of kRing register
// buffers: issue(buf, k) starts the loads of chunk k, attend(buf, k) consumes
// them.  The steady-state loop has no branch between an issue and the attend
// that follows it, so the compiler's wait counts are exact there: computing
// chunk k waits for chunk k's loads only, with chunks k+1 .. k+kRing-1 in
// flight.  The last (up to 2*kRing - 1) chunks run through a guarded copy.
template <int kRing, class Buf, class Issue, class Attend>
__device__ __forceinline__ void run_ring(int total, Buf (&buf)[kRing], Issue &&issue,
                                         Attend &&attend)
{
#pragma unroll
    for (int u = 0; u < kRing - 1; ++u)
        if (u < total)
            issue(buf[u], u);
    int k = 0;
    for (; k + 2 * kRing - 2 < total; k += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            issue(buf[(u + kRing - 1) % kRing], k + u + kRing - 1);
            attend(buf[u], k + u);
        }
    }
    for (;; k += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const int c = k + u;
            if (c + kRing - 1 < total)
                issue(buf[(u + kRing - 1) % kRing], c + kRing - 1);
            attend(buf[u], c);
            if (c + 1 >= total)
                return;
        }
    }
}

// One wave per (KV head, sequence) when a single partition (at most 1,024
// tokens) covers every context: the wave normalises and writes its rows.
// Several partitions run on the persistent waves of decode_balanced.hpp.
// Grid: (1, K, B).  BS: tokens per cache block (16 or 32).
template <class Fmt, int H, int BS = kBlockSize>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(DecodeParams p)
{
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x;
    const int col = lane & 15;    // query head within the group (tile column)
    const int quad = lane >> 4;   // 0..3

    // The sequence's block ids (at most 64: the partition holds <= 1024
    // tokens), one per lane, so a chunk reads its two ids with v_readlane
    // instead of a memory round trip.  They are fetched before the context
    // length is known (every entry up to the table row's end is in bounds),
    // so the two loads overlap; entries past the last block are unused.
    const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks;
    const int table_avail = min(p.part / BS, p.max_blocks);
    int my_id = 0;
    if (lane < table_avail)
        my_id = table[lane];

    const int ctx = min(max(p.context_lens[b], 0), p.max_ctx);
    const bool live = col < p.group;
    const int n = kvh * p.group + col;

    // Sliding window: positions before lo are not attended.
    const int lo = window_start(p, ctx);
    if (ctx == 0) {                       // empty sequence: zeros
        if (live) {
            float *o = p.out + ((int64_t)b * p.num_heads + n) * H;
#pragma unroll
            for (int c = 0; c < H / 16; ++c)
                *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }
    const int end = min(p.part, ctx);
    const int n_blocks = (end - 1) / BS + 1;
    my_id = clamp_block(my_id, p.num_blocks);

    bf16x8 qf[H / 32];
    {
        const uint16_t *qrow = p.q + ((int64_t)b * p.num_heads + (live ? n : 0)) * H;
#pragma unroll
        for (int s = 0; s < H / 32; ++s) {
            u32x4 raw = load16(qrow + Fmt::dim_offset(s, quad));
            if (!live)
                raw = u32x4{0u, 0u, 0u, 0u};
            qf[s] = as_bf16x8(raw ^ p.q_sign);
        }
    }

    const int64_t tile_elems = (int64_t)BS * H;                      // one (block, head) tile
    const int64_t block_elems = (int64_t)p.num_kv_heads * tile_elems;
    using Elem = typename Fmt::Elem;
    using Regs = typename Fmt::template Regs<H>;
    const Elem *kbase = static_cast<const Elem *>(p.key_cache) + kvh * tile_elems;
    const Elem *vbase = static_cast<const Elem *>(p.value_cache) + kvh * tile_elems;

    // Chunks start at cbeg: the 32-token boundary at or below the window
    // start (0 without a window).
    const int cbeg = __builtin_amdgcn_readfirstlane(lo - lo % kChunk);
    const int boff = cbeg / BS;                     // table entries before cbeg
    const int head = lo - cbeg;                      // masked leading positions of chunk 0

    // Issue the loads of chunk ci (tokens cbeg + 32ci ...); its second block
    // is addressed only if the chunk reaches into it.
    auto issue = [&](Regs &r, int ci) {
        const int k0 = boff + (kChunk / BS) * ci;
        const int id0 = __builtin_amdgcn_readlane(my_id, k0);
        const int id1 = (BS == 16 && k0 + 1 < n_blocks) ? __builtin_amdgcn_readlane(my_id, k0 + 1)
                                                        : id0;
        const uint64_t o0 = (uint64_t)id0 * block_elems, o1 = (uint64_t)id1 * block_elems;
        Fmt::template load<H, BS>(r, kbase + o0, kbase + key_hi<BS, H>(o1), vbase + o0,
                                  vbase + value_hi<BS>(o1), col, quad);
    };

    float m = -INFINITY, l = 0.f;
    f32x4 acc[H / 16];
#pragma unroll
    for (int c = 0; c < H / 16; ++c)
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int n_full = (end - cbeg) / kChunk;                 // chunks of 32 tokens below end
    const int n_chunks = n_full + ((end - cbeg) % kChunk != 0);
    const int tail_rem = end - cbeg - n_full * kChunk;
    auto qfrag = [&](int s) { return qf[s]; };
    auto attend = [&](const Regs &r, int ci) {
        const bool front = ci == 0 && head > 0;
        if (ci < n_full && !front)
            attend_chunk<Fmt, H, false>(r, qfrag, kChunk, 0, quad, p.scale_log2, m, l, acc);
        else
            attend_chunk<Fmt, H, true>(r, qfrag, ci < n_full ? kChunk : tail_rem,
                                       front ? head : 0, quad, p.scale_log2, m, l, acc);
    };

    Regs ring[Fmt::kRing];
    run_ring<Fmt::kRing>(n_chunks, ring, issue, attend);

    // Each lane summed its own 8 tokens per chunk; add the four quads.
    l = sum_over_rows(l);
    if (!live)
        return;
    // acc[c] holds O^T[16c + 4quad + i][col], i = 0..3.
    const float inv = p.out_scale / l;
    float *o = p.out + ((int64_t)b * p.num_heads + n) * H;
#pragma unroll
    for (int c = 0; c < H / 16; ++c)
        *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = acc[c] * inv;
}

// Small batches, one launch: a workgroup of kSplitWaves waves per (KV head,
// sequence).  Wave w attends chunks [n w / kSplitWaves, n (w + 1) /
// kSplitWaves) of the n chunks from the window start, then the waves' partial
// results (running maximum m, sum l, unnormalised output o, per query column)
// are combined through LDS by the log-sum-exp rule of the split-K merge:
// M = max m_w, out = sum_w 2^(m_w - M) o_w / sum_w 2^(m_w - M) l_w, taken in
// wave order.  No partials go to global memory and no merge launch follows,
// which is what a small batch spends most of its time on.  The host uses it
// when the batch's (sequence, KV head) pairs times kSplitWaves fit one round
// of waves and a context holds at most kSplitMaxBytes of keys and values
// (and at most kSplitMaxChunks chunks, so each wave's block ids fit its
// lanes): a workgroup runs on one compute unit, and past that size one
// unit's share of the bandwidth makes it slower than spreading the pair over
// the chip.
constexpr int kSplitWaves = 4;
constexpr int kSplitMaxChunks = 32 * kSplitWaves;
constexpr int64_t kSplitMaxBytes = 256 * 1024;

template <class Fmt, int H, int BS = kBlockSize>
__global__ __launch_bounds__(kWave * kSplitWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_split_kernel(DecodeParams p)
{
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int col = lane & 15;
    const int quad = lane >> 4;
    const bool live = col < p.group;
    const int n = kvh * p.group + col;
    float *o = p.out + ((int64_t)b * p.num_heads + n) * H;

    const int ctx = min(max(scalar_load(p.context_lens + b), 0), p.max_ctx);
    if (ctx == 0) {                       // empty sequence: zeros (every wave leaves here)
        if (wv == 0 && live)
#pragma unroll
            for (int c = 0; c < H / 16; ++c)
                *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = f32x4{0.f, 0.f, 0.f, 0.f};
        return;
    }
    const int lo = window_start(p, ctx);
    const int cbeg = lo - lo % kChunk;    // chunks start at the 32-token boundary below lo
    const int head = lo - cbeg;           // masked leading positions of chunk 0
    const int n_full = (ctx - cbeg) / kChunk;
    const int tail_rem = ctx - cbeg - n_full * kChunk;
    const int total = n_full + (tail_rem != 0);
    const int c0 = total * wv / kSplitWaves;
    const int n_chunks = total * (wv + 1) / kSplitWaves - c0;

    // This wave's block ids, one per lane (at most 32 chunks: 64 blocks of 16).
    const int bfirst = (cbeg + kChunk * c0) / BS;
    const int n_blocks = (ctx - 1) / BS + 1;
    const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks;
    int my_id = 0;
    if (bfirst + lane < n_blocks)
        my_id = table[bfirst + lane];
    my_id = clamp_block(my_id, p.num_blocks);

    bf16x8 qf[H / 32];
    {
        const uint16_t *qrow = p.q + ((int64_t)b * p.num_heads + (live ? n : 0)) * H;
#pragma unroll
        for (int s = 0; s < H / 32; ++s) {
            u32x4 raw = load16(qrow + Fmt::dim_offset(s, quad));
            if (!live)
                raw = u32x4{0u, 0u, 0u, 0u};
            qf[s] = as_bf16x8(raw ^ p.q_sign);
        }
    }

    const int64_t tile_elems = (int64_t)BS * H;
    const int64_t block_elems = (int64_t)p.num_kv_heads * tile_elems;
    using Elem = typename Fmt::Elem;
    using Regs = typename Fmt::template Regs<H>;
    const Elem *kbase = static_cast<const Elem *>(p.key_cache) + kvh * tile_elems;
    const Elem *vbase = static_cast<const Elem *>(p.value_cache) + kvh * tile_elems;

    auto issue = [&](Regs &r, int ci) {
        const int k0 = (kChunk / BS) * ci;    // table entry of the chunk, from bfirst
        const int id0 = __builtin_amdgcn_readlane(my_id, k0);
        const int id1 = (BS == 16 && bfirst + k0 + 1 < n_blocks)
                            ? __builtin_amdgcn_readlane(my_id, k0 + 1)
                            : id0;
        const uint64_t o0 = (uint64_t)id0 * block_elems, o1 = (uint64_t)id1 * block_elems;
        Fmt::template load<H, BS>(r, kbase + o0, kbase + key_hi<BS, H>(o1), vbase + o0,
                                  vbase + value_hi<BS>(o1), col, quad);
    };

    float m = -INFINITY, l = 0.f;
    f32x4 acc[H / 16];
#pragma unroll
    for (int c = 0; c < H / 16; ++c)
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto qfrag = [&](int s) { return qf[s]; };
    auto attend = [&](const Regs &r, int ci) {
        const int g = c0 + ci;                // chunk index from cbeg
        const bool front = g == 0 && head > 0;
        if (g < n_full && !front)
            attend_chunk<Fmt, H, false>(r, qfrag, kChunk, 0, quad, p.scale_log2, m, l, acc);
        else
            attend_chunk<Fmt, H, true>(r, qfrag, g < n_full ? kChunk : tail_rem,
                                       front ? head : 0, quad, p.scale_log2, m, l, acc);
    };
    if (n_chunks > 0) {
        Regs ring[Fmt::kRing];
        run_ring<Fmt::kRing>(n_chunks, ring, issue, attend);
    }
    l = sum_over_rows(l);                 // each lane summed its own 8 tokens per chunk

    // Partials to LDS: acc[c] holds O^T[16c + 4quad + i][col], i = 0..3; m
    // and l are the same in the four quads of a column.
    __shared__ float s_m[kSplitWaves][16];
    __shared__ float s_l[kSplitWaves][16];
    __shared__ f32x4 s_o[kSplitWaves][H / 16][kWave];
    if (quad == 0) {
        s_m[wv][col] = m;
        s_l[wv][col] = l;
    }
#pragma unroll
    for (int c = 0; c < H / 16; ++c)
        s_o[wv][c][lane] = acc[c];
    __syncthreads();

    // Wave w combines the output tiles c = w, w + kSplitWaves, ...
    float mw[kSplitWaves];
    float big = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
        mw[w] = s_m[w][col];
        big = mw[w] > -INFINITY ? fmaxf(big, mw[w]) : big;
    }
    float e[kSplitWaves];
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
        e[w] = mw[w] > -INFINITY ? __builtin_amdgcn_exp2f(mw[w] - big) : 0.f;
        den += e[w] * s_l[w][col];
    }
    if (!live)
        return;
    const float inv = den > 0.f ? p.out_scale / den : 0.f;
#pragma unroll
    for (int c = 0; c < H / 16; ++c) {
        if (c % kSplitWaves != wv)
            continue;
        f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kSplitWaves; ++w)
            sum += s_o[w][c][lane] * e[w];
        *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = sum * inv;
    }
}

struct MergeParams {
    float *out;                   // [B][Q][N][H]
    const float *part_o;          // [B][Q][N][P][H]
    const float *part_ml;         // [B][Q][N][P][2]
    const int32_t *context_lens;  // [B]
    int32_t num_queries;          // Q (1 for plain decode)
    int32_t window;               // sliding window (0 = none): earlier partitions are skipped
    int32_t num_heads;
    int32_t max_ctx;
    int32_t part;
    int32_t num_parts;
    int32_t group;                // G = N / K (merge_parts_kernel)
};

constexpr int kMergeThreads = 256;

// Sum (or max) over the 256 threads of a workgroup; every thread gets the result.
template <bool kMax>
__device__ __forceinline__ float block_reduce(float v, float *scratch)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float o = __shfl_xor(v, off);
        v = kMax ? fmaxf(v, o) : v + o;
    }
    const int wave = threadIdx.x / kWave;
    __syncthreads();                       // scratch may still be read by a previous call
    if ((threadIdx.x % kWave) == 0)
        scratch[wave] = v;
    __syncthreads();
    v = scratch[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / kWave; ++w)
        v = kMax ? fmaxf(v, scratch[w]) : v + scratch[w];
    return v;
}

// Log-sum-exp merge of the partitions of one (sequence, query token, query
// head) row, one workgroup each.  The partition maxima and weighted sums are
// reduced across the threads; then kGroups groups of H/4 threads, each
// thread four consecutive values of the row, accumulate every kGroups-th
// partition's o with 16-byte loads, kUnroll partitions in flight per thread
// (a row of hundreds of partitions is then a few memory round trips, not one
// per partition), combined through LDS.  Partition maxima are in log2 units;
// a row that saw no position in any partition (maximum -inf, sums 0) gets
// zeros.
template <int H>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p)
{
    constexpr int kLanes = H / 4;                      // threads per partition row
    constexpr int kGroups = kMergeThreads / kLanes;
    constexpr int kUnroll = 8;
    __shared__ float red[kMergeThreads / kWave];
    __shared__ f32x4 part_sum[kGroups][kLanes];

    const int n = blockIdx.x;
    const int bq = blockIdx.y;                     // b * Q + query token
    const int b = bq / p.num_queries;
    const int tid = threadIdx.x;
    const int ctx = min(max(p.context_lens[b], 0), p.max_ctx);
    const int parts = (ctx + p.part - 1) / p.part;
    const int first = p.window > 0 ? max(ctx - p.window, 0) / p.part : 0;
    const int64_t row = (int64_t)bq * p.num_heads + n;
    const float *ml = p.part_ml + row * p.num_parts * 2;
    const float *po = p.part_o + row * p.num_parts * H;

    float big = -INFINITY;
    for (int j = first + tid; j < parts; j += kMergeThreads)
        big = fmaxf(big, ml[2 * j]);
    big = block_reduce<true>(big, red);
    float den = 0.f;
    for (int j = first + tid; j < parts; j += kMergeThreads)
        den += __builtin_amdgcn_exp2f(ml[2 * j] - big) * ml[2 * j + 1];
    den = block_reduce<false>(den, red);

    const int h4 = tid % kLanes;
    const int grp = tid / kLanes;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    int j = first + grp;
    for (; j + (kUnroll - 1) * kGroups < parts; j += kUnroll * kGroups) {
        f32x4 v[kUnroll];
        float m[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int jj = j + u * kGroups;
            v[u] = *reinterpret_cast<const f32x4 *>(po + (int64_t)jj * H + 4 * h4);
            m[u] = ml[2 * jj];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            num += __builtin_amdgcn_exp2f(m[u] - big) * v[u];
    }
    for (; j < parts; j += kGroups)
        num += __builtin_amdgcn_exp2f(ml[2 * j] - big) *
               *reinterpret_cast<const f32x4 *>(po + (int64_t)j * H + 4 * h4);
    part_sum[grp][h4] = num;
    __syncthreads();
    if (grp == 0) {
        f32x4 total = part_sum[0][h4];
#pragma unroll
        for (int g2 = 1; g2 < kGroups; ++g2)
            total += part_sum[g2][h4];
        // A row with no position has big = -inf and NaN weights: select zeros.
        *reinterpret_cast<f32x4 *>(p.out + row * H + 4 * h4) =
            (parts && den > 0.f) ? total * (1.0f / den) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// The same merge for rows of few partitions (at most kMergePartsMax): one
// wave per (query row, KV head) combines the partials of the group's G heads,
// up to eight partitions per memory round trip, with the running maximum
// rescaled as it grows.  Lane layout: heads padded to Gp (a power of two >=
// G), 64/Gp lanes per head, each lane H*Gp/64 consecutive values of its
// head's row.  A partial that saw no position (m = -inf, l = 0: a query
// token of the multi-query call whose positions end before the partition)
// takes no part.  Grid: (K, B * Q).
constexpr int kMergePartsMax = 16;

template <int H, int Gp>
__global__ __launch_bounds__(kWave) void merge_parts_kernel(MergeParams p)
{
    constexpr int kLanesPerHead = kWave / Gp;
    constexpr int kVals = H / kLanesPerHead;      // values per lane (multiple of 4)
    constexpr int kBatch = kVals / 4 >= 8 ? 4 : 8;
    const int kvh = blockIdx.x;
    const int bq = blockIdx.y;                     // b * Q + query token
    const int b = bq / p.num_queries;
    const int lane = threadIdx.x;
    const int g = lane / kLanesPerHead;
    const int h0 = (lane % kLanesPerHead) * kVals;
    const bool live = g < p.group;
    const int ctx = min(max(p.context_lens[b], 0), p.max_ctx);
    const int parts = (ctx + p.part - 1) / p.part;
    const int first = p.window > 0 ? max(ctx - p.window, 0) / p.part : 0;
    const int64_t row = (int64_t)bq * p.num_heads + kvh * p.group + (live ? g : 0);
    const float *ml = p.part_ml + row * p.num_parts * 2;
    const float *po = p.part_o + row * p.num_parts * H + h0;

    float big = -INFINITY, den = 0.f;
    f32x4 num[kVals / 4];
#pragma unroll
    for (int v = 0; v < kVals / 4; ++v)
        num[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = first; j0 < parts; j0 += kBatch) {
        float mv[kBatch], lv[kBatch];
        f32x4 ov[kBatch][kVals / 4];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = min(j0 + u, parts - 1);  // in range; unused ones are masked below
            mv[u] = ml[2 * j];
            lv[u] = ml[2 * j + 1];
#pragma unroll
            for (int v = 0; v < kVals / 4; ++v)
                ov[u][v] = *reinterpret_cast<const f32x4 *>(po + (int64_t)j * H + 4 * v);
        }
        bool use[kBatch];
        float nb = big;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            use[u] = j0 + u < parts && mv[u] > -INFINITY;
            nb = use[u] ? fmaxf(nb, mv[u]) : nb;
        }
        const float sc = big == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(big - nb);
        den *= sc;
#pragma unroll
        for (int v = 0; v < kVals / 4; ++v)
            num[v] *= sc;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const float wt = use[u] ? __builtin_amdgcn_exp2f(mv[u] - nb) : 0.f;
            den += use[u] ? wt * lv[u] : 0.f;
#pragma unroll
            for (int v = 0; v < kVals / 4; ++v)
                num[v] += use[u] ? wt * ov[u][v] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        big = nb;
    }
    if (live) {
        const float inv = den > 0.f ? 1.0f / den : 0.f;
        float *o = p.out + row * H + h0;
#pragma unroll
        for (int v = 0; v < kVals / 4; ++v)
            *reinterpret_cast<f32x4 *>(o + 4 * v) = num[v] * inv;
    }
}

}  // namespace pkv
