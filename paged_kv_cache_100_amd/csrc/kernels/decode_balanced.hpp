// Token-balanced decode attention for ragged batches (continuous batching).
//
// A launch of one wave per (partition, KV head, sequence) leaves, on ragged
// contexts -- the continuous-batching mix of "CS336 Lecture 10: Inference",
// part 6 -- a tail of unequal waves and pays the start-up latency of every
// wave (context length, block ids, first loads) once per partition.  Here the
// grid is exactly the number of waves the chip holds at once, and the work is
// cut by tokens instead:
//
//   * segments s = (sequence b, KV head kvh), in order b-major; segment s has
//     nc_b = ceil(ctx_b / 32) chunks of 32 tokens (counted from the sliding
//     window's first chunk, or, for kPrefix, from the end of the positions
//     that b's prefix group reads for it);
//   * the flattened chunk list [0, T), T = K * sum_b nc_b, is split evenly:
//     wave w gets chunks [floor(w T / W), floor((w+1) T / W));
//   * a wave walks its chunks in order, crossing segment boundaries without
//     draining its load pipeline; each (wave, segment) intersection is a
//     "piece" with its own running maximum, sum and weighted V.
//
// A piece that is a whole segment is normalised and written to `out` by its
// wave.  Other pieces go to the workspace at slot w + s (unique: along the
// flattened list every wave or segment boundary starts a new piece) and the
// merge kernel combines them with the log-sum-exp rule.  With kPrefix, a
// sequence that shares positions with its prefix group never writes `out`
// from the decode wave: its pieces are merged with the group kernel's
// partials.
//
// For more than 256 sequences a one-workgroup schedule kernel runs first: it
// scans the context lengths into chunk offsets cs[b] (exclusive prefix sum of
// nc_b) and writes each wave's starting (b, kvh, chunk) so that a wave needs
// one load to begin; smaller batches are scanned inside every wave.
// Finished pieces wait in LDS until the wave's loads are done (see the
// kernel).
//
// Fixed partitions (kFixed, part_chunks chunks each) run on the same
// schedule: both ends of every wave's range move down to a partition
// boundary (a multiple of part_chunks chunks, counted from position 0 of the
// sequence), so each partition belongs to one wave, and a piece also ends at
// every partition boundary.  Each partition's partial (m, l, o) goes to its
// split-K slot, as the one-wave-per-partition grid would have written it
// (the same chunks in the same order), and the log-sum-exp merge over
// partitions finishes the rows.  The waves keep their load pipelines full
// across partitions instead of paying a start-up per partition.
#pragma once

#include "decode_prefix.hpp"
#include "pagedkv.h"

namespace pkv {

constexpr int kScheduleThreads = 1024;
constexpr int kMaxBalancedWaves = 4096;
// Waves per workgroup of the decode kernel, at most: a workgroup of four
// fills a CU (one wave per SIMD).  Dispatching 256 four-wave workgroups
// starts the last wave several microseconds sooner than 1,024 one-wave
// workgroups.  Grids of fewer waves than the chip holds use smaller
// workgroups (blockDim.x / 64 waves), which spreads them over more CUs.
constexpr int kGroupWaves = 4;

struct BalancedParams {
    DecodeParams d;               // shapes, pointers, scale (part: kFixed partitions or
                                  // kPrefix pieces; num_parts: kFixed only)
    int32_t *chunk_start;         // [B + 1]: exclusive prefix sum of nc_b (schedule output)
    int32_t *total_chunks;        // [1]: T = K * chunk_start[B]
    int4 *wave_start;             // [W]: (b, kvh, chunk in segment, ctx of b)
    float *piece_o;               // [W + B*K][G][H]
    float *piece_ml;              // [W + B*K][G][2]
    int32_t num_waves;            // W (grid size of the decode kernel), a power of two
    int32_t log2_waves;           // log2(W)
    int32_t num_seqs;             // B
    int32_t inline_schedule;      // 1: small batch, waves scan the context lengths themselves
    int32_t part_chunks;          // kFixed: chunks per partition (partials to d.part_o /
                                  // d.part_ml); else unused
    int32_t prefix_parts;         // kPrefix: prefix partials per member row (d.part_o /
                                  // d.part_ml, d.part tokens each); else unused
};

constexpr int kInlineScheduleSeqs = 256;   // largest B scanned inside every wave

__device__ __forceinline__ int chunks_of(int ctx) { return (ctx + kChunk - 1) / kChunk; }

// A segment's chunks run from the 32-token boundary at or below the sliding
// window's start (0 without a window) to the end of the context of sequence
// b.  kPrefix (shared-prefix decode, no window): from the end of the
// positions that b's prefix group reads for it (a chunk boundary).
template <bool kPrefix = false>
__device__ __forceinline__ int first_chunk(const DecodeParams &d, int b, int ctx)
{
    if constexpr (kPrefix) {
        const int shared = stored_shared_tokens(d, b);
        return ctx > 0 ? shared / kChunk : 0;
    }
    else
        return window_start(d, ctx) / kChunk;
}
template <bool kPrefix = false>
__device__ __forceinline__ int seg_chunks(const DecodeParams &d, int b, int ctx)
{
    return chunks_of(ctx) - first_chunk<kPrefix>(d, b, ctx);
}

// Uniform (scalar) value of a load whose address is the same in every lane.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int seq_ctx(const DecodeParams &d, int b)
{
    return min(max(d.context_lens[b], 0), d.max_ctx);
}

// seq_ctx for a sequence index that is the same in every lane of the wave.
__device__ __forceinline__ int seq_ctx_uniform(const DecodeParams &d, int b)
{
    return min(max(scalar_load(d.context_lens + b), 0), d.max_ctx);
}

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(v, off);
        if (lane >= off)
            v += t;
    }
    return v;
}

// floor(w * T / W): first chunk of wave w (W = 2^log2W, so no division).
__device__ __forceinline__ int wave_begin(int64_t w, int64_t T, int log2W)
{
    return (int)((w * T) >> log2W);
}
// The wave whose range holds chunk c < T: the largest w with
// floor(w T / W) <= c, i.e. w T < (c + 1) W: w = floor(((c + 1) W - 1) / T).
// One integer division (32-bit when the operands fit).
__device__ __forceinline__ int wave_of(int64_t c, int64_t T, int log2W)
{
    const uint64_t num = ((uint64_t)(c + 1) << log2W) - 1;
    const uint64_t w = (num >> 32) == 0 && (T >> 32) == 0
                           ? (uint64_t)((uint32_t)num / (uint32_t)T)
                           : num / (uint64_t)T;
    return (int)min(w, (uint64_t)((1 << log2W) - 1));
}

// ---------------------------------------------------------------- schedule --

template <bool kPrefix = false>
__global__ __launch_bounds__(kScheduleThreads) void schedule_kernel(BalancedParams p)
{
    __shared__ int32_t incl[kScheduleThreads];   // inclusive prefix of nc within the tile
    __shared__ int32_t excl[kScheduleThreads];   // exclusive prefix of nc within the tile
    __shared__ int32_t carry_s;
    const int tid = threadIdx.x;
    const int B = p.num_seqs;
    const int K = p.d.num_kv_heads;
    const int W = p.num_waves;
    const int lg = p.log2_waves;

    // Pass 1: T = K * sum_b nc_b (needed to place the wave boundaries).
    int mine = 0;
    for (int b = tid; b < B; b += kScheduleThreads)
        mine += seg_chunks<kPrefix>(p.d, b, seq_ctx(p.d, b));
    incl[tid] = mine;
    __syncthreads();
    for (int off = kScheduleThreads / 2; off >= 1; off >>= 1) {
        if (tid < off)
            incl[tid] += incl[tid + off];
        __syncthreads();
    }
    const int total_seq = incl[0];
    const int64_t T = (int64_t)total_seq * K;
    if (tid == 0) {
        carry_s = 0;
        p.total_chunks[0] = (int32_t)T;
        p.chunk_start[B] = total_seq;
    }
    __syncthreads();

    // Pass 2, one tile of sequences at a time: exclusive prefix sums (written
    // out for the merge), then the start of every wave whose first chunk
    // falls in this tile, found by binary search over the tile's prefix sums.
    for (int base = 0; base < B; base += kScheduleThreads) {
        const int b = base + tid;
        const int nc = b < B ? seg_chunks<kPrefix>(p.d, b, seq_ctx(p.d, b)) : 0;
        incl[tid] = nc;
        __syncthreads();
        for (int off = 1; off < kScheduleThreads; off <<= 1) {   // Hillis-Steele scan
            const int v = tid >= off ? incl[tid - off] : 0;
            __syncthreads();
            incl[tid] += v;
            __syncthreads();
        }
        excl[tid] = incl[tid] - nc;
        const int carry = carry_s;
        if (b < B)
            p.chunk_start[b] = carry + incl[tid] - nc;
        __syncthreads();
        const int tile_n = min(kScheduleThreads, B - base);
        const int64_t lo = (int64_t)carry * K;
        const int64_t hi = (int64_t)(carry + incl[tile_n - 1]) * K;
        for (int w = tid; w < W; w += kScheduleThreads) {
            const int64_t c0 = wave_begin(w, T, lg);
            if (c0 < lo || c0 >= hi)
                continue;
            // largest i with (carry + excl[i]) * K <= c0: the sequence holding c0
            int left = 0, right = tile_n - 1;
            while (left < right) {
                const int mid = (left + right + 1) >> 1;
                if ((int64_t)(carry + excl[mid]) * K <= c0)
                    left = mid;
                else
                    right = mid - 1;
            }
            const int ncb = incl[left] - excl[left];
            const int local = (int)(c0 - (int64_t)(carry + excl[left]) * K);
            const int kvh = local / ncb;
            p.wave_start[w] = make_int4(base + left, kvh, local - kvh * ncb,
                                        seq_ctx(p.d, base + left));
        }
        __syncthreads();
        if (tid == tile_n - 1)
            carry_s = carry + incl[tid];
        __syncthreads();
    }
}

// ------------------------------------------------------------------ decode --

// Staged results of the decode waves (see decode_balanced_kernel).
constexpr uint32_t kStageDead = 0;      // lane of a column past the group: nothing
constexpr uint32_t kStageFinal = 1;     // a whole segment: normalised row of `out`
constexpr uint32_t kStagePiece = 2;     // a piece: piece_o / piece_ml row
constexpr uint32_t kStagePartial = 3;   // a fixed partition: part_o / part_ml row

// LDS a decode wave stages finished pieces in (eight pieces of a group of 8
// at H = 128): with the per-column records 37 KiB per wave, so a workgroup
// of four waves (one CU) takes 148 KiB of its 160 KiB.
constexpr int kStageBytes = 32 * 1024;
constexpr int kStageMax = 16;      // pieces staged at most

// Position of one chunk in the flattened order: segment (b, kvh), chunk j of
// the nc chunks of sequence b (ctx tokens); the segment's chunk j covers
// positions 32 * (fc + j) .. (fc counts the chunks before the sliding window).
struct Pos {
    int b, kvh, j, nc, ctx, fc;
    const int32_t *row;   // sequence b's block-table row
    int nblk;             // its blocks: ceil(ctx / 16)
};

// One ring slot: the chunk's key/value operands, plus the group's query
// rows when the chunk opens a segment (or is the wave's first chunk).
template <class Fmt, int H>
struct BalancedBuf {
    typename Fmt::template Regs<H> kv;
    u32x4 q[H / 32];
};

// kGroupTiles > 0 (with kPrefix): the grid also holds the prefix groups'
// waves (prefix_group_wave, kGroupTiles tiles each) after the W persistent
// ones; they share the stage's LDS.  For small batches they also store the
// shared spans for the merge, which the persistent waves compute for
// themselves.
template <class Fmt, int H, bool kFixed = false, bool kPrefix = false, int kGroupTiles = 0,
          int BS = kBlockSize>
__global__ __launch_bounds__(kWave * kGroupWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_balanced_kernel(BalancedParams p)
{
    using Elem = typename Fmt::Elem;
    using Buf = BalancedBuf<Fmt, H>;
    const DecodeParams &d = p.d;
    // Wave wv of the grid is wave wig of workgroup blockIdx.x; the waves of a
    // workgroup share nothing but the CU (each has its own LDS slice).
    // (read from the first lane: the compiler must see the wave index as
    // uniform, or everything derived from it leaves the scalar unit)
    const int wig = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int wv = (int)blockIdx.x * ((int)blockDim.x / kWave) + wig;
    const int lane = (int)threadIdx.x % kWave;
    __shared__ f32x4 stage_all[kGroupWaves][kStageBytes / 16];   // staged pieces (see below)
    f32x4 *stage_o = stage_all[wig];
    if constexpr (kGroupTiles > 0) {
        static_assert(kPrefix && kGroupTiles * (H / 32) * kWave * 16 <= kStageBytes,
                      "group queries fit the stage");
        if (wv >= p.num_waves) {
            prefix_group_wave<Fmt, H, kGroupTiles, BS>(d, p.prefix_parts, wv - p.num_waves,
                                                   reinterpret_cast<u32x4 *>(stage_o),
                                                   p.inline_schedule != 0);
            return;
        }
    }
    if (wv >= p.num_waves)           // the last workgroup's spare waves
        return;
    const int col = lane & 15;
    const int quad = lane >> 4;
    const int K = d.num_kv_heads;
    const int B = p.num_seqs;
    const bool live = col < d.group;

    // Where this wave starts: (sequence, KV head, chunk) and that sequence's
    // context length.  Small batches: every wave loads all context lengths
    // at once (one round trip) and scans them; large ones: the schedule
    // kernel's table.
    int64_t T;
    int4 st = make_int4(0, 0, 0, 0);
    int4 st_end = make_int4(0, 0, 0, 0);   // kFixed: the position of c_end (x, z, w used)
    int c_begin, c_end;
    // kPrefix, small batches: S_b of sequence t * 64 + lane, computed here
    // from the groups (larger batches read d.shared_tokens, which a kernel
    // before this one stores).
    constexpr int kTiles = kInlineScheduleSeqs / kWave;
    int shv[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
        shv[t] = 0;
    // kPrefix: first chunk of sequence b's segments (b the same in every
    // lane); the other instances call first_chunk / seg_chunks directly.
    auto fc_at = [&](int b, int ctx) {
        if (!p.inline_schedule)
            return first_chunk<kPrefix>(d, b, ctx);
        int span = 0;
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
            span = (b >> 6) == t ? __builtin_amdgcn_readlane(shv[t], b & 63) : span;
        return ctx > 0 ? span / kChunk : 0;
    };
    auto nc_at = [&](int b, int ctx) { return chunks_of(ctx) - fc_at(b, ctx); };
    if (p.inline_schedule) {
        int cx[kTiles];
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            const int b = t * kWave + lane;
            cx[t] = b < B ? seq_ctx(d, b) : 0;
            if constexpr (kPrefix)
                shv[t] = b < B && d.shared_tokens ? prefix_shared_tokens(d, b) : 0;
        }
        // kPrefix: chunks of the lane's sequence in tile t.
        auto nc_lane = [&](int t) { return chunks_of(cx[t]) - (cx[t] > 0 ? shv[t] / kChunk : 0); };
        int total_seq = 0;
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
            if (t * kWave < B) {           // tiles past the batch hold zeros
                if constexpr (kPrefix)
                    total_seq += wave_sum(nc_lane(t));
                else
                    total_seq += wave_sum(seg_chunks<kPrefix>(d, t * kWave + lane, cx[t]));
            }
        T = (int64_t)uniform(total_seq) * K;
        // Wave 0 also stores the schedule's per-sequence chunk offsets and
        // T, as schedule_kernel does for larger batches: the merge launch
        // then reads two values per segment instead of scanning every
        // context length in each of its waves.
        if (wv == 0) {
            int carry0 = 0;
#pragma unroll
            for (int t = 0; t < kTiles; ++t) {
                if (t * kWave >= B)
                    break;
                int nc;
                if constexpr (kPrefix)
                    nc = nc_lane(t);
                else
                    nc = seg_chunks<kPrefix>(d, t * kWave + lane, cx[t]);
                const int incl = wave_inclusive_scan(nc, lane);
                if (t * kWave + lane < B)
                    p.chunk_start[t * kWave + lane] = carry0 + incl - nc;
                carry0 += __shfl(incl, kWave - 1);
            }
            if (lane == 0) {
                p.total_chunks[0] = (int32_t)T;
                p.chunk_start[B] = carry0;
            }
        }
        if (T == 0)
            return;
        c_begin = wave_begin(wv, T, p.log2_waves);
        c_end = wave_begin(wv + 1, T, p.log2_waves);
        if (c_begin >= c_end)
            return;
        // The sequence holding chunk c_begin: the last b whose chunks start at
        // or before it (empty sequences start where the next one does).  With
        // fixed partitions, also the position of c_end (the next wave's start).
        int carry = 0;
        bool found = false, found_end = !kFixed || c_end >= T;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            int nc;
            if constexpr (kPrefix)
                nc = nc_lane(t);
            else
                nc = seg_chunks<kPrefix>(d, t * kWave + lane, cx[t]);
            const int incl = wave_inclusive_scan(nc, lane);
            const int tile_total = __shfl(incl, kWave - 1);
            if (!found && (int64_t)(carry + tile_total) * K > c_begin) {
                const int excl = carry + incl - nc;
                const uint64_t mask = __builtin_amdgcn_ballot_w64(t * kWave + lane < B &&
                                                                  (int64_t)excl * K <= c_begin);
                const int src = 63 - __builtin_clzll(mask);
                const int ncb = __shfl(nc, src);
                const int local = c_begin - __shfl(excl, src) * K;
                const int kvh = local / ncb;
                st = make_int4(t * kWave + src, kvh, local - kvh * ncb, __shfl(cx[t], src));
                found = true;
            }
            if (kFixed && !found_end && (int64_t)(carry + tile_total) * K > c_end) {
                const int excl = carry + incl - nc;
                const uint64_t mask = __builtin_amdgcn_ballot_w64(t * kWave + lane < B &&
                                                                  (int64_t)excl * K <= c_end);
                const int src = 63 - __builtin_clzll(mask);
                const int ncb = __shfl(nc, src);
                const int local = c_end - __shfl(excl, src) * K;
                st_end = make_int4(t * kWave + src, 0, local - (local / ncb) * ncb,
                                   __shfl(cx[t], src));
                found_end = true;
            }
            carry += tile_total;
        }
    } else {
        T = (int64_t)uniform(p.total_chunks[0]);
        if (T == 0)
            return;
        c_begin = wave_begin(wv, T, p.log2_waves);
        c_end = wave_begin(wv + 1, T, p.log2_waves);
        if (c_begin >= c_end)
            return;
        st = p.wave_start[wv];
        if (kFixed && c_end < T)
            st_end = p.wave_start[wv + 1];
    }
    const int pc = p.part_chunks;
    if constexpr (kFixed) {
        // Fixed partitions: move both ends down to a partition boundary (the
        // next wave moves its start the same way).  back(b, j, ctx): chunks
        // from the start of chunk j's partition (or of the segment) to chunk j.
        auto back = [&](int b, int j, int ctx) {
            const int fc = first_chunk<kPrefix>(d, b, min(max(ctx, 0), d.max_ctx));
            return j - (max(fc, ((fc + j) / pc) * pc) - fc);
        };
        const int ob = back(uniform(st.x), uniform(st.z), uniform(st.w));
        const int oe =
            c_end < T ? back(uniform(st_end.x), uniform(st_end.z), uniform(st_end.w)) : 0;
        c_begin -= ob;
        st.z = uniform(st.z) - ob;
        c_end -= oe;
        if (c_begin >= c_end)
            return;
    }
    const int total = c_end - c_begin;           // chunks of this wave

    Pos start;
    start.b = uniform(st.x);
    start.kvh = uniform(st.y);
    start.j = uniform(st.z);
    start.ctx = min(max(uniform(st.w), 0), d.max_ctx);
    start.row = d.block_tables + (int64_t)start.b * d.max_blocks;
    start.nblk = (start.ctx + BS - 1) / BS;
    if constexpr (kPrefix) {
        start.nc = nc_at(start.b, start.ctx);
        start.fc = fc_at(start.b, start.ctx);
    } else {
        start.nc = seg_chunks<kPrefix>(d, start.b, start.ctx);
        start.fc = first_chunk<kPrefix>(d, start.b, start.ctx);
    }
    if (start.j >= start.nc)          // cannot happen for a consistent schedule
        return;

    // The chunk after q in flattened order (the caller knows one exists).
    auto next_seq = [&](int b) {      // next sequence after b with chunks
        int nb = b + 1;
        int ctx = nb < B ? seq_ctx_uniform(d, nb) : 0;
        // Without kPrefix only an empty context has no chunks; with it, so has
        // a sharer whose context lies wholly in its group's partitions.
        if constexpr (kPrefix) {
            while (nc_at(nb, ctx) == 0 && nb + 1 < B) {
                ++nb;
                ctx = seq_ctx_uniform(d, nb);
            }
        } else {
            while (ctx == 0 && nb + 1 < B) {
                ++nb;
                ctx = seq_ctx_uniform(d, nb);
            }
        }
        return make_int2(nb, ctx);
    };
    auto next_pos = [&](Pos &q) {
        if (++q.j < q.nc)
            return;
        q.j = 0;
        if (++q.kvh < K)
            return;
        q.kvh = 0;
        const int2 nx = next_seq(q.b);
        q.b = nx.x;
        q.ctx = nx.y;
        q.row = d.block_tables + (int64_t)q.b * d.max_blocks;
        q.nblk = (q.ctx + BS - 1) / BS;
        if constexpr (kPrefix) {
            q.nc = nc_at(q.b, q.ctx);
            q.fc = fc_at(q.b, q.ctx);
        } else {
            q.nc = seg_chunks<kPrefix>(d, q.b, q.ctx);
            q.fc = first_chunk<kPrefix>(d, q.b, q.ctx);
        }
    };

    constexpr uint32_t tile_elems = BS * H;
    const uint32_t block_elems = (uint32_t)K * tile_elems;   // < 2^31 (K <= 65535)
    const uint32_t id_lim = id_bound(d.num_blocks);
    const Elem *kcache = static_cast<const Elem *>(d.key_cache);
    const Elem *vcache = static_cast<const Elem *>(d.value_cache);

    // ---- issue side: its own cursor; each chunk's two block ids are loaded
    // one chunk ahead (load_chunk_ids) ----
    Pos ip = start;
    ChunkIds ids = load_chunk_ids<BS>(ip.row, ip.fc + ip.j, ip.nblk);
    auto issue = [&](Buf &r, int k) {
        // ip is chunk k; ids are its blocks
        const uint64_t head_off = (uint32_t)ip.kvh * tile_elems;
        const uint64_t o0 = head_off + block_offset(ids.raw0, id_lim, block_elems);
        const uint64_t o1 = head_off + block_offset(ids.raw1, id_lim, block_elems);
        Fmt::template load<H, BS>(r.kv, kcache + o0, kcache + key_hi<BS, H>(o1), vcache + o0,
                                  vcache + value_hi<BS>(o1), col, quad);
        if (k == 0 || ip.j == 0) {    // the chunk opens a segment: bring its queries
            // Columns past the group repeat its last query; their results are
            // never stored.
            const int n = ip.kvh * d.group + min(col, d.group - 1);
            const uint16_t *qrow = d.q + ((int64_t)ip.b * d.num_heads + n) * H;
#pragma unroll
            for (int s = 0; s < H / 32; ++s)
                r.q[s] = load16(qrow + Fmt::dim_offset(s, quad));
        }
        if (k + 1 < total) {          // step to chunk k + 1 and fetch its block ids
            next_pos(ip);
            ids = load_chunk_ids<BS>(ip.row, ip.fc + ip.j, ip.nblk);
        }
    };

    // ---- attend side: its own cursor, the running softmax state ----
    Pos ap = start;
    u32x4 qcur[H / 32];
    float m = -INFINITY, l = 0.f;
    f32x4 acc[H / 16];
#pragma unroll
    for (int c = 0; c < H / 16; ++c)
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool piece_from_start = start.j == 0;   // this wave's piece began at the segment start

    // Finished pieces are staged in LDS (each lane its own values, the
    // quad-0 lane of a column its row, m and l) and written out once the
    // load pipeline has drained, or when the stage is
    // full: a global store issued while chunk loads are in flight turns the
    // next wait for chunk data into a wait for everything outstanding
    // (loads and stores share one completion counter and may complete out
    // of order), which stalls the wave for a full memory latency.
    // Only the G live columns are kept: a piece takes G * H * 4 bytes, so
    // the stage holds more pieces for smaller groups (up to kStageMax).
    __shared__ int64_t stage_row_all[kGroupWaves][kStageMax][16];   // destination row of each column
    __shared__ float stage_m_all[kGroupWaves][kStageMax][16];
    __shared__ float stage_l_all[kGroupWaves][kStageMax][16];
    __shared__ uint32_t stage_kind_all[kGroupWaves][kStageMax][16];
    auto &stage_row = stage_row_all[wig];
    auto &stage_m = stage_m_all[wig];
    auto &stage_l = stage_l_all[wig];
    auto &stage_kind = stage_kind_all[wig];
    const int G = d.group;
    const int slot_vecs = G * H / 4;                // f32x4 per staged piece
    const int cap = min(kStageMax, (kStageBytes / 16) / slot_vecs);
    int staged = 0;
    auto flush = [&]() {
        if (live) {
            for (int s = 0; s < staged; ++s) {
                const uint32_t kind = stage_kind[s][col];
                const int64_t row = stage_row[s][col];
                float *o = (kind == kStageFinal ? d.out
                                                : kind == kStagePiece ? p.piece_o : d.part_o) +
                           row * H;
                const f32x4 *src = stage_o + s * slot_vecs + quad * G + col;
#pragma unroll
                for (int c = 0; c < H / 16; ++c)
                    *reinterpret_cast<f32x4 *>(o + 16 * c + 4 * quad) = src[4 * c * G];
                if (kind != kStageFinal && quad == 0) {
                    float *ml = kind == kStagePiece ? p.piece_ml : d.part_ml;
                    ml[2 * row] = stage_m[s][col];
                    ml[2 * row + 1] = stage_l[s][col];
                }
            }
        }
        staged = 0;
    };
    // kFixed: partition of the current chunk and chunks left in it
    // (counting the current one); divisions only where a segment begins.
    int pidx = 0, pleft = 0;
    auto qfrag = [&](int s) { return as_bf16x8(qcur[s]); };

    auto attend = [&](const Buf &r, int k) {
        if (k > 0)
            next_pos(ap);
        if (k == 0 || ap.j == 0) {
#pragma unroll
            for (int s = 0; s < H / 32; ++s)
                qcur[s] = r.q[s] ^ d.q_sign;
            if constexpr (kFixed) {
                const int a = ap.fc + ap.j;
                pidx = a / pc;
                pleft = pc - (a - pidx * pc);
            }
        }
        const bool seg_end = ap.j + 1 == ap.nc;
        // Leading positions of a segment's first chunk before the window start.
        const int head = ap.j == 0 ? window_start(d, ap.ctx) - kChunk * ap.fc : 0;
        if ((!seg_end || ap.ctx % kChunk == 0) && head == 0)
            attend_chunk<Fmt, H, false>(r.kv, qfrag, kChunk, 0, quad, d.scale_log2, m, l, acc);
        else
            attend_chunk<Fmt, H, true>(r.kv, qfrag, ap.ctx - kChunk * (ap.fc + ap.j), head, quad,
                                       d.scale_log2, m, l, acc);
        if constexpr (kFixed) {
            if (!seg_end && pleft != 1 && k + 1 < total) {
                --pleft;
                return;
            }
        } else {
            if (!seg_end && k + 1 < total)
                return;
        }
        // The piece ends here (segment end, partition end with kFixed, or the
        // wave's last chunk): stage it.
        if (staged == cap)
            flush();
        const float lt = sum_over_rows(l);
        if (live) {
            const int n = ap.kvh * G + col;
            uint32_t kind;
            int64_t row;
            float scl = d.out_scale;
            if (kFixed) {                               // a partition's split-K partial
                kind = kStagePartial;
                row = ((int64_t)ap.b * d.num_heads + n) * d.num_parts + pidx;
            } else if (piece_from_start && seg_end && !(kPrefix && ap.fc > 0)) {
                // the whole segment (and no prefix partials to join): final output
                kind = kStageFinal;
                row = (int64_t)ap.b * d.num_heads + n;
                scl = d.out_scale / lt;
            } else {
                kind = kStagePiece;
                row = ((int64_t)wv + (int64_t)ap.b * K + ap.kvh) * G + col;
            }
            f32x4 *dst = stage_o + staged * slot_vecs + quad * G + col;
#pragma unroll
            for (int c = 0; c < H / 16; ++c)
                dst[4 * c * G] = acc[c] * scl;
            if (quad == 0) {
                stage_kind[staged][col] = kind;
                stage_row[staged][col] = row;
                stage_m[staged][col] = m;
                stage_l[staged][col] = lt;
            }
        }
        ++staged;
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int c = 0; c < H / 16; ++c)
            acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        piece_from_start = true;                    // the next piece opens a segment
        if constexpr (kFixed) {                     // the next chunk opens a partition
            ++pidx;
            pleft = pc;
        }
    };

    Buf ring[Fmt::kBalancedRing];
    run_ring<Fmt::kBalancedRing>(total, ring, issue, attend);
    flush();
}

// ------------------------------------------------------------------- merge --

// One wave per segment (sequence, KV head): combines the pieces of the
// segment for all G query heads of its group, or writes zeros for an empty
// sequence.  Segments held whole by one wave were written by that wave and
// are skipped.  The segment's pieces are the waves that hold its chunks:
// with at least as many chunks as waves (T >= W) every wave holds one or
// more, so they are the waves w_first .. w_last; with fewer (T < W) every
// wave holds at most one, so they are the waves of its nc chunks, and the
// empty waves between them are never read.
// Lane layout: heads padded to Gp (a power of two >= G), 64/Gp lanes per
// head, each lane VPL = H*Gp/64 consecutive values of its head's row; a
// piece's G rows are contiguous, so each piece is one coalesced read.
// kPrefix: the row of a sequence with shared positions also joins its prefix
// group's partials (ceil(S_b / P) of them, ahead of its pieces), also when
// one wave holds the whole segment or the context has no chunk of its own.
template <int H, int Gp, bool kPrefix = false>
__global__ __launch_bounds__(kWave) void merge_pieces_kernel(BalancedParams p)
{
    constexpr int kLanesPerHead = kWave / Gp;
    constexpr int kVals = H / kLanesPerHead;      // values per lane (multiple of 4)
    // Pieces per memory round trip: up to 8, within about 128 registers of rows.
    constexpr int kBatch = kVals / 4 >= 8 ? 4 : 8;
    const DecodeParams &d = p.d;
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    const int g = lane / kLanesPerHead;
    const int h0 = (lane % kLanesPerHead) * kVals;
    const bool live = g < d.group;
    const int K = d.num_kv_heads;
    const int lg = p.log2_waves;

    // The schedule's sequence offsets and T, stored by schedule_kernel or
    // (batches it does not run for) by the decode launch's wave 0.
    const int nc = seg_chunks<kPrefix>(d, b, seq_ctx_uniform(d, b));
    const int64_t T = scalar_load(p.total_chunks);
    const int64_t seq_first = scalar_load(p.chunk_start + b);
    int n_pre = 0;                        // prefix partials of this row
    if constexpr (kPrefix)
        n_pre = uniform((stored_shared_tokens(d, b) + d.part - 1) / d.part);
    float *o = d.out + ((int64_t)b * d.num_heads + kvh * d.group + g) * H + h0;
    if (nc == 0 && n_pre == 0) {
        if (live)
#pragma unroll
            for (int v = 0; v < kVals; v += 4)
                *reinterpret_cast<f32x4 *>(o + v) = f32x4{0.f, 0.f, 0.f, 0.f};
        return;
    }
    const bool sparse = T < ((int64_t)1 << lg);   // fewer chunks than waves
    const int64_t first = seq_first * K + (int64_t)kvh * nc;
    int w_first = 0, count = 0;
    if (nc > 0) {
        w_first = wave_of(first, T, lg);
        const int w_last = wave_of(first + nc - 1, T, lg);
        if (w_first == w_last && n_pre == 0)
            return;
        count = sparse ? nc : w_last - w_first + 1;
    }
    const int64_t seg = (int64_t)b * K + kvh;
    const int total = n_pre + count;      // inputs: prefix partials, then pieces
    const int gg = live ? g : 0;
    // Input i: prefix partial i (rows ((b K + kvh) prefix_parts + i) G + g'),
    // else piece j = i - n_pre, written by wave w_first + j (or, sparse, by
    // the wave of chunk first + j) at rows (w + seg) G + g'.
    auto row_of = [&](int i) -> int64_t {
        if (i < n_pre)
            return (seg * p.prefix_parts + i) * d.group + gg;
        const int j = i - n_pre;          // a piece exists, so nc > 0 and T > 0
        const int64_t w = sparse ? wave_of(first + j, T, lg) : (int64_t)w_first + j;
        return (w + seg) * d.group + gg;
    };

    // Pieces are combined kBatch at a time: every load of a batch in one
    // memory round trip, then the batch joins the running log-sum-exp state
    // (maximum `big`, denominator `den`, numerator `num`), rescaled when the
    // maximum grows.  Most segments span at most kBatch waves: one round trip.
    float big = -INFINITY, den = 0.f;
    f32x4 num[kVals / 4];
#pragma unroll
    for (int v = 0; v < kVals / 4; ++v)
        num[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < total; i0 += kBatch) {
        float mv[kBatch], lv[kBatch];
        f32x4 ov[kBatch][kVals / 4];
        auto load_input = [&](int u, int i) {
            const bool pre = kPrefix && i < n_pre;
            const int64_t r = row_of(i);
            const float *mlp = pre ? d.part_ml : p.piece_ml;
            const float *op = pre ? d.part_o : p.piece_o;
            mv[u] = mlp[2 * r];
            lv[u] = mlp[2 * r + 1];
#pragma unroll
            for (int v = 0; v < kVals / 4; ++v)
                ov[u][v] = *reinterpret_cast<const f32x4 *>(op + r * H + h0 + 4 * v);
        };
        // A full batch loads straight through; the last, partial one loads
        // only its live inputs (most segments have two or three pieces).
        if (i0 + kBatch <= total) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                load_input(u, i0 + u);
        } else {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                mv[u] = -INFINITY;
                lv[u] = 0.f;
#pragma unroll
                for (int v = 0; v < kVals / 4; ++v)
                    ov[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (i0 + u < total)
                    load_input(u, i0 + u);
            }
        }
        bool use[kBatch];
        float nb = big;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u;
            use[u] = i < total;
            nb = use[u] ? fmaxf(nb, mv[u]) : nb;
        }
        // Every input covers at least one position, so nb is finite from the
        // first batch on.
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
        const float inv = 1.0f / den;
#pragma unroll
        for (int v = 0; v < kVals / 4; ++v)
            *reinterpret_cast<f32x4 *>(o + 4 * v) = num[v] * inv;
    }
}

}  // namespace pkv
