// C ABI of the paged-KV library: host-side argument checks, launch shapes and
// kernel launches.  Declarations and their documentation: include/pagedkv.h.
#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <atomic>
#include <mutex>
#include <random>

#include "pagedkv.h"
#include "kernels/append.hpp"
#include "kernels/decode.hpp"
#include "kernels/decode_balanced.hpp"
#include "kernels/decode_multi.hpp"
#include "kernels/decode_prefix.hpp"
#include "kernels/stream_read.hpp"

namespace {

constexpr int kVersionMajor = 1;
constexpr int kVersionMinor = 6;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool supported_head_dim(int32_t h) { return h == 64 || h == 128; }
bool supported_block_size(int32_t bs) { return bs == 16 || bs == 32; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Fixed-partition mode: partial results ([B][N][P][H] o, then [B][N][P][2]
// (m, l)), then the schedule of the single-query path's persistent waves
// (T, chunk offsets, wave starts); 0 bytes when one partition covers the
// context.
struct FixedLayout {
    size_t total, part_o, part_ml, total_chunks, chunk_start, wave_start;
};

FixedLayout fixed_layout(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_ctx,
                         int32_t part)
{
    FixedLayout L{};
    const int64_t parts = ceil_div(max_ctx, part);
    if (parts <= 1)
        return L;
    const int64_t rows = (int64_t)num_seqs * num_heads * parts;
    size_t off = 0;
    L.part_o = off;
    off = align256(off + (size_t)(rows * head_dim * 4));
    L.part_ml = off;
    off = align256(off + (size_t)(rows * 2 * 4));
    L.total_chunks = off;
    off = align256(off + 16);
    L.chunk_start = off;
    off = align256(off + (size_t)(num_seqs + 1) * 4);
    L.wave_start = off;
    off = align256(off + (size_t)pkv::kMaxBalancedWaves * 16);
    L.total = off;
    return L;
}

size_t fixed_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                             int32_t max_ctx, int32_t part)
{
    return fixed_layout(num_seqs, num_heads, head_dim, max_ctx, part).total;
}

// The partials alone (the multi-query path, which runs one wave per
// partition and needs no schedule).
size_t partials_bytes(int32_t num_rows, int32_t num_heads, int32_t head_dim, int32_t max_ctx,
                      int32_t part)
{
    const int64_t parts = ceil_div(max_ctx, part);
    if (parts <= 1)
        return 0;
    const int64_t rows = (int64_t)num_rows * num_heads * parts;
    return align256((size_t)(rows * head_dim * 4)) + (size_t)(rows * 2 * 4);
}

// The multi-query call's workspace: the partials, and for exactly two
// partitions per context the pair tags after them (one per (sequence, KV
// head) pair of partition waves; sized by num_seqs * num_heads, a bound of
// num_seqs * K * column groups).
size_t mq_pair_tags_offset(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                           int32_t head_dim, int32_t max_ctx, int32_t part)
{
    const int64_t rows = (int64_t)num_seqs * num_queries;
    return align256(partials_bytes((int32_t)(rows > INT32_MAX ? INT32_MAX : rows), num_heads,
                                   head_dim, max_ctx, part));
}

size_t mq_workspace_bytes(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                          int32_t head_dim, int32_t max_ctx, int32_t part)
{
    const size_t base = mq_pair_tags_offset(num_seqs, num_queries, num_heads, head_dim, max_ctx,
                                            part);
    if (ceil_div(max_ctx, part) != 2)
        return partials_bytes((int32_t)((int64_t)num_seqs * num_queries > INT32_MAX
                                             ? INT32_MAX
                                             : (int64_t)num_seqs * num_queries),
                              num_heads, head_dim, max_ctx, part);
    return base + align256((size_t)num_seqs * num_heads * 8);
}

// A fresh tag value per two-partition multi-query call: a process-wide
// counter from a random start, never 0.
uint64_t next_pair_epoch()
{
    static std::atomic<uint64_t> counter{[] {
        std::random_device rd;
        return ((uint64_t)rd() << 32) ^ (uint64_t)rd();
    }()};
    uint64_t e;
    do
        e = counter.fetch_add(1, std::memory_order_relaxed);
    while (e == 0);
    return e;
}

// Token-balanced mode: the layout of its workspace, sized for the largest
// wave count any device uses (so the size does not depend on the device).
struct BalancedLayout {
    size_t total, chunk_start, total_chunks, wave_start, piece_ml, piece_o;
};

BalancedLayout balanced_layout(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim)
{
    const int64_t group = num_heads / num_kv_heads;
    const int64_t pieces = (int64_t)pkv::kMaxBalancedWaves + (int64_t)num_seqs * num_kv_heads;
    BalancedLayout L;
    size_t off = 0;
    L.total_chunks = off;
    off = align256(off + 16);
    L.chunk_start = off;
    off = align256(off + (size_t)(num_seqs + 1) * 4);
    L.wave_start = off;
    off = align256(off + (size_t)pkv::kMaxBalancedWaves * 16);
    L.piece_ml = off;
    off = align256(off + (size_t)(pieces * group * 2 * 4));
    L.piece_o = off;
    off = align256(off + (size_t)(pieces * group * head_dim * 4));
    L.total = off;
    return L;
}

// Shared-prefix decode: the token-balanced layout, then the prefix group
// kernel's partials, prefix_parts per (sequence, query head) row: [B][K]
// [prefix_parts][G] rows of head_dim values, and their (m, l) pairs; then
// every sequence's shared span S_b (int32).
struct PrefixLayout {
    BalancedLayout bal;
    size_t pre_o, pre_ml, shared, total;
};

// Partitions of the longest shared span: its positions are a whole number of
// chunks (the bound rounded down), cut into partitions of `part` tokens.
int64_t prefix_parts_of(int32_t max_context_len, int32_t part, int32_t max_prefix_tokens)
{
    const int64_t span = (int64_t)(max_prefix_tokens < max_context_len ? max_prefix_tokens
                                                                        : max_context_len);
    if (span <= 0 || part <= 0)
        return 0;
    return ceil_div(span / pkv::kChunk * pkv::kChunk, part);
}

PrefixLayout prefix_layout(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int64_t prefix_parts)
{
    PrefixLayout L;
    L.bal = balanced_layout(num_seqs, num_heads, num_kv_heads, head_dim);
    const int64_t rows = (int64_t)num_seqs * num_heads * prefix_parts;
    size_t off = L.bal.total;
    L.pre_o = off;
    off = align256(off + (size_t)(rows * head_dim * 4));
    L.pre_ml = off;
    off = align256(off + (size_t)(rows * 2 * 4));
    L.shared = off;
    off = align256(off + (size_t)num_seqs * 4);
    L.total = off;
    return L;
}

// The kernels take the softmax scale in log2 units as a positive number: they
// apply it to a chunk's maximum score and fuse it into each exponent.  A
// negative scale is carried by flipping the query's signs (exact in bf16:
// every score changes sign).  A magnitude below FLT_MIN, zero included, is
// raised to FLT_MIN: for any score below 2^100 in magnitude the exponents
// then stay within 2^-26 of 0 and round to weight 1, which is what a zero
// scale gives.
void set_softmax_scale(pkv::DecodeParams &p, float scale, float k_scale)
{
    float s = scale * k_scale * 1.4426950408889634f;
    p.q_sign = s < 0.f ? 0x80008000u : 0u;
    s = fabsf(s);
    p.scale_log2 = s < FLT_MIN ? FLT_MIN : s;
}

// Waves the decode kernel keeps resident: one per SIMD, four SIMDs per CU.
// The balanced schedule uses the largest power of two not above that, so
// that wave boundaries need no division.
constexpr int kWavesPerCU = 4;
constexpr int64_t kMinChunksPerWave = 4;
constexpr int64_t kPiecesPerMergeBatch = 8;   // merge_pieces_kernel's batch at H = 128

int device_waves(int *log2_waves)
{
    static std::atomic<int> cached[64];   // zero-initialised; written once per device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return PKV_ERR_DEVICE;
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *log2_waves = c;
            return PKV_OK;
        }
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return PKV_ERR_DEVICE;
    int lg = 0;
    while ((2 << lg) <= cus * kWavesPerCU && (2 << lg) <= pkv::kMaxBalancedWaves)
        ++lg;
    if (dev < 64)
        cached[dev].store(lg, std::memory_order_relaxed);
    *log2_waves = lg;
    return PKV_OK;
}

// Merge kernel of the balanced schedule for a head dim and group size: the
// group is padded to a power of two, and to at least 256/H so that every
// lane owns a whole 16-byte slice of a row.
template <int H, bool kPrefix>
const void *merge_pieces_h(int group)
{
    constexpr int kMin = 256 / H;
    const int gp = group <= kMin ? kMin : group <= 4 ? 4 : group <= 8 ? 8 : 16;
    switch (gp) {
    case 2: return (const void *)pkv::merge_pieces_kernel<H, (kMin > 2 ? kMin : 2), kPrefix>;
    case 4: return (const void *)pkv::merge_pieces_kernel<H, 4, kPrefix>;
    case 8: return (const void *)pkv::merge_pieces_kernel<H, 8, kPrefix>;
    default: return (const void *)pkv::merge_pieces_kernel<H, 16, kPrefix>;
    }
}

template <bool kPrefix>
const void *merge_pieces_for(int head_dim, int group)
{
    return head_dim == 128 ? merge_pieces_h<128, kPrefix>(group)
                           : merge_pieces_h<64, kPrefix>(group);
}

// True when `stream` is being captured into a graph (or its state cannot be
// read).  A graph replays each launch with the arguments fixed at capture,
// so a launch that relies on a fresh per-call value must not be captured.
bool stream_capturing(void *stream)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(reinterpret_cast<hipStream_t>(stream), &st) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return st != hipStreamCaptureStatusNone;
}

int launch(const void *kernel, dim3 grid, dim3 block, void *params, void *stream)
{
    void *args[] = {params};
    hipError_t err = hipLaunchKernel(kernel, grid, block, args, 0,
                                     reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

// Checks shared by both appends (the grid size is checked too).
int check_append(const void *k, const void *v, const int64_t *slot_mapping, void *key_cache,
                 void *value_cache, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                 int32_t block_size, int64_t num_blocks)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0)
        return PKV_ERR_SHAPE;
    if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PKV_ERR_UNSUPPORTED;
    if (num_tokens == 0)
        return PKV_OK;
    if (!k || !v || !slot_mapping || !key_cache || !value_cache)
        return PKV_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(key_cache) || !aligned16(value_cache) ||
        (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
        return PKV_ERR_ALIGN;
    if ((int64_t)num_tokens * num_kv_heads * (head_dim / 8) + 256 > INT32_MAX)
        return PKV_ERR_SHAPE;                      // bounds the append grid, T * K / 4
    return PKV_OK;
}

// One wave per (token, KV head), four per 256-thread workgroup.
dim3 append_grid(int32_t num_tokens, int32_t num_kv_heads)
{
    return dim3((unsigned)ceil_div((int64_t)num_tokens * num_kv_heads, 4));
}

// An FP8 pool scale: finite, positive, with a finite fp32 inverse.
bool valid_pool_scale(float s)
{
    return isfinite(s) && s > 0.0f && isfinite(1.0f / s);
}

// Both decode entry points: bf16 pools (k_scale = v_scale = 1) or FP8 pools.
// The log-sum-exp merge over fixed partitions: one wave per (query row, KV
// head) for rows of at most kMergePartsMax partitions, else one workgroup
// per (query row, head).  rows = num_seqs * num_queries.
int launch_merge(pkv::MergeParams &mp, int head_dim, int32_t num_kv_heads, int64_t rows,
                 void *stream)
{
    if (mp.num_parts <= pkv::kMergePartsMax) {
        const int kmin = 256 / head_dim;
        const int g = mp.group;
        const int gp = g <= kmin ? kmin : g <= 4 ? 4 : g <= 8 ? 8 : 16;
        const void *mk;
        if (head_dim == 128)
            mk = gp == 2   ? (const void *)pkv::merge_parts_kernel<128, 2>
                 : gp == 4 ? (const void *)pkv::merge_parts_kernel<128, 4>
                 : gp == 8 ? (const void *)pkv::merge_parts_kernel<128, 8>
                           : (const void *)pkv::merge_parts_kernel<128, 16>;
        else
            mk = gp == 4   ? (const void *)pkv::merge_parts_kernel<64, 4>
                 : gp == 8 ? (const void *)pkv::merge_parts_kernel<64, 8>
                           : (const void *)pkv::merge_parts_kernel<64, 16>;
        return launch(mk, dim3((unsigned)num_kv_heads, (unsigned)rows), dim3(pkv::kWave), &mp,
                      stream);
    }
    const void *mk = head_dim == 128 ? (const void *)pkv::merge_kernel<128>
                                     : (const void *)pkv::merge_kernel<64>;
    return launch(mk, dim3((unsigned)mp.num_heads, (unsigned)rows), dim3(pkv::kMergeThreads), &mp,
                  stream);
}

// Fixed partitions (several) on persistent waves: schedule (large batches),
// then the balanced kernel in partition mode writing every partition's
// partial to the workspace's split-K slots; the caller launches the merge.
template <class Fmt>
int persistent_launch(pkv::DecodeParams &p, int head_dim, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t max_context_len, void *workspace,
                      size_t workspace_bytes, void *stream)
{
    const int32_t part = p.part;
    const FixedLayout FL = fixed_layout(num_seqs, num_heads, head_dim, max_context_len, part);
    if (!workspace || workspace_bytes < FL.total)
        return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return PKV_ERR_ALIGN;
    if ((int64_t)num_seqs * num_kv_heads * ceil_div(max_context_len, pkv::kChunk) >= INT32_MAX)
        return PKV_ERR_SHAPE;
    char *ws = static_cast<char *>(workspace);
    p.part_o = reinterpret_cast<float *>(ws + FL.part_o);
    p.part_ml = reinterpret_cast<float *>(ws + FL.part_ml);
    p.num_parts = (int32_t)ceil_div(max_context_len, part);
    int log2_waves = 0;
    int rc = device_waves(&log2_waves);
    if (rc != PKV_OK)
        return rc;
    pkv::BalancedParams bp;
    bp.d = p;
    bp.total_chunks = reinterpret_cast<int32_t *>(ws + FL.total_chunks);
    bp.chunk_start = reinterpret_cast<int32_t *>(ws + FL.chunk_start);
    bp.wave_start = reinterpret_cast<int4 *>(ws + FL.wave_start);
    bp.piece_o = nullptr;
    bp.piece_ml = nullptr;
    bp.num_waves = 1 << log2_waves;
    bp.log2_waves = log2_waves;
    bp.num_seqs = num_seqs;
    bp.inline_schedule = num_seqs <= pkv::kInlineScheduleSeqs;
    bp.part_chunks = part / pkv::kChunk;
    if (!bp.inline_schedule) {
        rc = launch((const void *)pkv::schedule_kernel<false>, dim3(1),
                    dim3(pkv::kScheduleThreads), &bp, stream);
        if (rc != PKV_OK)
            return rc;
    }
    const bool bs32 = p.block_size == 32;
    const void *dk =
        head_dim == 128
            ? (bs32 ? (const void *)pkv::decode_balanced_kernel<Fmt, 128, true, false, 0, 32>
                    : (const void *)pkv::decode_balanced_kernel<Fmt, 128, true, false, 0, 16>)
            : (bs32 ? (const void *)pkv::decode_balanced_kernel<Fmt, 64, true, false, 0, 32>
                    : (const void *)pkv::decode_balanced_kernel<Fmt, 64, true, false, 0, 16>);
    return launch(dk, dim3((unsigned)ceil_div(bp.num_waves, pkv::kGroupWaves)),
                  dim3(pkv::kWave * pkv::kGroupWaves), &bp, stream);   // the full chip
}

// Token-balanced kernel of the shared-prefix path for a head dim, block size
// and the group waves' tiles (0: no group waves in the grid; else 1 to 4).
template <class Fmt, int H, int BS>
const void *balanced_prefix_kernel_bs(int tiles)
{
    switch (tiles) {
    case 0: return (const void *)pkv::decode_balanced_kernel<Fmt, H, false, true, 0, BS>;
    case 1: return (const void *)pkv::decode_balanced_kernel<Fmt, H, false, true, 1, BS>;
    case 2: return (const void *)pkv::decode_balanced_kernel<Fmt, H, false, true, 2, BS>;
    case 3: return (const void *)pkv::decode_balanced_kernel<Fmt, H, false, true, 3, BS>;
    default: return (const void *)pkv::decode_balanced_kernel<Fmt, H, false, true, 4, BS>;
    }
}
template <class Fmt, int H>
const void *balanced_prefix_kernel(int tiles, int block_size)
{
    return block_size == 32 ? balanced_prefix_kernel_bs<Fmt, H, 32>(tiles)
                            : balanced_prefix_kernel_bs<Fmt, H, 16>(tiles);
}

// Token-balanced decode: schedule (large batches), persistent decode, merge
// of the split segments.  kPrefix: segments start after the positions each
// sequence's prefix group reads (its prefix_parts partials per row are in
// p.part_o / p.part_ml), and the merge joins those partials; group_waves
// waves of group_tiles tiles that compute them follow the persistent ones
// in the grid.
template <class Fmt, bool kPrefix>
int balanced_launch(pkv::DecodeParams &p, int head_dim, int32_t num_seqs, int32_t num_kv_heads,
                    const BalancedLayout &L, char *ws, int64_t prefix_parts, void *stream,
                    int group_tiles = 0, int64_t group_waves = 0)
{
    int log2_waves = 0;
    int rc = device_waves(&log2_waves);
    if (rc != PKV_OK)
        return rc;
    // Small problems: fewer waves when every wave would get fewer than
    // kMinChunksPerWave chunks (on the bound of T from the host-known
    // context bound) and the segments would average more pieces than one
    // merge batch reads (a batch of one 1,024-token sequence of 40 heads
    // otherwise gives each of 1,024 waves about one chunk and every segment
    // some 26 pieces to merge).
    int64_t seg_chunks_bound = ceil_div(p.max_ctx, pkv::kChunk);
    if (p.window > 0 && ceil_div(p.window, pkv::kChunk) + 1 < seg_chunks_bound)
        seg_chunks_bound = ceil_div(p.window, pkv::kChunk) + 1;
    const int64_t segments = (int64_t)num_seqs * num_kv_heads;
    const int64_t t_bound = segments * seg_chunks_bound;
    while (log2_waves > 0 && ((int64_t)1 << log2_waves) * kMinChunksPerWave > t_bound &&
           ((int64_t)1 << log2_waves) > kPiecesPerMergeBatch * segments)
        --log2_waves;
    const int waves = 1 << log2_waves;
    pkv::BalancedParams bp;
    bp.d = p;
    bp.total_chunks = reinterpret_cast<int32_t *>(ws + L.total_chunks);
    bp.chunk_start = reinterpret_cast<int32_t *>(ws + L.chunk_start);
    bp.wave_start = reinterpret_cast<int4 *>(ws + L.wave_start);
    bp.piece_ml = reinterpret_cast<float *>(ws + L.piece_ml);
    bp.piece_o = reinterpret_cast<float *>(ws + L.piece_o);
    bp.num_waves = waves;
    bp.log2_waves = log2_waves;
    bp.num_seqs = num_seqs;
    bp.inline_schedule = num_seqs <= pkv::kInlineScheduleSeqs;
    bp.part_chunks = 0;
    bp.prefix_parts = (int32_t)prefix_parts;
    if (!bp.inline_schedule) {
        rc = launch((const void *)pkv::schedule_kernel<kPrefix>, dim3(1),
                    dim3(pkv::kScheduleThreads), &bp, stream);
        if (rc != PKV_OK)
            return rc;
    }
    const void *dk;
    if constexpr (kPrefix)
        dk = head_dim == 128 ? balanced_prefix_kernel<Fmt, 128>(group_tiles, p.block_size)
                             : balanced_prefix_kernel<Fmt, 64>(group_tiles, p.block_size);
    else
        dk = head_dim == 128
                 ? (p.block_size == 32
                        ? (const void *)pkv::decode_balanced_kernel<Fmt, 128, false, false, 0, 32>
                        : (const void *)pkv::decode_balanced_kernel<Fmt, 128, false, false, 0, 16>)
                 : (p.block_size == 32
                        ? (const void *)pkv::decode_balanced_kernel<Fmt, 64, false, false, 0, 32>
                        : (const void *)pkv::decode_balanced_kernel<Fmt, 64, false, false, 0, 16>);
    // Four-wave workgroups for a full chip of waves; a trimmed grid (small
    // problems) takes one or two waves per workgroup, so it spreads over the
    // CUs instead of filling a quarter or half of them.
    int device_lg = 0;
    rc = device_waves(&device_lg);
    if (rc != PKV_OK)
        return rc;
    const int per_group = log2_waves >= device_lg ? pkv::kGroupWaves
                          : log2_waves == device_lg - 1 ? 2 : 1;
    rc = launch(dk, dim3((unsigned)ceil_div(waves + group_waves, per_group)),
                dim3(pkv::kWave * per_group), &bp, stream);
    if (rc != PKV_OK)
        return rc;
    const void *mk = merge_pieces_for<kPrefix>(head_dim, p.group);
    return launch(mk, dim3((unsigned)num_kv_heads, (unsigned)num_seqs), dim3(pkv::kWave), &bp,
                  stream);
}

// Host-side checks of the single-query decode calls, in the order the
// statuses are documented (no device is touched).
int check_decode(float *out, const void *q, const void *key_cache, const void *value_cache,
                 const int32_t *block_tables, const int32_t *context_lens, float scale,
                 float k_scale, int32_t window, int32_t num_kv_heads, int32_t block_size,
                 int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                 int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                 int32_t partition_size)
{
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
        max_context_len < 0 || num_blocks < 0 || window < 0)
        return PKV_ERR_SHAPE;
    if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PKV_ERR_UNSUPPORTED;
    if (num_heads % num_kv_heads != 0)
        return PKV_ERR_SHAPE;
    if (num_heads / num_kv_heads > PKV_MAX_GROUP)
        return PKV_ERR_UNSUPPORTED;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return PKV_ERR_SHAPE;
    if ((int64_t)max_context_len + partition_size > INT32_MAX)   // partition ends fit in int
        return PKV_ERR_SHAPE;
    if (num_seqs > 65535 || num_kv_heads > 65535)
        return PKV_ERR_SHAPE;
    if (partition_size != 0 &&
        (partition_size < PKV_PARTITION_GRAIN || partition_size > PKV_MAX_PARTITION ||
         partition_size % PKV_PARTITION_GRAIN != 0))
        return PKV_ERR_SHAPE;
    if (!isfinite(scale) || !isfinite(scale * k_scale))
        return PKV_ERR_SHAPE;
    if (num_seqs == 0)
        return PKV_OK;
    if (!out || !q || !block_tables || !context_lens)
        return PKV_ERR_NULL;
    if (max_context_len > 0 && (!key_cache || !value_cache))
        return PKV_ERR_NULL;
    if (max_context_len > 0 && num_blocks == 0)
        return PKV_ERR_SHAPE;
    if (!aligned16(out) || !aligned16(q) || (key_cache && !aligned16(key_cache)) ||
        (value_cache && !aligned16(value_cache)) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
        (reinterpret_cast<uintptr_t>(context_lens) & 3u))
        return PKV_ERR_ALIGN;
    return PKV_OK;
}

// The one-launch small-batch kernel for a head dim and block size.
template <class Fmt>
const void *split_kernel(int head_dim, int block_size)
{
    const bool bs32 = block_size == 32;
    return head_dim == 128 ? (bs32 ? (const void *)pkv::decode_split_kernel<Fmt, 128, 32>
                                   : (const void *)pkv::decode_split_kernel<Fmt, 128, 16>)
                           : (bs32 ? (const void *)pkv::decode_split_kernel<Fmt, 64, 32>
                                   : (const void *)pkv::decode_split_kernel<Fmt, 64, 16>);
}

template <class Fmt>
int decode_impl(float *out, const void *q, const void *key_cache, const void *value_cache,
                const int32_t *block_tables, const int32_t *context_lens, float scale,
                float k_scale, float v_scale, int32_t window, int32_t num_kv_heads,
                int32_t block_size,
                int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                int32_t partition_size, void *workspace, size_t workspace_bytes, void *stream)
{
    const int rc0 = check_decode(out, q, key_cache, value_cache, block_tables, context_lens,
                                 scale, k_scale, window, num_kv_heads, block_size, num_seqs,
                                 num_heads, head_dim, max_blocks_per_seq, max_context_len,
                                 num_blocks, partition_size);
    if (rc0 != PKV_OK || num_seqs == 0)
        return rc0;

    pkv::DecodeParams p;
    p.out = out;
    p.part_o = nullptr;
    p.part_ml = nullptr;
    p.q = static_cast<const uint16_t *>(q);
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    set_softmax_scale(p, scale, k_scale);
    p.out_scale = v_scale;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.block_size = block_size;
    p.group = num_heads / num_kv_heads;
    p.max_blocks = max_blocks_per_seq;
    p.max_ctx = max_context_len;
    p.part = partition_size;
    p.num_parts = 1;
    p.num_queries = 1;
    p.col_groups = 1;
    p.num_seqs = num_seqs;
    p.num_blocks = num_blocks;
    p.seq_group = nullptr;
    p.group_members = nullptr;
    p.prefix_tokens = nullptr;
    p.num_groups = 0;
    p.max_members = 0;
    p.max_prefix = 0;
    p.shared_tokens = nullptr;
    p.window = window;

    if (partition_size == 0) {
        // Token-balanced: schedule, persistent decode, merge of split segments.
        if ((int64_t)num_seqs * num_kv_heads * ceil_div(max_context_len, pkv::kChunk) >= INT32_MAX)
            return PKV_ERR_SHAPE;
        const BalancedLayout L = balanced_layout(num_seqs, num_heads, num_kv_heads, head_dim);
        if (!workspace || workspace_bytes < L.total)
            return PKV_ERR_WORKSPACE;
        if (!aligned16(workspace))
            return PKV_ERR_ALIGN;
        // Small batches: when each (sequence, KV head) pair's workgroup fits
        // one round of waves and reads at most kSplitMaxBytes, one launch
        // whose workgroups merge in LDS.  A workgroup runs on one compute
        // unit, whose share of the bandwidth bounds it: past that size the
        // persistent kernel, spread over every unit, is faster even with its
        // merge launch.
        int log2_waves = 0;
        const int rc = device_waves(&log2_waves);
        if (rc != PKV_OK)
            return rc;
        const int64_t chunks = ceil_div(max_context_len, pkv::kChunk);
        const int64_t chunk_bytes =
            (int64_t)pkv::kChunk * head_dim * (int64_t)sizeof(typename Fmt::Elem) * 2;
        if ((int64_t)num_seqs * num_kv_heads * pkv::kSplitWaves <= ((int64_t)1 << log2_waves) &&
            chunks <= pkv::kSplitMaxChunks && chunks * chunk_bytes <= pkv::kSplitMaxBytes)
            return launch(split_kernel<Fmt>(head_dim, block_size),
                          dim3((unsigned)num_kv_heads, (unsigned)num_seqs),
                          dim3(pkv::kWave * pkv::kSplitWaves), &p, stream);
        return balanced_launch<Fmt, false>(p, head_dim, num_seqs, num_kv_heads, L,
                                           static_cast<char *>(workspace), 0, stream);
    }

    // Fixed partitions of partition_size tokens.  One partition: one wave per
    // (KV head, sequence) writes the output.  Several: persistent waves on
    // the token-balanced schedule, each taking a run of whole partitions and
    // writing their partials, then the merge over partitions.
    const int32_t part = partition_size;
    const int64_t parts = max_context_len > 0 ? ceil_div(max_context_len, part) : 1;
    const bool split = parts > 1;
    p.num_parts = (int32_t)parts;
    if (!split) {
        const dim3 grid(1u, (unsigned)num_kv_heads, (unsigned)num_seqs);
        const bool bs32 = block_size == 32;
        const void *kern =
            head_dim == 128 ? (bs32 ? (const void *)pkv::decode_kernel<Fmt, 128, 32>
                                    : (const void *)pkv::decode_kernel<Fmt, 128, 16>)
                            : (bs32 ? (const void *)pkv::decode_kernel<Fmt, 64, 32>
                                    : (const void *)pkv::decode_kernel<Fmt, 64, 16>);
        return launch(kern, grid, dim3(pkv::kWave), &p, stream);
    }
    int rc = persistent_launch<Fmt>(p, head_dim, num_seqs, num_heads, num_kv_heads,
                                           max_context_len, workspace, workspace_bytes, stream);
    if (rc != PKV_OK)
        return rc;

    pkv::MergeParams mp;
    mp.out = out;
    mp.part_o = p.part_o;
    mp.part_ml = p.part_ml;
    mp.context_lens = context_lens;
    mp.num_queries = 1;
    mp.window = p.window;
    mp.num_heads = num_heads;
    mp.max_ctx = max_context_len;
    mp.part = part;
    mp.num_parts = (int32_t)parts;
    mp.group = num_heads / num_kv_heads;
    return launch_merge(mp, head_dim, num_kv_heads, num_seqs, stream);
}

// Multi-query decode: kernel for a head dim, block size, tiles per wave (1 to
// 4) and split.
template <class Fmt, int H, int BS>
const void *multi_kernel_bs(int tiles, bool split)
{
    switch (tiles) {
    case 1: return split ? (const void *)pkv::decode_multi_kernel<Fmt, H, 1, true, BS>
                         : (const void *)pkv::decode_multi_kernel<Fmt, H, 1, false, BS>;
    case 2: return split ? (const void *)pkv::decode_multi_kernel<Fmt, H, 2, true, BS>
                         : (const void *)pkv::decode_multi_kernel<Fmt, H, 2, false, BS>;
    case 3: return split ? (const void *)pkv::decode_multi_kernel<Fmt, H, 3, true, BS>
                         : (const void *)pkv::decode_multi_kernel<Fmt, H, 3, false, BS>;
    default: return split ? (const void *)pkv::decode_multi_kernel<Fmt, H, 4, true, BS>
                          : (const void *)pkv::decode_multi_kernel<Fmt, H, 4, false, BS>;
    }
}
template <class Fmt, int H>
const void *multi_kernel(int tiles, bool split, int block_size)
{
    return block_size == 32 ? multi_kernel_bs<Fmt, H, 32>(tiles, split)
                            : multi_kernel_bs<Fmt, H, 16>(tiles, split);
}

// Tiles per wave of the shared-prefix group waves: the fewest (most waves,
// shortest kernel) that still fit one wave per SIMD of the chip (wave_slots);
// the waves that split an item's columns re-read its blocks from their XCD's
// L2.
int prefix_tiles_per_wave(int64_t items, int tiles, int64_t wave_slots)
{
    for (int pw = 1; pw < pkv::kTilesPerWave && pw < tiles; ++pw)
        if (items * ceil_div(tiles, pw) <= wave_slots)
            return pw;
    return tiles < pkv::kTilesPerWave ? tiles : pkv::kTilesPerWave;
}



template <class Fmt>
int decode_mq_launch(pkv::DecodeParams &p, int head_dim, int32_t num_seqs, int32_t num_queries,
                     int32_t num_heads, int32_t num_kv_heads, int32_t max_context_len,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    const int32_t part = p.part;
    const int64_t parts = max_context_len > 0 ? ceil_div(max_context_len, part) : 1;
    const bool split = parts > 1;
    if (split) {
        const size_t need = mq_workspace_bytes(num_seqs, num_queries, num_heads, head_dim,
                                               max_context_len, part);
        if (!workspace || workspace_bytes < need)
            return PKV_ERR_WORKSPACE;
        if (!aligned16(workspace))
            return PKV_ERR_ALIGN;
        const int64_t rows = (int64_t)num_seqs * num_queries * num_heads * parts;
        const int64_t o_bytes = ((rows * head_dim * 4) + 255) / 256 * 256;
        p.part_o = static_cast<float *>(workspace);
        p.part_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + o_bytes);
    }
    p.num_parts = (int32_t)parts;
    const int tiles = (int)ceil_div((int64_t)num_queries * (num_heads / num_kv_heads), 16);
    p.col_groups = (int32_t)ceil_div(tiles, pkv::kTilesPerWave);
    p.num_seqs = num_seqs;
    const int per_wave = tiles < pkv::kTilesPerWave ? tiles : pkv::kTilesPerWave;
    const void *kern = head_dim == 128 ? multi_kernel<Fmt, 128>(per_wave, split, p.block_size)
                                       : multi_kernel<Fmt, 64>(per_wave, split, p.block_size);
    const int64_t items = parts * num_kv_heads * num_seqs;
    const int64_t waves = ceil_div(items, pkv::kXcds) * pkv::kXcds * p.col_groups;
    if (waves > INT32_MAX)
        return PKV_ERR_SHAPE;
    // Two partitions: the second partition wave of each pair merges (no
    // merge launch).  The pair tags need a new value per call, which a graph
    // replay would not bring, so a captured call takes the merge launch (same
    // arithmetic, same result).
    const bool pair = split && parts == 2 && per_wave < pkv::kMaxQueryTiles &&
                      !stream_capturing(stream);
    if (pair) {
        p.pair_tags = reinterpret_cast<uint64_t *>(
            static_cast<char *>(workspace) +
            mq_pair_tags_offset(num_seqs, num_queries, num_heads, head_dim, max_context_len,
                                part));
        p.epoch = next_pair_epoch();
    }
    int rc = launch(kern, dim3((unsigned)waves), dim3(pkv::kWave), &p, stream);
    if (rc != PKV_OK || !split || pair)
        return rc;
    pkv::MergeParams mp;
    mp.out = p.out;
    mp.part_o = p.part_o;
    mp.part_ml = p.part_ml;
    mp.context_lens = p.context_lens;
    mp.num_queries = num_queries;
    mp.window = 0;
    mp.num_heads = num_heads;
    mp.max_ctx = max_context_len;
    mp.part = part;
    mp.num_parts = (int32_t)parts;
    mp.group = num_heads / num_kv_heads;
    return launch_merge(mp, head_dim, num_kv_heads, (int64_t)num_seqs * num_queries, stream);
}

// Prefix-aware decode: one grid of the token-balanced waves (the rest of
// every context) followed by the group waves (every shared span once, its
// partitions' partials per member), then the merge that joins the two.  For
// more sequences than the waves scan themselves, a spans kernel first stores
// every S_b, which the schedule and the per-sequence waves read.
template <class Fmt>
int decode_prefix_launch(pkv::DecodeParams &p, int head_dim, int32_t num_seqs, int32_t num_heads,
                         int32_t num_kv_heads, int32_t max_context_len, int32_t max_prefix_tokens,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    const int64_t prefix_parts = prefix_parts_of(max_context_len, p.part, max_prefix_tokens);
    const PrefixLayout L = prefix_layout(num_seqs, num_heads, num_kv_heads, head_dim,
                                         prefix_parts);
    if (!workspace || workspace_bytes < L.total)
        return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return PKV_ERR_ALIGN;
    if ((int64_t)num_seqs * num_kv_heads * ceil_div(max_context_len, pkv::kChunk) >= INT32_MAX)
        return PKV_ERR_SHAPE;
    char *ws = static_cast<char *>(workspace);
    p.part_o = reinterpret_cast<float *>(ws + L.pre_o);
    p.part_ml = reinterpret_cast<float *>(ws + L.pre_ml);
    p.num_parts = 1;
    // No shared span outgrows the partials the workspace holds (a group whose
    // prefix_tokens exceeds the stated bound shares only this much).
    p.max_prefix = (int32_t)(prefix_parts * p.part);
    p.shared_tokens = nullptr;      // no group: nothing is shared

    // The group waves' partials (and, for small batches, the spans they
    // store) are complete when the merge, a later kernel on the same stream,
    // reads them.
    int group_tiles = 0;
    int64_t group_waves = 0;
    if (prefix_parts > 0 && p.num_groups > 0) {
        const int tiles = (int)ceil_div((int64_t)p.max_members * (num_heads / num_kv_heads), 16);
        const int64_t items = (int64_t)p.num_groups * num_kv_heads * prefix_parts;
        int log2_waves = 0;
        int rc = device_waves(&log2_waves);
        if (rc != PKV_OK)
            return rc;
        group_tiles = prefix_tiles_per_wave(items, tiles, (int64_t)1 << log2_waves);
        p.col_groups = (int32_t)ceil_div(tiles, group_tiles);
        group_waves = ceil_div(items, pkv::kXcds) * pkv::kXcds * p.col_groups;
        // Small batches: at least one group wave per 64 sequences stores the spans.
        const bool inline_spans = num_seqs <= pkv::kInlineScheduleSeqs;
        if (inline_spans && group_waves < ceil_div(num_seqs, pkv::kWave))
            group_waves = ceil_div(num_seqs, pkv::kWave);
        if (group_waves > INT32_MAX - ((int64_t)1 << log2_waves))
            return PKV_ERR_SHAPE;
        p.shared_tokens = reinterpret_cast<int32_t *>(ws + L.shared);
        if (!inline_spans) {
            rc = launch((const void *)pkv::prefix_spans_kernel,
                        dim3((unsigned)ceil_div(num_seqs, pkv::kWave)), dim3(pkv::kWave), &p,
                        stream);
            if (rc != PKV_OK)
                return rc;
        }
    }
    return balanced_launch<Fmt, true>(p, head_dim, num_seqs, num_kv_heads, L.bal, ws,
                                      prefix_parts, stream, group_tiles, group_waves);
}

// Scratch of the allocation-free entry point (paged_decode_attention_noalloc):
// a static device array, so every device the library runs on holds its own
// copy of PKV_NOALLOC_SCRATCH_BYTES until the process ends.  On the host,
// `scratch` names a host-side stand-in, not device memory: host code uses
// only the device address hipGetSymbolAddress returns for it (per device).
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_address[kMaxDevices];   // per device, set on the first call there

// Device address of the current device's scratch array (looked up once per
// device, with that device current).
int device_scratch(void **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return PKV_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_address[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return PKV_ERR_DEVICE;
        scratch_address[dev] = p;
    }
    *ptr = scratch_address[dev];
    return PKV_OK;
}

}  // namespace

extern "C" {

int pagedkv_version(void) { return (kVersionMajor << 16) | kVersionMinor; }

const char *pagedkv_status_string(int status)
{
    switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "sizes inconsistent or out of range";
    case PKV_ERR_UNSUPPORTED: return "head_dim, block_size or group size not supported";
    case PKV_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_DEVICE: return "no usable HIP device";
    case PKV_ERR_SCRATCH:
        return "problem needs more scratch than the allocation-free call holds "
               "(PKV_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

int paged_kv_append(const void *k, const void *v, const int64_t *slot_mapping, void *key_cache,
                    void *value_cache, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int64_t num_blocks, void *stream)
{
    int rc = check_append(k, v, slot_mapping, key_cache, value_cache, num_tokens, num_kv_heads,
                          head_dim, block_size, num_blocks);
    if (rc != PKV_OK || num_tokens == 0)
        return rc;
    pkv::AppendParams p;
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.slot_mapping = slot_mapping;
    p.key_cache = static_cast<uint16_t *>(key_cache);
    p.value_cache = static_cast<uint16_t *>(value_cache);
    p.num_tokens = num_tokens;
    p.num_kv_heads = num_kv_heads;
    p.num_slots = num_blocks * block_size;
    const bool bs32 = block_size == 32;
    const void *kern = head_dim == 128 ? (bs32 ? (const void *)pkv::append_kernel<128, 32>
                                               : (const void *)pkv::append_kernel<128, 16>)
                                       : (bs32 ? (const void *)pkv::append_kernel<64, 32>
                                               : (const void *)pkv::append_kernel<64, 16>);
    return launch(kern, append_grid(num_tokens, num_kv_heads), dim3(256), &p, stream);
}

int paged_kv_append_fp8(const void *k, const void *v, const int64_t *slot_mapping,
                        void *key_cache, void *value_cache, float k_scale, float v_scale,
                        int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int64_t num_blocks, void *stream)
{
    int rc = check_append(k, v, slot_mapping, key_cache, value_cache, num_tokens, num_kv_heads,
                          head_dim, block_size, num_blocks);
    if (rc != PKV_OK)
        return rc;
    if (!valid_pool_scale(k_scale) || !valid_pool_scale(v_scale))
        return PKV_ERR_SHAPE;
    if (num_tokens == 0)
        return PKV_OK;
    pkv::AppendFp8Params p;
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.slot_mapping = slot_mapping;
    p.key_cache = static_cast<uint8_t *>(key_cache);
    p.value_cache = static_cast<uint8_t *>(value_cache);
    p.k_inv = 1.0f / k_scale;
    p.v_inv = 1.0f / v_scale;
    p.num_tokens = num_tokens;
    p.num_kv_heads = num_kv_heads;
    p.num_slots = num_blocks * block_size;
    const bool bs32 = block_size == 32;
    const void *kern = head_dim == 128 ? (bs32 ? (const void *)pkv::append_fp8_kernel<128, 32>
                                               : (const void *)pkv::append_fp8_kernel<128, 16>)
                                       : (bs32 ? (const void *)pkv::append_fp8_kernel<64, 32>
                                               : (const void *)pkv::append_fp8_kernel<64, 16>);
    return launch(kern, append_grid(num_tokens, num_kv_heads), dim3(256), &p, stream);
}

size_t paged_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t max_context_len,
                                   int32_t partition_size)
{
    if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_context_len <= 0 || partition_size < 0 || num_heads % num_kv_heads != 0)
        return 0;
    if (partition_size == 0)
        return balanced_layout(num_seqs, num_heads, num_kv_heads, head_dim).total;
    return fixed_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size);
}

size_t paged_decode_prefix_workspace_size(int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_context_len, int32_t partition_size,
                                          int32_t max_prefix_tokens)
{
    if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_context_len < 0 || partition_size <= 0 || max_prefix_tokens < 0 ||
        num_heads % num_kv_heads != 0)
        return 0;
    return prefix_layout(num_seqs, num_heads, num_kv_heads, head_dim,
                         prefix_parts_of(max_context_len, partition_size, max_prefix_tokens))
        .total;
}

int paged_decode_attention(float *out, const void *q, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *context_lens, float scale, int32_t num_kv_heads,
                           int32_t block_size, int32_t num_seqs, int32_t num_heads,
                           int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                           int64_t num_blocks, int32_t partition_size, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    return decode_impl<pkv::KvBf16>(out, q, key_cache, value_cache, block_tables, context_lens,
                                    scale, 1.0f, 1.0f, 0, num_kv_heads, block_size, num_seqs,
                                    num_heads, head_dim, max_blocks_per_seq, max_context_len,
                                    num_blocks, partition_size, workspace, workspace_bytes,
                                    stream);
}

int paged_decode_attention_noalloc(float *out, const void *q, const void *key_cache,
                                   const void *value_cache, const int32_t *block_tables,
                                   const int32_t *context_lens, float scale,
                                   int32_t num_kv_heads, int32_t block_size, int32_t num_seqs,
                                   int32_t num_heads, int32_t head_dim,
                                   int32_t max_blocks_per_seq, int32_t max_context_len,
                                   int64_t num_blocks, int32_t partition_size, void *stream)
{
    int rc = check_decode(out, q, key_cache, value_cache, block_tables, context_lens, scale,
                          1.0f, 0, num_kv_heads, block_size, num_seqs, num_heads, head_dim,
                          max_blocks_per_seq, max_context_len, num_blocks, partition_size);
    if (rc != PKV_OK || num_seqs == 0)
        return rc;
    // The workspace paged_decode_attention would need for this shape.
    const size_t need =
        partition_size == 0
            ? balanced_layout(num_seqs, num_heads, num_kv_heads, head_dim).total
            : fixed_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                                    partition_size);
    if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES)
        return PKV_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        rc = device_scratch(&ws);
        if (rc != PKV_OK)
            return rc;
    }
    return decode_impl<pkv::KvBf16>(out, q, key_cache, value_cache, block_tables, context_lens,
                                    scale, 1.0f, 1.0f, 0, num_kv_heads, block_size, num_seqs,
                                    num_heads, head_dim, max_blocks_per_seq, max_context_len,
                                    num_blocks, partition_size, ws,
                                    need > 0 ? (size_t)PKV_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int paged_decode_attention_fp8(float *out, const void *q, const void *key_cache,
                               const void *value_cache, const int32_t *block_tables,
                               const int32_t *context_lens, float scale, float k_scale,
                               float v_scale, int32_t num_kv_heads, int32_t block_size,
                               int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int32_t max_context_len,
                               int64_t num_blocks, int32_t partition_size, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    if (!valid_pool_scale(k_scale) || !valid_pool_scale(v_scale))
        return PKV_ERR_SHAPE;
    return decode_impl<pkv::KvFp8>(out, q, key_cache, value_cache, block_tables, context_lens,
                                   scale, k_scale, v_scale, 0, num_kv_heads, block_size, num_seqs,
                                   num_heads, head_dim, max_blocks_per_seq, max_context_len,
                                   num_blocks, partition_size, workspace, workspace_bytes, stream);
}

size_t paged_decode_mq_workspace_size(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                      int32_t head_dim, int32_t max_context_len,
                                      int32_t partition_size)
{
    if (num_seqs <= 0 || num_queries <= 0 || num_heads <= 0 || head_dim <= 0 ||
        max_context_len <= 0 || partition_size <= 0)
        return 0;
    return mq_workspace_bytes(num_seqs, num_queries, num_heads, head_dim, max_context_len,
                              partition_size);
}

int paged_decode_attention_mq(float *out, const void *q, const void *key_cache,
                              const void *value_cache, const int32_t *block_tables,
                              const int32_t *context_lens, float scale, int32_t kv_dtype,
                              float k_scale, float v_scale, int32_t num_kv_heads,
                              int32_t block_size, int32_t num_seqs, int32_t num_queries,
                              int32_t num_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                              int32_t max_context_len, int64_t num_blocks,
                              int32_t partition_size, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    if (num_seqs < 0 || num_queries <= 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks < 0)
        return PKV_ERR_SHAPE;
    if (kv_dtype != PKV_KV_BF16 && kv_dtype != PKV_KV_FP8_E4M3)
        return PKV_ERR_UNSUPPORTED;
    if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PKV_ERR_UNSUPPORTED;
    if (num_heads % num_kv_heads != 0)
        return PKV_ERR_SHAPE;
    if ((int64_t)num_queries * (num_heads / num_kv_heads) > PKV_MAX_QUERY_ROWS)
        return PKV_ERR_UNSUPPORTED;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return PKV_ERR_SHAPE;
    if ((int64_t)max_context_len + partition_size > INT32_MAX)   // partition ends fit in int
        return PKV_ERR_SHAPE;
    if ((int64_t)num_seqs * num_queries > 65535 || num_kv_heads > 65535)
        return PKV_ERR_SHAPE;
    if (partition_size < PKV_PARTITION_GRAIN || partition_size > PKV_MAX_MQ_PARTITION ||
        partition_size % PKV_PARTITION_GRAIN != 0)
        return PKV_ERR_SHAPE;
    if (kv_dtype == PKV_KV_BF16) {
        k_scale = 1.0f;
        v_scale = 1.0f;
    } else if (!valid_pool_scale(k_scale) || !valid_pool_scale(v_scale)) {
        return PKV_ERR_SHAPE;
    }
    if (!isfinite(scale) || !isfinite(scale * k_scale))
        return PKV_ERR_SHAPE;
    if (num_seqs == 0)
        return PKV_OK;
    if (!out || !q || !block_tables || !context_lens)
        return PKV_ERR_NULL;
    if (max_context_len > 0 && (!key_cache || !value_cache))
        return PKV_ERR_NULL;
    if (max_context_len > 0 && num_blocks == 0)
        return PKV_ERR_SHAPE;
    if (!aligned16(out) || !aligned16(q) || (key_cache && !aligned16(key_cache)) ||
        (value_cache && !aligned16(value_cache)) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
        (reinterpret_cast<uintptr_t>(context_lens) & 3u))
        return PKV_ERR_ALIGN;

    pkv::DecodeParams p;
    p.out = out;
    p.part_o = nullptr;
    p.part_ml = nullptr;
    p.q = static_cast<const uint16_t *>(q);
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    set_softmax_scale(p, scale, k_scale);
    p.out_scale = v_scale;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.block_size = block_size;
    p.group = num_heads / num_kv_heads;
    p.max_blocks = max_blocks_per_seq;
    p.max_ctx = max_context_len;
    p.part = partition_size;
    p.num_parts = 1;
    p.num_queries = num_queries;
    p.col_groups = 1;
    p.num_seqs = num_seqs;
    p.num_blocks = num_blocks;
    p.seq_group = nullptr;
    p.group_members = nullptr;
    p.prefix_tokens = nullptr;
    p.num_groups = 0;
    p.max_members = 0;
    p.max_prefix = 0;
    p.shared_tokens = nullptr;
    p.window = 0;
    if (kv_dtype == PKV_KV_FP8_E4M3)
        return decode_mq_launch<pkv::KvFp8>(p, head_dim, num_seqs, num_queries, num_heads,
                                            num_kv_heads, max_context_len, workspace,
                                            workspace_bytes, stream);
    return decode_mq_launch<pkv::KvBf16>(p, head_dim, num_seqs, num_queries, num_heads,
                                         num_kv_heads, max_context_len, workspace,
                                         workspace_bytes, stream);
}

int paged_decode_attention_window(float *out, const void *q, const void *key_cache,
                                  const void *value_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, float scale, int32_t kv_dtype,
                                  float k_scale, float v_scale, int32_t window,
                                  int32_t num_kv_heads, int32_t block_size, int32_t num_seqs,
                                  int32_t num_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  int64_t num_blocks, int32_t partition_size, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    if (window < 1)
        return PKV_ERR_SHAPE;
    if (kv_dtype == PKV_KV_BF16)
        return decode_impl<pkv::KvBf16>(out, q, key_cache, value_cache, block_tables,
                                        context_lens, scale, 1.0f, 1.0f, window, num_kv_heads,
                                        block_size, num_seqs, num_heads, head_dim,
                                        max_blocks_per_seq, max_context_len, num_blocks,
                                        partition_size, workspace, workspace_bytes, stream);
    if (kv_dtype != PKV_KV_FP8_E4M3)
        return PKV_ERR_UNSUPPORTED;
    if (!valid_pool_scale(k_scale) || !valid_pool_scale(v_scale))
        return PKV_ERR_SHAPE;
    return decode_impl<pkv::KvFp8>(out, q, key_cache, value_cache, block_tables, context_lens,
                                   scale, k_scale, v_scale, window, num_kv_heads, block_size,
                                   num_seqs, num_heads, head_dim, max_blocks_per_seq,
                                   max_context_len, num_blocks, partition_size, workspace,
                                   workspace_bytes, stream);
}

int paged_decode_attention_prefix(float *out, const void *q, const void *key_cache,
                                  const void *value_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, float scale, int32_t kv_dtype,
                                  float k_scale, float v_scale, int32_t num_kv_heads,
                                  int32_t block_size, int32_t num_seqs, int32_t num_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int32_t max_context_len, int64_t num_blocks,
                                  int32_t partition_size, const int32_t *seq_group,
                                  const int32_t *group_members, const int32_t *prefix_tokens,
                                  int32_t num_groups, int32_t max_members,
                                  int32_t max_prefix_tokens, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
        max_context_len < 0 || num_blocks < 0 || num_groups < 0 || max_members < 0 ||
        max_prefix_tokens < 0)
        return PKV_ERR_SHAPE;
    if (kv_dtype != PKV_KV_BF16 && kv_dtype != PKV_KV_FP8_E4M3)
        return PKV_ERR_UNSUPPORTED;
    if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PKV_ERR_UNSUPPORTED;
    if (num_heads % num_kv_heads != 0)
        return PKV_ERR_SHAPE;
    if (num_heads / num_kv_heads > PKV_MAX_GROUP)
        return PKV_ERR_UNSUPPORTED;
    if ((int64_t)max_members * (num_heads / num_kv_heads) > PKV_MAX_PREFIX_ROWS)
        return PKV_ERR_UNSUPPORTED;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return PKV_ERR_SHAPE;
    if ((int64_t)max_context_len + partition_size > INT32_MAX)   // partition ends fit in int
        return PKV_ERR_SHAPE;
    if (num_seqs > 65535 || num_kv_heads > 65535)
        return PKV_ERR_SHAPE;
    if (partition_size < PKV_PARTITION_GRAIN || partition_size > PKV_MAX_PARTITION ||
        partition_size % PKV_PARTITION_GRAIN != 0)
        return PKV_ERR_SHAPE;
    if (kv_dtype == PKV_KV_BF16) {
        k_scale = 1.0f;
        v_scale = 1.0f;
    } else if (!valid_pool_scale(k_scale) || !valid_pool_scale(v_scale)) {
        return PKV_ERR_SHAPE;
    }
    if (!isfinite(scale) || !isfinite(scale * k_scale))
        return PKV_ERR_SHAPE;
    if (num_seqs == 0)
        return PKV_OK;
    if (!out || !q || !block_tables || !context_lens || !seq_group)
        return PKV_ERR_NULL;
    if (num_groups > 0 && (!group_members || !prefix_tokens || max_members == 0))
        return PKV_ERR_NULL;
    if (max_context_len > 0 && (!key_cache || !value_cache))
        return PKV_ERR_NULL;
    if (max_context_len > 0 && num_blocks == 0)
        return PKV_ERR_SHAPE;
    if (!aligned16(out) || !aligned16(q) || (key_cache && !aligned16(key_cache)) ||
        (value_cache && !aligned16(value_cache)) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
        (reinterpret_cast<uintptr_t>(context_lens) & 3u) ||
        (reinterpret_cast<uintptr_t>(seq_group) & 3u) ||
        (reinterpret_cast<uintptr_t>(group_members) & 3u) ||
        (reinterpret_cast<uintptr_t>(prefix_tokens) & 3u))
        return PKV_ERR_ALIGN;

    pkv::DecodeParams p;
    p.out = out;
    p.part_o = nullptr;
    p.part_ml = nullptr;
    p.q = static_cast<const uint16_t *>(q);
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    set_softmax_scale(p, scale, k_scale);
    p.out_scale = v_scale;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.block_size = block_size;
    p.group = num_heads / num_kv_heads;
    p.max_blocks = max_blocks_per_seq;
    p.max_ctx = max_context_len;
    p.part = partition_size;
    p.num_parts = 1;
    p.num_queries = 1;
    p.col_groups = 1;
    p.num_seqs = num_seqs;
    p.num_blocks = num_blocks;
    p.seq_group = seq_group;
    p.group_members = group_members;
    p.prefix_tokens = prefix_tokens;
    p.num_groups = num_groups;
    p.max_members = max_members;
    p.max_prefix = 0;
    p.shared_tokens = nullptr;
    p.window = 0;
    if (kv_dtype == PKV_KV_FP8_E4M3)
        return decode_prefix_launch<pkv::KvFp8>(p, head_dim, num_seqs, num_heads, num_kv_heads,
                                                max_context_len, max_prefix_tokens, workspace,
                                                workspace_bytes, stream);
    return decode_prefix_launch<pkv::KvBf16>(p, head_dim, num_seqs, num_heads, num_kv_heads,
                                             max_context_len, max_prefix_tokens, workspace,
                                             workspace_bytes, stream);
}

int paged_kv_copy_blocks(void *key_cache, void *value_cache, const int32_t *src_blocks,
                         const int32_t *dst_blocks, int32_t num_pairs, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int64_t num_blocks,
                         int32_t kv_dtype, void *stream)
{
    if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks < 0)
        return PKV_ERR_SHAPE;
    if (kv_dtype != PKV_KV_BF16 && kv_dtype != PKV_KV_FP8_E4M3)
        return PKV_ERR_UNSUPPORTED;
    if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PKV_ERR_UNSUPPORTED;
    if (num_pairs == 0)
        return PKV_OK;
    if (num_pairs > 65535)
        return PKV_ERR_SHAPE;
    if (!key_cache || !value_cache || !src_blocks || !dst_blocks)
        return PKV_ERR_NULL;
    if (!aligned16(key_cache) || !aligned16(value_cache) ||
        (reinterpret_cast<uintptr_t>(src_blocks) & 3u) ||
        (reinterpret_cast<uintptr_t>(dst_blocks) & 3u))
        return PKV_ERR_ALIGN;
    pkv::CopyBlocksParams p;
    p.key_cache = static_cast<uint8_t *>(key_cache);
    p.value_cache = static_cast<uint8_t *>(value_cache);
    p.src = src_blocks;
    p.dst = dst_blocks;
    p.block_bytes = (int64_t)num_kv_heads * block_size * head_dim *
                    (kv_dtype == PKV_KV_BF16 ? 2 : 1);
    p.num_blocks = num_blocks;
    const int64_t slices = ceil_div(p.block_bytes, (int64_t)pkv::kCopyThreads * 16);
    const unsigned gx = (unsigned)(slices < 64 ? slices : 64);
    return launch((const void *)pkv::copy_blocks_kernel, dim3(gx, (unsigned)num_pairs),
                  dim3(pkv::kCopyThreads), &p, stream);
}

size_t pagedkv_stream_read_sink_bytes(size_t bytes)
{
    (void)bytes;
    return (size_t)pkv::kMaxBalancedWaves * 16;    // one slot per wave, any device
}

int pagedkv_stream_read(const void *src, size_t bytes, void *sink, void *stream)
{
    if (bytes == 0)
        return PKV_OK;
    if (!src || !sink)
        return PKV_ERR_NULL;
    if (bytes % 16 != 0)
        return PKV_ERR_SHAPE;
    if (!aligned16(src) || !aligned16(sink))
        return PKV_ERR_ALIGN;
    int log2_waves = 0;
    const int rc = device_waves(&log2_waves);     // one wave per SIMD, as the decode runs
    if (rc != PKV_OK)
        return rc;
    const int64_t n16 = (int64_t)(bytes / 16);
    struct {
        const pkv::u32x4 *src;
        int64_t n16;
        pkv::u32x4 *sink;
    } a = {static_cast<const pkv::u32x4 *>(src), n16, static_cast<pkv::u32x4 *>(sink)};
    void *args[] = {&a.src, &a.n16, &a.sink};
    hipError_t err = hipLaunchKernel((const void *)pkv::stream_read_kernel,
                                     dim3(1u << log2_waves), dim3(pkv::kWave), args, 0,
                                     reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int pagedkv_stream_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (bytes == 0)
        return PKV_OK;
    if (!src || !dst)
        return PKV_ERR_NULL;
    if (bytes % 16 != 0)
        return PKV_ERR_SHAPE;
    if (!aligned16(src) || !aligned16(dst))
        return PKV_ERR_ALIGN;
    struct {
        const pkv::u32x4 *src;
        pkv::u32x4 *dst;
        int64_t n16;
    } a = {static_cast<const pkv::u32x4 *>(src), static_cast<pkv::u32x4 *>(dst),
           (int64_t)(bytes / 16)};
    void *args[] = {&a.src, &a.dst, &a.n16};
    hipError_t err = hipLaunchKernel((const void *)pkv::stream_copy_kernel,
                                     dim3(pkv::kStreamBlocksMax), dim3(pkv::kStreamThreads), args,
                                     0, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"
