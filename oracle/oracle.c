/*
 * Plain CPU reference ("oracle") for paged-KV decode attention and the
 * slot-mapped K/V append.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the CPU-baseline leg of the benchmark call it; the product path
 * never does.  It shares no code, header or constant with the HIP library.
 *
 * Everything is written as the plain definition, one output at a time, in
 * double precision.  bf16 values are passed as their raw 16-bit patterns.
 *
 * What it follows:
 *   - "Optimización de la inferencia" / "推理优化 (Inference Optimization)"
 *     lesson, Build-It step 2 (attention with the KV cache): scores are
 *     q.k divided by sqrt(head_dim), the row maximum is subtracted, the
 *     exponentials are normalised by their sum, and the weights multiply V.
 *     With a single query token no causal mask applies.
 *   - same lesson, step 1 (KV cache from scratch): the new step's K/V are
 *     written at the next position and the attention reads positions
 *     [0, end).
 *   - same lesson, "PagedAttention" concept section, and "CS336 Lecture 10:
 *     Inference", part 6 (PagedAttention): the cache is split in fixed-size
 *     blocks anywhere in memory, and a per-sequence table maps logical
 *     block j of the sequence to a physical block.
 *   - "CS336 Lecture 10: Inference", part 3 (GQA): each of the K key/value
 *     heads serves N/K query heads.  Query head n uses KV head n / (N/K)
 *     (consecutive grouping).
 *
 * Memory layouts (the pages leave them open; these are the library's):
 *   key_cache   [num_blocks][K][block_size][H]   token rows of H values
 *   value_cache [num_blocks][K][H][block_size]   one column per token
 *   q           [B][N][H],  k/v new tokens [T][K][H]
 *   block_tables[B][max_blocks_per_seq] int32, context_lens[B] int32
 *   slot = physical_block * block_size + offset_in_block (int64)
 *
 * FP8 caches ("Week 11. Inference", step 2, names quantising the cache to 8
 * bits as a way to halve it): the same layouts holding one-byte OCP FP8 E4M3
 * codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; S.1111.111 is NaN) with one scale per pool: a stored code c
 * stands for decode(c) * scale.  Appending value x stores the code nearest to
 * x * inv_scale (inv_scale = 1/scale rounded to fp32; product in fp32), after
 * clamping that product to +-448, the largest finite code; ties go to the
 * even code; NaN stores 0xFF.
 *
 * Return codes: 0 on success, -1 on an argument that makes the definition
 * meaningless (a block id or slot outside the pool, N not divisible by K,
 * a context longer than the block table).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int thread_id(void)
{
#ifdef _OPENMP
    return omp_get_thread_num();
#else
    return 0;
#endif
}

static double bf16_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Value of an OCP FP8 E4M3 code, exactly. */
double oracle_e4m3_value(uint8_t code)
{
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);             /* subnormal: m/8 * 2^-6 */
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Code nearest to y (ties to the even code), y finite with |y| <= 448:
 * the 127 non-negative finite codes are in increasing order of value. */
static uint8_t e4m3_nearest(float y)
{
    double a = fabs((double)y);
    int lo = 0;
    while (lo < 126 && oracle_e4m3_value((uint8_t)(lo + 1)) <= a)
        lo++;
    int code = lo;
    if (lo < 126) {
        double d_lo = a - oracle_e4m3_value((uint8_t)lo);
        double d_hi = oracle_e4m3_value((uint8_t)(lo + 1)) - a;
        if (d_hi < d_lo || (d_hi == d_lo && ((lo + 1) & 1) == 0))
            code = lo + 1;
    }
    return (uint8_t)(code | (signbit(y) ? 0x80 : 0));
}

/* Quantisation of one bf16 value for an FP8 pool with inverse scale inv. */
uint8_t oracle_e4m3_quantize(uint16_t bits, float inv)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    float y = x * inv;                          /* one fp32 rounding */
    if (isnan(y))
        return 0xFF;
    if (y > 448.0f)
        y = 448.0f;
    if (y < -448.0f)
        y = -448.0f;
    return e4m3_nearest(y);
}

/* A cache element as a double: bf16 bits, or an FP8 code times its scale. */
enum { KV_BF16 = 0, KV_FP8 = 1 };

static double cache_value(const void *pool, size_t index, int dtype, double scale)
{
    if (dtype == KV_BF16)
        return bf16_to_double(((const uint16_t *)pool)[index]);
    return oracle_e4m3_value(((const uint8_t *)pool)[index]) * scale;
}

/* Address of key element (block p, kv head g, offset o, dim h). */
static size_t key_index(int64_t p, int g, int o, int h, int K, int bs, int H)
{
    return (((size_t)p * K + g) * bs + o) * H + h;
}

/* Address of value element (block p, kv head g, dim h, offset o). */
static size_t value_index(int64_t p, int g, int h, int o, int K, int bs, int H)
{
    return (((size_t)p * K + g) * H + h) * bs + o;
}

/*
 * Append (lesson step 1, in paged form): for each new token i whose slot is
 * not negative, copy k[i][g][:] and v[i][g][:] bit for bit into the cache
 * position (slot / bs, g, slot % bs).  Negative slots are padding and skipped.
 */
int oracle_append(const uint16_t *k, const uint16_t *v, const int64_t *slot_mapping,
                  uint16_t *key_cache, uint16_t *value_cache,
                  int T, int K, int H, int bs, int64_t num_blocks)
{
    for (int i = 0; i < T; i++) {
        int64_t s = slot_mapping[i];
        if (s < 0)
            continue;
        if (s >= num_blocks * (int64_t)bs)
            return -1;
        int64_t p = s / bs;
        int o = (int)(s % bs);
        for (int g = 0; g < K; g++)
            for (int h = 0; h < H; h++) {
                size_t src = ((size_t)i * K + g) * H + h;
                key_cache[key_index(p, g, o, h, K, bs, H)] = k[src];
                value_cache[value_index(p, g, h, o, K, bs, H)] = v[src];
            }
    }
    return 0;
}

/*
 * Copy-on-write block split ("CS336 Lecture 10: Inference", part 6: blocks
 * shared by several sequences are copied when one of them must write into
 * its own version): for each pair i, every element of physical block
 * src[i] -- all KV heads, all offsets, all dims, in both pools -- is copied
 * bit for bit to block dst[i].  The pools hold elem_bytes bytes per element
 * (2 for bf16, 1 for E4M3 codes); they are handled as raw bytes.  Pairs are
 * applied in order; a negative src or dst skips the pair.
 */
int oracle_copy_blocks(uint8_t *key_cache, uint8_t *value_cache, const int32_t *src,
                       const int32_t *dst, int n, int K, int H, int bs, int elem_bytes,
                       int64_t num_blocks)
{
    for (int i = 0; i < n; i++) {
        if (src[i] < 0 || dst[i] < 0)
            continue;
        if (src[i] >= num_blocks || dst[i] >= num_blocks)
            return -1;
        for (int g = 0; g < K; g++)
            for (int o = 0; o < bs; o++)
                for (int h = 0; h < H; h++)
                    for (int e = 0; e < elem_bytes; e++) {
                        size_t ks = key_index(src[i], g, o, h, K, bs, H) * elem_bytes + e;
                        size_t kd = key_index(dst[i], g, o, h, K, bs, H) * elem_bytes + e;
                        size_t vs = value_index(src[i], g, h, o, K, bs, H) * elem_bytes + e;
                        size_t vd = value_index(dst[i], g, h, o, K, bs, H) * elem_bytes + e;
                        key_cache[kd] = key_cache[ks];
                        value_cache[vd] = value_cache[vs];
                    }
    }
    return 0;
}

/*
 * Append into FP8 pools: the same scatter, storing each value's quantised code
 * (see the header comment).  k_inv / v_inv are the fp32 inverse scales.
 */
int oracle_append_fp8(const uint16_t *k, const uint16_t *v, const int64_t *slot_mapping,
                      uint8_t *key_cache, uint8_t *value_cache, float k_inv, float v_inv,
                      int T, int K, int H, int bs, int64_t num_blocks)
{
    for (int i = 0; i < T; i++) {
        int64_t s = slot_mapping[i];
        if (s < 0)
            continue;
        if (s >= num_blocks * (int64_t)bs)
            return -1;
        int64_t p = s / bs;
        int o = (int)(s % bs);
        for (int g = 0; g < K; g++)
            for (int h = 0; h < H; h++) {
                size_t src = ((size_t)i * K + g) * H + h;
                key_cache[key_index(p, g, o, h, K, bs, H)] = oracle_e4m3_quantize(k[src], k_inv);
                value_cache[value_index(p, g, h, o, K, bs, H)] =
                    oracle_e4m3_quantize(v[src], v_inv);
            }
    }
    return 0;
}

/*
 * One output row (query row qrow of query head n): the definition of
 * softmax(q K^T * scale) V over positions first .. ctx - 1 of the sequence
 * whose block-table row is `table`, gathering each position t through it.
 * `scores` is caller scratch of length ctx.  Writes H doubles to `row`
 * (zeros when the range is empty).
 */
static int decode_row(double *row, double *scores,
                      const uint16_t *qrow, const void *key_cache,
                      const void *value_cache, int dtype, double k_scale, double v_scale,
                      const int32_t *table, int first, int ctx, int n, float scale,
                      int N, int K, int H, int bs, int64_t num_blocks)
{
    int G = N / K;
    int g = n / G;
    double sc = (double)scale;

    for (int h = 0; h < H; h++)
        row[h] = 0.0;
    if (first >= ctx)
        return 0;

    double m = -INFINITY;
    for (int t = first; t < ctx; t++) {
        int64_t p = table[t / bs];
        int o = t % bs;
        if (p < 0 || p >= num_blocks)
            return -1;
        double dot = 0.0;
        for (int h = 0; h < H; h++)
            dot += bf16_to_double(qrow[h]) *
                   cache_value(key_cache, key_index(p, g, o, h, K, bs, H), dtype, k_scale);
        scores[t] = sc * dot;
        if (scores[t] > m)
            m = scores[t];
    }
    double z = 0.0;
    for (int t = first; t < ctx; t++) {
        scores[t] = exp(scores[t] - m);
        z += scores[t];
    }
    for (int t = first; t < ctx; t++) {
        int64_t p = table[t / bs];
        int o = t % bs;
        for (int h = 0; h < H; h++)
            row[h] += scores[t] *
                      cache_value(value_cache, value_index(p, g, h, o, K, bs, H), dtype, v_scale);
    }
    for (int h = 0; h < H; h++)
        row[h] /= z;
    return 0;
}

static int check_shape(const int32_t *context_lens, int B, int N, int K, int bs,
                       int max_blocks)
{
    if (B < 0 || N <= 0 || K <= 0 || N % K != 0 || bs <= 0 || max_blocks < 0)
        return -1;
    for (int b = 0; b < B; b++)
        if (context_lens[b] < 0 || context_lens[b] > (int64_t)max_blocks * bs)
            return -1;
    return 0;
}

/*
 * Decode attention for every (sequence, query head): out[b][n][h], double.
 * `scratch` must hold max(context_lens) doubles per OpenMP thread; the
 * Python wrapper allocates it.
 */
static int decode_all(double *out, const uint16_t *q, const void *key_cache,
                      const void *value_cache, int dtype, double k_scale, double v_scale,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      int B, int N, int K, int H, int bs, int max_blocks,
                      int64_t num_blocks, double *scratch, int scratch_stride)
{
    if (check_shape(context_lens, B, N, K, bs, max_blocks))
        return -1;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int r = 0; r < B * N; r++) {
        int b = r / N, n = r % N;
        int tid = thread_id();
        if (context_lens[b] > scratch_stride) {
            status |= 1;
            continue;
        }
        status |= decode_row(out + (size_t)r * H, scratch + (size_t)tid * scratch_stride,
                             q + ((size_t)b * N + n) * H, key_cache, value_cache, dtype,
                             k_scale, v_scale, block_tables + (size_t)b * max_blocks,
                             0, context_lens[b], n, scale, N, K, H, bs, num_blocks) != 0;
    }
    return status ? -1 : 0;
}

/*
 * The same rows, but only the R (b, n) pairs listed: lets a test check
 * sampled outputs of a workload too large to recompute whole.
 */
static int decode_rows_all(double *out_rows, const int32_t *rows_b, const int32_t *rows_n,
                           int R, const uint16_t *q, const void *key_cache,
                           const void *value_cache, int dtype, double k_scale, double v_scale,
                           const int32_t *block_tables, const int32_t *context_lens,
                           float scale, int B, int N, int K, int H, int bs, int max_blocks,
                           int64_t num_blocks, double *scratch, int scratch_stride)
{
    if (check_shape(context_lens, B, N, K, bs, max_blocks))
        return -1;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int r = 0; r < R; r++) {
        int b = rows_b[r], n = rows_n[r];
        int tid = thread_id();
        if (b < 0 || b >= B || n < 0 || n >= N || context_lens[b] > scratch_stride) {
            status |= 1;
            continue;
        }
        status |= decode_row(out_rows + (size_t)r * H, scratch + (size_t)tid * scratch_stride,
                             q + ((size_t)b * N + n) * H, key_cache, value_cache, dtype,
                             k_scale, v_scale, block_tables + (size_t)b * max_blocks,
                             0, context_lens[b], n, scale, N, K, H, bs, num_blocks) != 0;
    }
    return status ? -1 : 0;
}

int oracle_decode(double *out, const uint16_t *q, const uint16_t *key_cache,
                  const uint16_t *value_cache, const int32_t *block_tables,
                  const int32_t *context_lens, float scale,
                  int B, int N, int K, int H, int bs, int max_blocks,
                  int64_t num_blocks, double *scratch, int scratch_stride)
{
    return decode_all(out, q, key_cache, value_cache, KV_BF16, 1.0, 1.0, block_tables,
                      context_lens, scale, B, N, K, H, bs, max_blocks, num_blocks, scratch,
                      scratch_stride);
}

/* FP8 pools: keys and values are their codes times k_scale / v_scale. */
int oracle_decode_fp8(double *out, const uint16_t *q, const uint8_t *key_cache,
                      const uint8_t *value_cache, float k_scale, float v_scale,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      int B, int N, int K, int H, int bs, int max_blocks,
                      int64_t num_blocks, double *scratch, int scratch_stride)
{
    return decode_all(out, q, key_cache, value_cache, KV_FP8, k_scale, v_scale, block_tables,
                      context_lens, scale, B, N, K, H, bs, max_blocks, num_blocks, scratch,
                      scratch_stride);
}

int oracle_decode_rows(double *out_rows, const int32_t *rows_b, const int32_t *rows_n, int R,
                       const uint16_t *q, const uint16_t *key_cache,
                       const uint16_t *value_cache, const int32_t *block_tables,
                       const int32_t *context_lens, float scale,
                       int B, int N, int K, int H, int bs, int max_blocks,
                       int64_t num_blocks, double *scratch, int scratch_stride)
{
    return decode_rows_all(out_rows, rows_b, rows_n, R, q, key_cache, value_cache, KV_BF16,
                           1.0, 1.0, block_tables, context_lens, scale, B, N, K, H, bs,
                           max_blocks, num_blocks, scratch, scratch_stride);
}

int oracle_decode_rows_fp8(double *out_rows, const int32_t *rows_b, const int32_t *rows_n,
                           int R, const uint16_t *q, const uint8_t *key_cache,
                           const uint8_t *value_cache, float k_scale, float v_scale,
                           const int32_t *block_tables, const int32_t *context_lens,
                           float scale, int B, int N, int K, int H, int bs, int max_blocks,
                           int64_t num_blocks, double *scratch, int scratch_stride)
{
    return decode_rows_all(out_rows, rows_b, rows_n, R, q, key_cache, value_cache, KV_FP8,
                           k_scale, v_scale, block_tables, context_lens, scale, B, N, K, H,
                           bs, max_blocks, num_blocks, scratch, scratch_stride);
}

/*
 * Several query tokens per sequence: the Q tokens of a speculative-decoding
 * verification pass (the lesson's speculative-decoding section: the target
 * model checks all draft tokens in one forward pass), appended to the cache
 * before attention like a single decode token.  The lesson's Build-It step 2
 * masks, for seq_len_q > 1, every score whose key index exceeds the query
 * index by seq_len_k - seq_len_q or more (an upper triangle anchored at the
 * bottom-right corner), so query i of Q -- the token at position
 * ctx - Q + i -- sees positions 0 .. ctx - Q + i, as if the tokens had been
 * decoded one after another.  A query that sees no position (ctx < Q - i)
 * gets zeros, like an empty sequence.
 * q and out are [B][Q][N][H]; kv_dtype is KV_BF16 (pools of bf16 bits) or
 * KV_FP8 (E4M3 codes with scales k_scale, v_scale).
 */
static int visible_positions(int ctx, int Q, int i)
{
    int v = ctx - Q + i + 1;
    return v < 0 ? 0 : v;
}

int oracle_decode_multi(double *out, const uint16_t *q, const void *key_cache,
                        const void *value_cache, int kv_dtype, float k_scale, float v_scale,
                        const int32_t *block_tables, const int32_t *context_lens, float scale,
                        int B, int Q, int N, int K, int H, int bs, int max_blocks,
                        int64_t num_blocks, double *scratch, int scratch_stride)
{
    if (Q < 1 || (kv_dtype != KV_BF16 && kv_dtype != KV_FP8) ||
        check_shape(context_lens, B, N, K, bs, max_blocks))
        return -1;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int r = 0; r < B * Q * N; r++) {
        int b = r / (Q * N), i = (r / N) % Q, n = r % N;
        int tid = thread_id();
        if (context_lens[b] > scratch_stride) {
            status |= 1;
            continue;
        }
        status |= decode_row(out + (size_t)r * H, scratch + (size_t)tid * scratch_stride,
                             q + (size_t)r * H, key_cache, value_cache, kv_dtype, k_scale,
                             v_scale, block_tables + (size_t)b * max_blocks,
                             0, visible_positions(context_lens[b], Q, i), n, scale, N, K, H, bs,
                             num_blocks) != 0;
    }
    return status ? -1 : 0;
}

/* Rows (rows_b[r], rows_i[r], rows_n[r]) of oracle_decode_multi only. */
int oracle_decode_multi_rows(double *out_rows, const int32_t *rows_b, const int32_t *rows_i,
                             const int32_t *rows_n, int R, const uint16_t *q,
                             const void *key_cache, const void *value_cache, int kv_dtype,
                             float k_scale, float v_scale, const int32_t *block_tables,
                             const int32_t *context_lens, float scale, int B, int Q, int N,
                             int K, int H, int bs, int max_blocks, int64_t num_blocks,
                             double *scratch, int scratch_stride)
{
    if (Q < 1 || (kv_dtype != KV_BF16 && kv_dtype != KV_FP8) ||
        check_shape(context_lens, B, N, K, bs, max_blocks))
        return -1;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int r = 0; r < R; r++) {
        int b = rows_b[r], i = rows_i[r], n = rows_n[r];
        int tid = thread_id();
        if (b < 0 || b >= B || i < 0 || i >= Q || n < 0 || n >= N ||
            context_lens[b] > scratch_stride) {
            status |= 1;
            continue;
        }
        status |= decode_row(out_rows + (size_t)r * H, scratch + (size_t)tid * scratch_stride,
                             q + (((size_t)b * Q + i) * N + n) * H, key_cache, value_cache,
                             kv_dtype, k_scale, v_scale, block_tables + (size_t)b * max_blocks,
                             0, visible_positions(context_lens[b], Q, i), n, scale, N, K, H, bs,
                             num_blocks) != 0;
    }
    return status ? -1 : 0;
}

/*
 * Sliding-window decode ("CS336 Lecture 10: Inference", part 6, local or
 * sliding-window attention: each generated token looks only at the last
 * window tokens; "Week 11. Inference", step 1: a window caps the cache at
 * its size): sequence b's query attends positions
 * max(0, ctx_b - window) .. ctx_b - 1, the new token included.  window >= 1.
 * q and out are [B][N][H]; pools as for oracle_decode_multi.
 */
int oracle_decode_window(double *out, const uint16_t *q, const void *key_cache,
                         const void *value_cache, int kv_dtype, float k_scale, float v_scale,
                         const int32_t *block_tables, const int32_t *context_lens, float scale,
                         int window, int B, int N, int K, int H, int bs, int max_blocks,
                         int64_t num_blocks, double *scratch, int scratch_stride)
{
    if (window < 1 || (kv_dtype != KV_BF16 && kv_dtype != KV_FP8) ||
        check_shape(context_lens, B, N, K, bs, max_blocks))
        return -1;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int r = 0; r < B * N; r++) {
        int b = r / N, n = r % N;
        int tid = thread_id();
        int ctx = context_lens[b];
        int first = ctx - window > 0 ? ctx - window : 0;
        if (ctx > scratch_stride) {
            status |= 1;
            continue;
        }
        status |= decode_row(out + (size_t)r * H, scratch + (size_t)tid * scratch_stride,
                             q + (size_t)r * H, key_cache, value_cache, kv_dtype, k_scale,
                             v_scale, block_tables + (size_t)b * max_blocks, first, ctx, n,
                             scale, N, K, H, bs, num_blocks) != 0;
    }
    return status ? -1 : 0;
}

/*
 * Split-context form of the same result, used to pin the log-sum-exp merge
 * ("CS336 Lecture 10: Inference", part 6, names FlashDecoding: the context
 * is cut into pieces that are reduced separately and then combined).
 * Piece j covers positions [j*part, min((j+1)*part, ctx)).  For each piece
 * the oracle keeps its own maximum m_j, sum l_j = sum exp(s - m_j) and
 * unnormalised o_j = sum exp(s - m_j) v; the pieces are then combined with
 * M = max m_j, w_j = exp(m_j - M), out = sum w_j o_j / sum w_j l_j.
 * Only used on small inputs; loops are serial.
 */
int oracle_decode_split(double *out, const uint16_t *q, const uint16_t *key_cache,
                        const uint16_t *value_cache, const int32_t *block_tables,
                        const int32_t *context_lens, float scale,
                        int B, int N, int K, int H, int bs, int max_blocks,
                        int64_t num_blocks, int part,
                        double *piece_m, double *piece_l, double *piece_o, int max_pieces)
{
    if (check_shape(context_lens, B, N, K, bs, max_blocks) || part <= 0)
        return -1;
    int G = N / K;
    double sc = (double)scale;
    for (int b = 0; b < B; b++) {
        int ctx = context_lens[b];
        int pieces = (ctx + part - 1) / part;
        if (pieces > max_pieces)
            return -1;
        const int32_t *table = block_tables + (size_t)b * max_blocks;
        for (int n = 0; n < N; n++) {
            int g = n / G;
            const uint16_t *qrow = q + ((size_t)b * N + n) * H;
            double *row = out + ((size_t)b * N + n) * H;
            for (int j = 0; j < pieces; j++) {
                int t0 = j * part, t1 = t0 + part < ctx ? t0 + part : ctx;
                double m = -INFINITY;
                for (int t = t0; t < t1; t++) {
                    int64_t p = table[t / bs];
                    if (p < 0 || p >= num_blocks)
                        return -1;
                    double dot = 0.0;
                    for (int h = 0; h < H; h++)
                        dot += bf16_to_double(qrow[h]) *
                               bf16_to_double(key_cache[key_index(p, g, t % bs, h, K, bs, H)]);
                    if (sc * dot > m)
                        m = sc * dot;
                }
                double l = 0.0;
                double *o = piece_o + (size_t)j * H;
                for (int h = 0; h < H; h++)
                    o[h] = 0.0;
                for (int t = t0; t < t1; t++) {
                    int64_t p = table[t / bs];
                    double dot = 0.0;
                    for (int h = 0; h < H; h++)
                        dot += bf16_to_double(qrow[h]) *
                               bf16_to_double(key_cache[key_index(p, g, t % bs, h, K, bs, H)]);
                    double w = exp(sc * dot - m);
                    l += w;
                    for (int h = 0; h < H; h++)
                        o[h] += w * bf16_to_double(
                                        value_cache[value_index(p, g, h, t % bs, K, bs, H)]);
                }
                piece_m[j] = m;
                piece_l[j] = l;
            }
            double M = -INFINITY;
            for (int j = 0; j < pieces; j++)
                if (piece_m[j] > M)
                    M = piece_m[j];
            double L = 0.0;
            for (int h = 0; h < H; h++)
                row[h] = 0.0;
            for (int j = 0; j < pieces; j++) {
                double w = exp(piece_m[j] - M);
                L += w * piece_l[j];
                for (int h = 0; h < H; h++)
                    row[h] += w * piece_o[(size_t)j * H + h];
            }
            if (pieces > 0)
                for (int h = 0; h < H; h++)
                    row[h] /= L;
        }
    }
    return 0;
}

/*
 * KV-cache size formula, "Optimización de la inferencia" lesson, KV-cache
 * concept section (and "Week 11. Inference", step 2): bytes =
 * 2 (K and V) * layers * kv_heads * head_dim * tokens * bytes_per_value.
 */
int64_t oracle_kv_cache_bytes(int64_t layers, int64_t kv_heads, int64_t head_dim,
                              int64_t tokens, int64_t bytes_per_value)
{
    return 2 * layers * kv_heads * head_dim * tokens * bytes_per_value;
}
