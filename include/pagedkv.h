/*
 * pagedkv.h -- C ABI of the paged-KV decode-attention library (libpagedkv.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * Two operations make one decode step of one attention layer:
 *
 *   paged_kv_append         writes the step's new K/V rows into the paged
 *                           cache at slot-mapped positions;
 *   paged_decode_attention  computes, for every sequence and query head,
 *                           softmax(q . K^T * scale) . V over the sequence's
 *                           cached positions, gathered through its block table.
 *
 * What they compute is defined on these pages:
 *   - "Optimización de la inferencia" (AI Engineering from Scratch, phase 10,
 *     lesson 12; the same lesson in Chinese as "推理优化 (Inference
 *     Optimization)"), Build-It step 1 (a KV cache: new keys/values are
 *     written at the next position, attention reads every position so far)
 *     and step 2 (attention with the cache: scaled scores, maximum
 *     subtracted, normalised exponentials, weighted sum of V; one query token
 *     needs no causal mask); and its PagedAttention section (the cache lives
 *     in fixed-size pages anywhere in GPU memory, found through a
 *     per-request page table, pages of 16 tokens being typical).
 *   - "CS336 Lecture 10: Inference", part 1 (notation B, N, K, H; generation
 *     attention reads the whole cache for one query token per sequence and is
 *     memory bound), part 3 (GQA: each of K KV heads serves N/K query heads)
 *     and part 6 (PagedAttention blocks, shared prefix blocks, a kernel that
 *     fuses the block reads with attention).
 *   - "Week 11. Inference", step 2 (a new token computes only its own q, k, v
 *     and attends to the stored ones).
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer (HIP global memory) unless
 *     stated otherwise.  The caller owns all memory; the library allocates
 *     nothing and keeps no state except a per-device attribute cache (and
 *     the static scratch array of paged_decode_attention_noalloc).
 *   - bf16 data is passed as raw 16-bit patterns (type-erased `void*`).
 *   - `stream` is a hipStream_t passed as `void*` (NULL = the null stream).
 *     Calls only enqueue work on that stream; they never synchronise, so
 *     buffers must stay alive until the stream has run the work.
 *   - Calls can be captured into a HIP graph: they enqueue only kernel
 *     launches (no memset, copy or allocation), and a replay reads the
 *     device buffers as they are at replay time (context lengths, block
 *     tables, queries may change between replays within the sizes given at
 *     capture).
 *   - Every argument check happens on the host before any launch.  The return
 *     value is PKV_OK (0) or a negative pkv_status; nothing is enqueued when
 *     a check fails.  Values stored in device memory (block ids, slots,
 *     context lengths) cannot be checked without a device-to-host copy; the
 *     kernels clamp them to stay inside the buffers, as documented per call,
 *     but the numeric result for such a sequence is then unspecified.
 *
 * Memory layouts (the pages leave these open; the library fixes them)
 *   key_cache   [num_blocks][K][block_size][H]   bf16: each token's key is a
 *               contiguous row of H values.
 *   value_cache [num_blocks][K][H][block_size]   bf16: each (head, dim) row
 *               holds the block's tokens, so one value tile is stored
 *               transposed (the layout the matrix-core operand wants).
 *   A slot is physical_block * block_size + offset_in_block.
 *   Query head n reads KV head n / (N / K).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_NULL = -1,        /* a required pointer is NULL                         */
    PKV_ERR_SHAPE = -2,       /* sizes inconsistent or out of range                 */
    PKV_ERR_UNSUPPORTED = -3, /* head_dim, block_size or group size not built in    */
    PKV_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                   */
    PKV_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required         */
    PKV_ERR_LAUNCH = -6,      /* the HIP runtime refused the launch                 */
    PKV_ERR_DEVICE = -7,      /* no HIP device / device query failed                */
    PKV_ERR_SCRATCH = -8      /* paged_decode_attention_noalloc: the problem needs
                                 more than PKV_NOALLOC_SCRATCH_BYTES of scratch     */
} pkv_status;

/* Supported shapes (compile-time kernel variants). */
#define PKV_BLOCK_SIZE 16          /* tokens per cache block (the usual size)     */
#define PKV_BLOCK_SIZE_LARGE 32    /* the other block size built in               */
#define PKV_MAX_GROUP 16           /* largest N / K (query heads per KV head)     */
#define PKV_PARTITION_GRAIN 32     /* partition sizes are multiples of this       */
#define PKV_MAX_PARTITION 1024
#define PKV_MAX_MQ_PARTITION (1 << 20)  /* partition cap of the multi-query call  */
#define PKV_MAX_QUERY_ROWS 64      /* num_queries * (N / K) for the multi-query call */
#define PKV_MAX_PREFIX_ROWS 1024   /* max_members * (N / K) for the prefix-aware call */

/* KV pool element types of paged_decode_attention_mq. */
#define PKV_KV_BF16 0              /* bf16 bit patterns                           */
#define PKV_KV_FP8_E4M3 1          /* OCP FP8 E4M3 codes, one scale per pool      */

/*
 * paged_kv_append -- write one decode step's keys and values into the cache.
 *
 *   k, v           [num_tokens][num_kv_heads][head_dim] bf16, contiguous.
 *   slot_mapping   [num_tokens] int64: token i goes to slot slot_mapping[i];
 *                  a negative slot means "padding, skip this token".
 *   key_cache      [num_blocks][num_kv_heads][block_size][head_dim] bf16,
 *   value_cache    [num_blocks][num_kv_heads][head_dim][block_size] bf16,
 *                  both modified in place; positions not named by a slot are
 *                  left untouched.
 * The copy is bit exact.  Two tokens naming the same slot race (which one
 * lands is unspecified).  A slot >= num_blocks * block_size is skipped (the
 * kernel never writes outside the pools).
 * Checks: NULL pointers (when num_tokens > 0), sizes, head_dim in {64, 128},
 * block_size 16 or 32, 16-byte alignment of k, v, key_cache, value_cache.
 * Cites: the lesson's Build-It step 1 (write at the next position) in the
 * paged form of its PagedAttention section.
 */
int paged_kv_append(const void *k, const void *v, const int64_t *slot_mapping,
                    void *key_cache, void *value_cache,
                    int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int64_t num_blocks, void *stream);

/*
 * paged_decode_workspace_size -- bytes of device workspace that
 * paged_decode_attention needs for this shape and partition_size (0 when no
 * workspace is needed).  Host-only and pure: the same arguments always give
 * the same size, on any device.
 */
size_t paged_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t max_context_len,
                                   int32_t partition_size);

/*
 * paged_decode_attention -- one decode step of attention over the paged cache.
 *
 *   out            [num_seqs][num_heads][head_dim] float32 (written).
 *   q              [num_seqs][num_heads][head_dim] bf16 (one query token per
 *                  sequence).
 *   key_cache, value_cache   as in paged_kv_append, num_blocks blocks each.
 *   block_tables   [num_seqs][max_blocks_per_seq] int32: logical block j of
 *                  sequence b is physical block block_tables[b][j].  Entries
 *                  past the sequence's last block do not affect the result.
 *   context_lens   [num_seqs] int32: tokens in each sequence's cache (append
 *                  this step's token first and count it).  Values above
 *                  max_context_len are treated as max_context_len, negative
 *                  values as 0; a sequence of length 0 yields zeros.
 *   scale          softmax scale applied to q . k (1/sqrt(head_dim) on the
 *                  pages); any finite value.  A negative scale is applied
 *                  by negating the query (exact in bf16); a magnitude
 *                  below FLT_MIN (zero included) acts as FLT_MIN, which for
 *                  scores below 2^100 in magnitude gives every position the
 *                  same weight, as zero does.
 *   num_kv_heads   K; num_heads (N) must be a multiple with N/K <= 16.
 *   block_size     16 or 32 (tokens per block; the kernels read 32-token
 *                  chunks: two blocks of 16 or one of 32).
 *   max_blocks_per_seq   row stride of block_tables.
 *   max_context_len      host-known upper bound of context_lens, at most
 *                  max_blocks_per_seq * block_size.
 *   num_blocks     blocks in each cache pool.
 *   partition_size how the context is split across waves (the split-K of
 *                  FlashDecoding, named in "CS336 Lecture 10: Inference",
 *                  part 6; partial results are merged with the log-sum-exp
 *                  rule):
 *                  0  token-balanced schedule: the cached tokens of the whole
 *                     batch are divided evenly over as many waves as the GPU
 *                     holds at once, whatever the mix of context lengths
 *                     (three kernel launches);
 *                  P  fixed partitions of P tokens (a multiple of 32 in
 *                     [32, 1024]) of each sequence.  When one partition
 *                     covers max_context_len: one wave per (KV head,
 *                     sequence), one launch.  Otherwise each wave of the
 *                     token-balanced schedule takes a run of whole
 *                     partitions and writes each one's partial, then the
 *                     merge over partitions (two launches, three when
 *                     num_seqs > 256); the result is the same as one wave
 *                     per partition.
 *   workspace, workspace_bytes   device scratch of at least
 *                  paged_decode_workspace_size(...) bytes, 16-byte aligned;
 *                  may be NULL when that size is 0.  Its contents on entry
 *                  do not matter; calls sharing one workspace must not run
 *                  concurrently.
 * Block ids outside [0, num_blocks) are read as block 0 (no out-of-bounds
 * access; that sequence's result is unspecified).
 * Arithmetic: bf16 inputs, fp32 accumulation (matrix cores for q.K^T and
 * P.V, with P carried as a two-term bf16 sum), fp32 output.  The result is
 * bit-deterministic for given inputs, partition_size, max_context_len and
 * device: no atomics, and the reduction order depends only on logical
 * positions and the kernels the host picks.  With partition_size 0, a batch
 * whose num_seqs * num_kv_heads pairs, four waves each, fit one round of the
 * device's waves (4 per compute unit) and whose max_context_len spans at
 * most 256 KiB of keys and values per pair (512 tokens of bf16 at head_dim
 * 128, 1,024 of FP8 or at head_dim 64) runs as one launch (a workgroup per
 * pair merging its four waves' partial results in LDS); otherwise on the
 * persistent token-balanced kernel.  Within each, a larger max_context_len gives the same bits; the
 * two agree to rounding (about 1e-6 relative).
 */
int paged_decode_attention(float *out, const void *q,
                           const void *key_cache, const void *value_cache,
                           const int32_t *block_tables, const int32_t *context_lens,
                           float scale, int32_t num_kv_heads, int32_t block_size,
                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                           int32_t max_blocks_per_seq, int32_t max_context_len,
                           int64_t num_blocks, int32_t partition_size,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * FP8 KV pools.  The same two operations over pools that hold one-byte OCP
 * FP8 E4M3 codes (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * no infinities; codes 0x7F / 0xFF are NaN) in the same layouts, with one
 * scale per pool: a stored code c stands for e4m3(c) * k_scale in the key
 * pool and e4m3(c) * v_scale in the value pool.  Quantising the cache to 8
 * bits is the lever "Week 11. Inference", step 2, names for halving the
 * cache, and the lesson's exercises ("Optimización de la inferencia")
 * ask for the FP8 cache's capacity; the pages fix neither the 8-bit format
 * nor the rounding, so the library takes E4M3 with round-to-nearest-even and
 * a per-pool scale.
 *
 * paged_kv_append_fp8 -- as paged_kv_append, except that each bf16 value x
 *   is stored as the code nearest to y = fp32(x * fp32(1 / scale)) (the pool's
 *   scale), where y is first clamped to [-448, 448] (the largest finite
 *   code); ties go to the code with an even last bit; NaN stores 0xFF; the
 *   sign of zero is kept (-0 stores 0x80).
 *   key_cache      [num_blocks][num_kv_heads][block_size][head_dim] uint8,
 *   value_cache    [num_blocks][num_kv_heads][head_dim][block_size] uint8.
 *   k_scale, v_scale   positive, finite, with finite fp32 inverses; else
 *                  PKV_ERR_SHAPE.  Other checks as for paged_kv_append.
 *   The codes are bit exact against that definition.
 *
 * paged_decode_attention_fp8 -- as paged_decode_attention over FP8 pools
 *   (same arguments, plus k_scale and v_scale as above; the workspace is
 *   sized by paged_decode_workspace_size with the same arguments).  Codes are
 *   widened to bf16 exactly before the matrix-core products; k_scale is
 *   folded into the softmax scale and v_scale into the output normalisation,
 *   both in fp32.  q and out are as in paged_decode_attention.
 */
int paged_kv_append_fp8(const void *k, const void *v, const int64_t *slot_mapping,
                        void *key_cache, void *value_cache, float k_scale, float v_scale,
                        int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int64_t num_blocks, void *stream);

int paged_decode_attention_fp8(float *out, const void *q,
                               const void *key_cache, const void *value_cache,
                               const int32_t *block_tables, const int32_t *context_lens,
                               float scale, float k_scale, float v_scale,
                               int32_t num_kv_heads, int32_t block_size,
                               int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int32_t max_context_len,
                               int64_t num_blocks, int32_t partition_size,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_decode_attention_mq -- attention for num_queries (Q) query tokens per
 * sequence: the Q tokens a speculative-decoding verification pass checks at
 * once (the lesson's speculative-decoding section: the target model processes
 * all draft tokens in one forward pass), appended to the cache beforehand
 * with paged_kv_append / paged_kv_append_fp8 (Q slots per sequence) and
 * counted in context_lens.
 *
 * Query token i (0 <= i < Q) of sequence b stands at position ctx_b - Q + i
 * and attends positions 0 .. ctx_b - Q + i: the causal mask of the lesson's
 * Build-It step 2 for seq_len_q > 1, an upper triangle anchored at the
 * bottom-right corner ("Week 11. Inference" warns against the top-left
 * alignment).  The result equals Q single-token decode steps.  A query that
 * sees no position (ctx_b < Q - i) gets zeros.
 *
 *   out            [num_seqs][Q][num_heads][head_dim] float32 (written).
 *   q              [num_seqs][Q][num_heads][head_dim] bf16.
 *   kv_dtype       PKV_KV_BF16 (k_scale, v_scale ignored) or PKV_KV_FP8_E4M3
 *                  (pools of E4M3 codes; scales as for the _fp8 calls).
 *   num_queries    Q >= 1 with Q * (N / K) <= PKV_MAX_QUERY_ROWS.
 *   partition_size fixed partitions only: a multiple of 32 in
 *                  [32, PKV_MAX_MQ_PARTITION].  One wave per (partition, KV
 *                  head, sequence, column group); a partition size that
 *                  gives about as many waves as the device holds at once (4
 *                  per CU) fills it in a single round.
 *   workspace      at least paged_decode_mq_workspace_size(num_seqs,
 *                  num_queries, num_heads, head_dim, max_context_len,
 *                  partition_size) bytes (0 when one partition covers
 *                  max_context_len), 16-byte aligned.  Its contents on entry
 *                  do not matter; calls sharing one workspace must not run
 *                  concurrently.
 * Other arguments, checks and clamping as for paged_decode_attention.  The
 * Q * G (query token, head) pairs of a KV head's group share each load of
 * its keys and values.  Several partitions are merged with the log-sum-exp
 * rule by a second launch, except when max_context_len spans exactly two
 * partitions and a wave holds at most three column tiles: then of the two
 * partition waves of a (sequence, KV head), the one that finishes second
 * merges both partials itself (one launch).  It finds out through an atomic
 * exchange of a per-call 64-bit tag in the workspace (a process-wide
 * counter from a random start), so the workspace needs no clearing; the
 * merge takes the partitions in order with the merge launch's arithmetic, so
 * the result is the same whichever wave merges.  A call made while its
 * stream is being captured into a graph takes the merge launch instead (a
 * replay repeats the captured tag), with the same result.
 */
size_t paged_decode_mq_workspace_size(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                      int32_t head_dim, int32_t max_context_len,
                                      int32_t partition_size);

int paged_decode_attention_mq(float *out, const void *q,
                              const void *key_cache, const void *value_cache,
                              const int32_t *block_tables, const int32_t *context_lens,
                              float scale, int32_t kv_dtype, float k_scale, float v_scale,
                              int32_t num_kv_heads, int32_t block_size,
                              int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                              int32_t head_dim, int32_t max_blocks_per_seq,
                              int32_t max_context_len, int64_t num_blocks,
                              int32_t partition_size, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * paged_decode_attention_window -- sliding-window decode: each sequence's
 * query attends only its last `window` positions, max(0, ctx_b - window) ..
 * ctx_b - 1, the step's new token included ("CS336 Lecture 10: Inference",
 * part 6: with local or sliding-window attention a generated token depends
 * only on the last tokens; "Week 11. Inference", step 1: a window caps the
 * cache at its size).  Positions before the window are never read (a 32-token
 * chunk holding the window's start is read whole, its earlier positions
 * masked), so the bytes read per step are bounded by the window.
 *   window         >= 1; a window at least the context is full attention.
 *   kv_dtype, k_scale, v_scale   as for paged_decode_attention_mq.
 * Other arguments, the workspace (paged_decode_workspace_size with the same
 * partition_size) and both partitioning modes as for paged_decode_attention.
 */
int paged_decode_attention_window(float *out, const void *q,
                                  const void *key_cache, const void *value_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  float scale, int32_t kv_dtype, float k_scale, float v_scale,
                                  int32_t window, int32_t num_kv_heads, int32_t block_size,
                                  int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  int64_t num_blocks, int32_t partition_size,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Shared prompt prefixes.  Sequences that share a prefix point their block
 * tables at the same physical blocks; a block is copied before one of its
 * sharers writes into it ("CS336 Lecture 10: Inference", part 6: shared
 * prefix blocks, copy on write; the lesson's prefix-caching section).
 *
 * paged_kv_copy_blocks -- for each pair i, physical block dst_blocks[i]
 *   becomes a bit-exact copy of block src_blocks[i]: every KV head, offset
 *   and head dim, in both pools.  kv_dtype (PKV_KV_BF16 or PKV_KV_FP8_E4M3)
 *   fixes the element size.  A pair with an id outside [0, num_blocks) or
 *   with src == dst is skipped.  Pairs run concurrently: no block may be the
 *   destination of one pair and the source or destination of another (the
 *   result is then unspecified).  src_blocks, dst_blocks: [num_pairs] int32
 *   device arrays, num_pairs <= 65535.  Checks as for paged_kv_append.
 *
 * paged_decode_attention_prefix -- paged_decode_attention that reads each
 *   shared prefix once for all of its sharers instead of once per sharer
 *   ("CS336 Lecture 10: Inference", part 6: shared prefix blocks).  The
 *   result is plain attention over each sequence's context (paging and
 *   sharing only change where blocks are read from), up to rounding.
 *   seq_group      [num_seqs] int32: the prefix group of each sequence, -1 for
 *                  none.
 *   group_members  [num_groups][max_members] int32: the sequences of each
 *                  group, -1 padded; the first is the group's lead.  Every
 *                  sequence b with seq_group[b] = g must be listed in row g.
 *   prefix_tokens  [num_groups] int32: positions 0 .. prefix_tokens - 1 of
 *                  every member map to the same physical blocks as the lead's.
 *   max_prefix_tokens  host-known bound of prefix_tokens.
 *   Member b of group g shares positions 0 .. S_b - 1, S_b = min(
 *   prefix_tokens[g], ctx_b, ctx_lead) rounded down to a multiple of 32:
 *   the group's waves read them once for all members, in partitions of
 *   partition_size P tokens (a multiple of 32 in [32, 1024]: smaller
 *   partitions spread the shared span over more waves, each adding one
 *   partial per member row to merge); the rest of every context runs on the
 *   token-balanced schedule of paged_decode_attention with partition_size 0,
 *   in the same grid ahead of the group waves, and one merge joins both.  max_members * (N / K) <= PKV_MAX_PREFIX_ROWS.  A member whose
 *   table disagrees with the lead's over its shared span gets attention over
 *   the lead's blocks there.  Workspace: paged_decode_prefix_workspace_size
 *   bytes; kv_dtype, k_scale, v_scale as for paged_decode_attention_mq; other
 *   arguments as for paged_decode_attention.
 */
int paged_kv_copy_blocks(void *key_cache, void *value_cache,
                         const int32_t *src_blocks, const int32_t *dst_blocks,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, int32_t kv_dtype,
                         void *stream);

/* Workspace bytes paged_decode_attention_prefix needs for these sizes (0 if
 * they are invalid): the token-balanced workspace plus the group waves'
 * partials, ceil(min(max_prefix_tokens, max_context_len) rounded down to 32,
 * over partition_size) per (sequence, query head) row, plus one int32 per
 * sequence. */
size_t paged_decode_prefix_workspace_size(int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_context_len, int32_t partition_size,
                                          int32_t max_prefix_tokens);

int paged_decode_attention_prefix(float *out, const void *q,
                                  const void *key_cache, const void *value_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  float scale, int32_t kv_dtype, float k_scale, float v_scale,
                                  int32_t num_kv_heads, int32_t block_size,
                                  int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  int64_t num_blocks, int32_t partition_size,
                                  const int32_t *seq_group, const int32_t *group_members,
                                  const int32_t *prefix_tokens, int32_t num_groups,
                                  int32_t max_members, int32_t max_prefix_tokens,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * pagedkv_stream_read -- measurement helper, not part of the method: reads
 * `bytes` (a multiple of 16, 16-byte aligned) from `src` in the decode
 * kernels' access pattern -- one wave per SIMD, each reading a contiguous
 * share with non-temporal 16-byte loads, 16 KiB per step, two steps in
 * flight -- and may write one 16-byte value per wave into `sink` (at most
 * 4,096 waves; pagedkv_stream_read_sink_bytes returns the size to
 * allocate).  The rate it reaches is the achievable-bandwidth ceiling the
 * decode kernels are compared with; a launch of known size also calibrates
 * HBM read counters.  Returns PKV_ERR_NULL / _SHAPE / _ALIGN / _DEVICE /
 * _LAUNCH as the other calls do.
 */
size_t pagedkv_stream_read_sink_bytes(size_t bytes);
int pagedkv_stream_read(const void *src, size_t bytes, void *sink, void *stream);

/*
 * pagedkv_stream_copy -- measurement helper, not part of the method: copies
 * `bytes` (a multiple of 16) from src to dst (non-overlapping, 16-byte
 * aligned) with 16-byte loads and stores.  A launch that reads and writes a
 * known number of bytes, for scaling HBM read/write counters.
 */
int pagedkv_stream_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * paged_decode_attention_noalloc -- paged_decode_attention without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It allocates nothing (no hipMalloc, hipFree or allocating
 * library call): the scratch that paged_decode_attention keeps in the
 * caller's workspace (split partials, the token-balanced schedule and its
 * pieces) lives in a static device array of PKV_NOALLOC_SCRATCH_BYTES that
 * every device the library runs on holds from first use until the process
 * ends.
 *
 * Arguments, layouts, results and checks are those of paged_decode_attention
 * (same kernels, bit-identical output).  PKV_ERR_SCRATCH: the shape needs
 * more scratch than the array holds, i.e. paged_decode_workspace_size(...)
 * > PKV_NOALLOC_SCRATCH_BYTES (64 MiB covers, e.g., 2,048 sequences of 32
 * query and 8 KV heads at head_dim 128 in the token-balanced mode, or 4
 * sequences of 64 heads at 131,072 tokens in 512-token partitions).
 * Nothing in the array needs clearing between calls (every value is written
 * before it is read).  All calls on one device share its array: calls that
 * can overlap on one device (on different streams, or from several host
 * threads without ordering) race and give undefined results; calls ordered
 * on one stream are safe.  PKV_ERR_DEVICE if the array's device address
 * cannot be obtained.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int paged_decode_attention_noalloc(float *out, const void *q, const void *key_cache,
                                   const void *value_cache, const int32_t *block_tables,
                                   const int32_t *context_lens, float scale,
                                   int32_t num_kv_heads, int32_t block_size, int32_t num_seqs,
                                   int32_t num_heads, int32_t head_dim,
                                   int32_t max_blocks_per_seq, int32_t max_context_len,
                                   int64_t num_blocks, int32_t partition_size, void *stream);

/* Human-readable name of a pkv_status value (static string, never NULL). */
const char *pagedkv_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
int pagedkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
