"""Pure-Python brute force of decode attention and append, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  A second statement of
the definition, written independently of ``oracle.c``: plain nested loops over
Python floats and ``math.exp``, with the block-table gather spelled out per
position.  Sources:
  * "Optimización de la inferencia" / "推理优化 (Inference Optimization)" lesson,
    Build-It step 2 (attention with the KV cache): scaled scores, maximum
    subtracted, exponentials normalised by their sum, weighted sum of V;
  * same lesson, "PagedAttention" concept section, and "CS336 Lecture 10:
    Inference", part 6: logical position t lives in block table[t // bs] at
    offset t % bs;
  * "CS336 Lecture 10: Inference", part 3 (GQA): N/K query heads per KV head.

Inputs are Python lists/tuples of floats (already decoded from bf16) so that
nothing here depends on the oracle's bit handling.
"""
from __future__ import annotations

import math


def attend_one(qrow, keys, values, scale):
    """softmax(q . k_t * scale) weighted sum of v_t for one query row.

    keys, values: lists of per-position vectors in logical order.
    """
    if not keys:
        return [0.0] * len(qrow)
    scores = [scale * sum(a * b for a, b in zip(qrow, k)) for k in keys]
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = sum(weights)
    return [sum(w * v[h] for w, v in zip(weights, values)) / total
            for h in range(len(qrow))]


def paged_decode(q, key_cache, value_cache, block_tables, context_lens, scale):
    """Decode attention with the block-table gather done position by position.

    q[b][n][h]; key_cache[p][g][o][h]; value_cache[p][g][h][o];
    block_tables[b][j]; context_lens[b].  Returns out[b][n][h].
    """
    B = len(q)
    N = len(q[0]) if B else 0
    K = len(key_cache[0]) if key_cache else 1
    bs = len(key_cache[0][0]) if key_cache else 1
    group = N // K
    out = []
    for b in range(B):
        rows = []
        for n in range(N):
            g = n // group
            keys, values = [], []
            for t in range(context_lens[b]):
                p = block_tables[b][t // bs]
                o = t % bs
                keys.append(list(key_cache[p][g][o]))
                values.append([value_cache[p][g][h][o] for h in range(len(q[b][n]))])
            rows.append(attend_one(q[b][n], keys, values, scale))
        out.append(rows)
    return out


def paged_append(k, v, slot_mapping, key_cache, value_cache):
    """Write k[i][g][:] / v[i][g][:] at slot_mapping[i]; negative slots skipped.

    Caches are nested lists, modified in place (K rows; V columns).
    """
    bs = len(key_cache[0][0])
    for i, s in enumerate(slot_mapping):
        if s < 0:
            continue
        p, o = divmod(s, bs)
        for g in range(len(k[i])):
            for h in range(len(k[i][g])):
                key_cache[p][g][o][h] = k[i][g][h]
                value_cache[p][g][h][o] = v[i][g][h]


def paged_decode_multi(q, key_cache, value_cache, block_tables, context_lens, scale):
    """Several query tokens per sequence: q[b][r][n][h] for the seq_len_q = Q
    tokens that end the sequence's seq_len_k = context_lens[b] cached ones.

    The lesson's Build-It step 2 drops score (r, j) when the key index j
    exceeds the query index r by at least seq_len_k - seq_len_q + 1 (its
    upper-triangle mask with that diagonal offset).  Returns out[b][r][n][h].
    """
    out = []
    for b in range(len(q)):
        seq_len_q, seq_len_k = len(q[b]), context_lens[b]
        rows_b = []
        for r in range(seq_len_q):
            keep = [j for j in range(seq_len_k) if j - r < seq_len_k - seq_len_q + 1]
            N = len(q[b][r])
            K = len(key_cache[0]) if key_cache else 1
            bs = len(key_cache[0][0]) if key_cache else 1
            group = N // K
            rows_r = []
            for n in range(N):
                g = n // group
                keys = [list(key_cache[block_tables[b][j // bs]][g][j % bs]) for j in keep]
                values = [[value_cache[block_tables[b][j // bs]][g][h][j % bs]
                           for h in range(len(q[b][r][n]))] for j in keep]
                rows_r.append(attend_one(q[b][r][n], keys, values, scale))
            rows_b.append(rows_r)
        out.append(rows_b)
    return out


def copy_blocks(key_cache, value_cache, src, dst):
    """Copy-on-write split: block dst[i] becomes a copy of block src[i] (every
    head, offset and dim of both pools); pairs in order, negative ids skipped.
    Caches are nested lists, modified in place."""
    for a, b in zip(src, dst):
        if a < 0 or b < 0:
            continue
        key_cache[b] = [[list(row) for row in head] for head in key_cache[a]]
        value_cache[b] = [[list(row) for row in head] for head in value_cache[a]]


def paged_decode_window(q, key_cache, value_cache, block_tables, context_lens, scale, window):
    """Sliding window: each query looks only at the last ``window`` tokens of
    its sequence (the new one included).  Returns out[b][n][h]."""
    out = []
    bs = len(key_cache[0][0]) if key_cache else 1
    K = len(key_cache[0]) if key_cache else 1
    for b in range(len(q)):
        ctx = context_lens[b]
        last = list(range(ctx))[-window:] if window < ctx else list(range(ctx))
        group = len(q[b]) // K
        rows = []
        for n in range(len(q[b])):
            g = n // group
            keys = [list(key_cache[block_tables[b][t // bs]][g][t % bs]) for t in last]
            values = [[value_cache[block_tables[b][t // bs]][g][h][t % bs]
                       for h in range(len(q[b][n]))] for t in last]
            rows.append(attend_one(q[b][n], keys, values, scale))
        out.append(rows)
    return out
