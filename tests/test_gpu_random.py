"""Seeded random sweep of decode shapes on the GPU against the fp64 oracle.

Each case draws, from its own seed, a batch of 1 to 24 sequences, a GQA
group of 1 to 16 heads per KV head (1 to 8 KV heads), head dim 64 or 128,
context lengths that mix empty contexts, one-token contexts, exact multiples
of the block and of the 32-token chunk, and arbitrary lengths up to 1,500,
a partitioning (token-balanced or fixed partitions of 32 to 1,024 tokens),
bf16 or FP8 pools, and for a third of the cases a sliding window; the
multi-query cases add 2 to 6 query tokens per sequence.  A third set of
cases repeats the draws with blocks of 32 tokens.  The append is
checked bit-exact on the whole pools and every output row against the
oracle (the lesson's step-2 softmax, gathered through the block table).
"""
import random

import pytest
import torch

from paged_kv_cache_100_amd import workloads as W

import gpu_harness as H

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def draw_contexts(rng, B):
    picks = []
    for _ in range(B):
        kind = rng.random()
        if kind < 0.08:
            picks.append(0)
        elif kind < 0.16:
            picks.append(1)
        elif kind < 0.36:
            picks.append(rng.choice([16, 32, 48, 64, 96, 512, 1024]))
        else:
            picks.append(rng.randint(2, 1500))
    if max(picks) == 0:
        picks[0] = rng.randint(1, 700)
    return picks


def draw(seed, queries=1, bs=16):
    rng = random.Random(seed)
    G = rng.choice([1, 2, 4, 8, 16])
    K = rng.choice([1, 2, 4, 8]) if G < 16 else rng.choice([1, 2])
    B = rng.randint(1, 24)
    Hd = rng.choice([64, 128])
    kv = rng.choice(["bf16", "bf16", "fp8"])
    ctx = draw_contexts(rng, B)
    if queries > 1:
        ctx = [max(c, 0) for c in ctx]
        part = rng.choice([32, 64, 256, 1024, 2048])
        window = 0
        G = min(G, 64 // queries)         # Q * G query rows per KV head, at most 64
    else:
        part = rng.choice([0, 0, 0, 32, 64, 96, 256, 1024])
        window = rng.choice([0, 0, rng.randint(1, 600)])
    spec = W.Spec(f"random{seed}", B=B, N=G * K, K=K, H=Hd, bs=bs, ctx=ctx,
                  max_blocks=(max(ctx) + bs - 1) // bs + 3, seed=seed, kv_dtype=kv,
                  queries=queries)
    return spec, part, window


def describe(spec, part, window):
    return (f"B={spec.B} N={spec.N} K={spec.K} H={spec.H} bs={spec.bs} {spec.kv_dtype} "
            f"Q={spec.queries} "
            f"partition={part} window={window} ctx={list(spec.ctx)[:10]}")


def single_query(seed, bs):
    spec, part, window = draw(seed, bs=bs)
    what = f"random {seed}: {describe(spec, part, window)}"
    H.log(f"case {what}")
    w = W.make(spec)
    ref, inp = H.oracle_step(w)
    if window:
        ref = H.oracle_decode_window(w, inp, window)
    g = w.to(DEV)
    H.gpu_append(g, w)
    out = torch.full(g.q.shape, float("nan"), dtype=torch.float32, device=DEV)
    if window:
        H.gpu_decode_window(out, g, w, window, partition=part)
    else:
        H.gpu_decode(out, g, w, partition=part)
    torch.cuda.synchronize()
    H.assert_append_exact(g, inp, what)
    H.assert_parity(out.cpu().numpy(), ref, what)


def multi_query(seed, bs):
    Q = random.Random(seed).randint(2, 6)
    spec, part, _ = draw(seed, queries=Q, bs=bs)
    what = f"random mq {seed}: {describe(spec, part, 0)}"
    H.log(f"case {what}")
    w = W.make(spec)
    ref, inp = H.oracle_step_mq(w)
    out, g = H.gpu_step_mq(w, part)
    H.assert_append_exact(g, inp, what)
    H.assert_parity(out.numpy(), ref, what)


@pytest.mark.parametrize("seed", range(7000, 7200))
def test_single_query(seed):
    single_query(seed, 16)


@pytest.mark.parametrize("seed", range(7300, 7360))
def test_multi_query(seed):
    multi_query(seed, 16)


@pytest.mark.parametrize("seed", range(7400, 7480))
def test_single_query_blocks_of_32(seed):
    single_query(seed, 32)


@pytest.mark.parametrize("seed", range(7500, 7530))
def test_multi_query_blocks_of_32(seed):
    multi_query(seed, 32)
