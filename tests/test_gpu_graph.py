"""GPU: every call captured into a HIP graph and replayed.

A serving loop captures its decode step once and replays it, changing only
the contents of its buffers (new queries, longer contexts).  Each case here
captures one step (the append, then a decode call) through the C ABI,
replays it several times with different queries and context lengths written
into the same buffers between the replays (eager work and a device
synchronisation in between), and checks every replay bit for bit against
the same step run eagerly on the same inputs: the token-balanced and fixed
partition decodes, FP8 pools, the sliding window, the multi-query kernel
(its merge launch, and the two-partition case whose in-kernel pair merge
needs a new tag per call, so a captured call takes the merge launch), the
shared-prefix read and the allocation-free call.  The first replay is also
checked against the fp64 oracle.
"""
import dataclasses

import pytest
import torch

import paged_kv_cache_100_amd as pkv
from paged_kv_cache_100_amd import workloads as W

import gpu_harness as H

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make_step(kind, w, g, out):
    s = w.spec
    mcl = w.max_context_len
    fp8 = w.kv_dtype == "fp8"

    def append():
        if fp8:
            pkv.paged_kv_append_fp8(g.k_new, g.v_new, g.slot_mapping, g.key_cache,
                                    g.value_cache, w.k_scale, w.v_scale)
        else:
            pkv.paged_kv_append(g.k_new, g.v_new, g.slot_mapping, g.key_cache, g.value_cache)

    if kind in ("balanced", "fixed64", "noalloc"):
        part = 64 if kind == "fixed64" else 0
        ws = torch.empty(max(pkv.workspace_size(s.B, s.N, s.K, s.H, mcl, part), 16),
                         dtype=torch.uint8, device=DEV)

        def decode():
            if kind == "noalloc":
                pkv.paged_decode_attention_noalloc(out, g.q, g.key_cache, g.value_cache,
                                                   g.block_tables, g.context_lens, w.scale, s.K,
                                                   s.bs, max_context_len=mcl, partition=part)
            elif fp8:
                pkv.paged_decode_attention_fp8(out, g.q, g.key_cache, g.value_cache,
                                               g.block_tables, g.context_lens, w.scale,
                                               w.k_scale, w.v_scale, s.K, s.bs,
                                               max_context_len=mcl, partition=part, workspace=ws)
            else:
                pkv.paged_decode_attention(out, g.q, g.key_cache, g.value_cache, g.block_tables,
                                           g.context_lens, w.scale, s.K, s.bs,
                                           max_context_len=mcl, partition=part, workspace=ws)
    elif kind == "window":
        ws = torch.empty(max(pkv.workspace_size(s.B, s.N, s.K, s.H, mcl, 0), 16),
                         dtype=torch.uint8, device=DEV)

        def decode():
            pkv.paged_decode_attention_window(out, g.q, g.key_cache, g.value_cache,
                                              g.block_tables, g.context_lens, w.scale, s.K, s.bs,
                                              300, k_scale=w.k_scale, v_scale=w.v_scale,
                                              max_context_len=mcl, workspace=ws)
    elif kind.startswith("mq"):
        part = int(kind[len("mq"):])
        ws = torch.empty(max(pkv.mq_workspace_size(s.B, s.queries, s.N, s.H, mcl, part), 16),
                         dtype=torch.uint8, device=DEV)

        def decode():
            pkv.paged_decode_attention_mq(out, g.q, g.key_cache, g.value_cache, g.block_tables,
                                          g.context_lens, w.scale, s.K, s.bs, part,
                                          k_scale=w.k_scale, v_scale=w.v_scale,
                                          max_context_len=mcl, workspace=ws)
    elif kind == "prefix":
        B = s.B
        seq_group = torch.full((B,), -1, dtype=torch.int32)
        seq_group[w.sharer_ids] = 0
        sg = seq_group.to(DEV)
        gm = torch.tensor([w.sharer_ids], dtype=torch.int32, device=DEV)
        pt = torch.tensor([len(w.shared_blocks) * s.bs], dtype=torch.int32, device=DEV)
        mpt = len(w.shared_blocks) * s.bs
        ws = torch.empty(max(pkv.prefix_workspace_size(B, s.N, s.K, s.H, mcl, 96, mpt), 16),
                         dtype=torch.uint8, device=DEV)

        def decode():
            pkv.paged_decode_attention_prefix(out, g.q, g.key_cache, g.value_cache,
                                              g.block_tables, g.context_lens, w.scale, s.K, s.bs,
                                              96, sg, gm, pt, max_prefix_tokens=mpt,
                                              k_scale=w.k_scale, v_scale=w.v_scale,
                                              max_context_len=mcl, workspace=ws)
    else:
        raise ValueError(kind)

    def step():
        append()
        decode()
    return step


def spec_for(kind, kv):
    if kind == "prefix":
        return dataclasses.replace(W.small("llama3_70b_ragged_b100"), kv_dtype=kv)
    if kind.startswith("mq"):
        # 3 queries x 4 heads per KV head: one tile; 1,024-token contexts span
        # two 512-token partitions (the pair merge) or sixteen 64-token ones
        return W.Spec("graph mq", B=5, N=16, K=4, H=128, ctx=[1024, 700, 3, 513, 64], seed=83,
                      kv_dtype=kv, queries=3)
    return W.Spec("graph", B=7, N=32, K=8, H=128, ctx=[1024, 1, 300, 513, 47, 0, 800], seed=81,
                  kv_dtype=kv, max_blocks=70)


CASES = [("balanced", "bf16"), ("fixed64", "bf16"), ("balanced", "fp8"), ("window", "bf16"),
         ("mq512", "bf16"), ("mq64", "bf16"), ("mq512", "fp8"), ("prefix", "bf16"),
         ("noalloc", "bf16")]


@pytest.mark.parametrize("kind,kv", CASES, ids=[f"{k}-{v}" for k, v in CASES])
def test_replays_match_eager_calls(kind, kv):
    sp = spec_for(kind, kv)
    w = W.make(sp)
    what = f"graph {kind} {kv}"
    H.log(f"case {what}: B={sp.B} N={sp.N} K={sp.K} Q={sp.queries} ctx={w.context_lens.tolist()}")
    ref0 = H.oracle_step_mq(w)[0] if sp.queries > 1 else None
    if ref0 is None and kind == "window":
        ref0, inp = H.oracle_step(w)
        ref0 = H.oracle_decode_window(w, inp, 300)
    elif ref0 is None:
        ref0 = H.oracle_step(w)[0]
    g = w.to(DEV)
    out = torch.full(g.q.shape, float("nan"), dtype=torch.float32, device=DEV)
    step = make_step(kind, w, g, out)

    # warm up on a side stream, then capture one step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(sp.seed + 1)
    ctx0 = g.context_lens.clone()
    q0 = g.q.clone()
    for r in range(4):
        if r > 0:      # new queries; some contexts shorter (never past the captured bound)
            g.q.copy_(torch.randn(q0.shape, generator=gen).to(torch.bfloat16))
            cut = torch.randint(0, 40, ctx0.shape, generator=gen, dtype=torch.int32).to(DEV)
            g.context_lens.copy_(torch.clamp(ctx0 - cut * (r % 2), min=0))
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        eager = out.clone()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"{what}: replay {r} differs from the eager step"
        if r == 0:
            H.assert_parity(out.cpu().numpy(), ref0, what)
    g.q.copy_(q0)
    g.context_lens.copy_(ctx0)
