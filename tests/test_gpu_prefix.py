"""GPU: shared-prefix-aware decode and the copy-on-write block copy.

``paged_decode_attention_prefix`` reads each shared prefix once for all of
its sharers (a group kernel over the shared span, in partition-sized pieces)
and the rest of every context on the token-balanced schedule, then merges
both.  What it computes is plain attention, so it is checked against the
oracle's decode (``oracle.decode``) and, to the same tolerance, against plain
``paged_decode_attention``: one group (the reduced ragged workload), several
groups built by re-pointing block tables, more sharers than one wave carries,
every tiles-per-wave choice of the group kernel, members shorter than the
shared span, spans that end inside a partition, sequences wholly inside
their shared span or with one chunk of their own, partition sizes, FP8
pools.  A member whose table disagrees with the lead's over its shared span
must get attention over the lead's blocks there: that pins that the shared
positions really come from the group kernel.

``paged_kv_copy_blocks`` is bit-exact against ``oracle.copy_blocks`` for
bf16 and FP8 pools, and a copy-on-write divergence (copy a shared block,
re-point one sharer, append into the copy) leaves the other sharers' results
unchanged and matches the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_100_amd as pkv
from paged_kv_cache_100_amd import workloads as W

import gpu_harness as H
from _util import bits, oracle_inputs, pool_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def groups_from(B, groups):
    """groups: list of (members, prefix_tokens) -> device arrays."""
    seq_group = torch.full((B,), -1, dtype=torch.int32)
    width = max(len(m) for m, _ in groups)
    members = torch.full((len(groups), width), -1, dtype=torch.int32)
    tokens = torch.zeros(len(groups), dtype=torch.int32)
    for g, (mem, t) in enumerate(groups):
        members[g, :len(mem)] = torch.tensor(mem, dtype=torch.int32)
        tokens[g] = t
        for b in mem:
            seq_group[b] = g
    return seq_group.to(DEV), members.to(DEV), tokens.to(DEV)


def prefix_decode(g, w, groups, partition):
    sg, gm, pt = groups_from(w.spec.B, groups)
    out = torch.full(g.q.shape, float("nan"), dtype=torch.float32, device=DEV)
    pkv.paged_decode_attention_prefix(out, g.q, g.key_cache, g.value_cache, g.block_tables,
                                      g.context_lens, w.scale, w.spec.K, w.spec.bs, partition,
                                      sg, gm, pt, max_prefix_tokens=int(pt.max()),
                                      k_scale=w.k_scale, v_scale=w.v_scale,
                                      max_context_len=w.max_context_len)
    return out


def run_prefix(w, groups, partition, what, ref_tables=None):
    """Append, then prefix-aware and plain decode on the same pools; compare
    with the oracle (over ``ref_tables`` when given) and with each other."""
    H.log(f"case {what}: B={w.spec.B} N={w.spec.N} K={w.spec.K} {w.kv_dtype} part {partition} "
          f"groups={[(len(m), t) for m, t in groups]}")
    inp = oracle_inputs(w)
    H.oracle_append(w, inp)
    if ref_tables is not None:
        inp["block_tables"] = ref_tables
    ref = H.oracle_decode(w, inp)
    g = w.to(DEV)
    H.gpu_append(g, w)
    out = prefix_decode(g, w, groups, partition)
    plain = torch.full_like(out, float("nan"))
    H.gpu_decode(plain, g, w, partition=0)
    torch.cuda.synchronize()
    H.assert_append_exact(g, inp, what)
    H.assert_parity(out.cpu().numpy(), ref, what)
    if ref_tables is None:
        H.assert_parity(out.cpu().numpy(), plain.cpu().numpy().astype(np.float64),
                        what + " vs plain decode")
    return out


def workload_groups(w):
    return [(w.sharer_ids, len(w.shared_blocks) * w.spec.bs)]


@pytest.mark.parametrize("partition", [32, 96, 256, 1024])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_ragged_small(kv, partition):
    spec = dataclasses.replace(W.small("llama3_70b_ragged_b100"), kv_dtype=kv)
    w = W.make(spec)
    run_prefix(w, workload_groups(w), partition, f"ragged small {kv}")


def repoint(w, groups_spec):
    """Make each group's members share the lead's first n blocks (tables only)."""
    groups = []
    for lead, others, nblk in groups_spec:
        for b in others:
            w.block_tables[b, :nblk] = w.block_tables[lead, :nblk]
        groups.append(([lead] + others, nblk * w.spec.bs))
    return groups


@pytest.mark.parametrize("partition", [32, 96])
def test_several_groups(partition):
    spec = W.Spec("groups", B=9, N=32, K=8, H=128, ctx=[700, 400, 650, 90, 333, 800, 41, 512, 200],
                  seed=61, max_blocks=60)
    w = W.make(spec)
    # group 0: 0, 2, 5 and 3 share 20 blocks (3 has only 90 tokens, fewer than
    # the shared span); group 1: 1, 7 share 8; group 2: 4 alone
    groups = repoint(w, [(0, [2, 5, 3], 20), (1, [7], 8), (4, [], 10)])
    run_prefix(w, groups, partition, f"three groups part {partition}")


@pytest.mark.parametrize("sharers", [5, 8, 12])
def test_many_sharers(sharers):
    # sharers x G = 8 (sharer, head) pairs: 40 -> three tiles in one wave,
    # 64 -> four, 96 -> two waves (four tiles, then two live of four)
    spec = W.Spec("many", B=14, N=64, K=8, H=128, ctx=[600 + 17 * i for i in range(14)],
                  seed=67, max_blocks=60)
    w = W.make(spec)
    others = [i for i in range(14) if i != 3][:sharers - 1]
    groups = repoint(w, [(3, others, 30)])
    run_prefix(w, groups, 64, f"{sharers} sharers")


@pytest.mark.parametrize("partition", [32, 96])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_sharers_wholly_shared(kv, partition):
    # sequences 1 and 2 (64 tokens) lie wholly in their shared span: no chunk
    # of their own is left for the per-sequence waves (rows made of prefix
    # partials alone); 5 (96 tokens) has one chunk of its own
    spec = W.Spec("whole", B=6, N=32, K=8, H=128, ctx=[700, 64, 64, 300, 33, 96], seed=97,
                  kv_dtype=kv)
    w = W.make(spec)
    groups = repoint(w, [(0, [1, 2, 5], 10)])
    run_prefix(w, groups, partition, f"wholly shared {kv} part {partition}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_members_read_the_leads_blocks(kv):
    """Members whose own tables point elsewhere over the shared span get
    attention over the lead's blocks there (and their own blocks after it):
    the shared positions come from the group kernel, not from each member's
    table."""
    spec = W.Spec("lead", B=5, N=32, K=8, H=128, ctx=[500, 430, 300, 70, 520], seed=103,
                  kv_dtype=kv, max_blocks=40)
    w = W.make(spec)
    members, tokens = [0, 1, 2, 3], 200
    tables = w.block_tables.numpy().astype(np.int32).copy()
    ctx = w.context_lens.numpy()
    for b in members[1:]:
        span = min(tokens, ctx[b], ctx[0]) // 32 * 32
        tables[b, :span // 16] = tables[0, :span // 16]
    run_prefix(w, [(members, tokens)], 64, f"lead's blocks {kv}", ref_tables=tables)


@pytest.mark.parametrize("partition", [32, 64, 160, 1024])
def test_span_ends_inside_a_partition(partition):
    # spans of 1000 positions (992 shared: whole chunks) and of members
    # shorter than that: 300 (-> 288), 150 (-> 128), 40 (-> 32), 20 (-> 0);
    # the group kernel masks each member's columns past its own span
    spec = W.Spec("spans", B=7, N=16, K=4, H=128, ctx=[1300, 1100, 300, 150, 40, 20, 1000],
                  seed=107, max_blocks=90)
    w = W.make(spec)
    groups = repoint(w, [(0, [1, 2, 3, 4, 5, 6], 63)])
    groups = [(groups[0][0], 1000)]
    run_prefix(w, groups, partition, f"spans, part {partition}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_nothing_shared_below_one_chunk(kv):
    # every group's prefix under one 32-token chunk: no span, no group waves,
    # and the result is plain decode's
    spec = W.Spec("nochunk", B=6, N=32, K=8, H=128, ctx=[300, 200, 90, 45, 33, 120], seed=163,
                  kv_dtype=kv)
    w = W.make(spec)
    groups = repoint(w, [(0, [1, 2, 3], 2), (4, [5], 2)])   # 32 positions mapped alike
    groups = [(groups[0][0], 20), (groups[1][0], 31)]
    run_prefix(w, groups, 64, f"prefixes under a chunk {kv}")


def test_group_with_an_empty_span_beside_a_shared_one():
    # group 0's lead holds 20 tokens, so its span is empty and its waves find
    # nothing to read; group 1 shares 160 positions
    spec = W.Spec("emptyspan", B=6, N=32, K=8, H=128, ctx=[20, 300, 45, 500, 400, 161], seed=167)
    w = W.make(spec)
    groups = repoint(w, [(0, [1, 2], 1), (3, [4, 5], 10)])
    run_prefix(w, groups, 64, "empty span beside a shared one")


def test_large_batch():
    # more than 256 sequences: the schedule kernel's table, with shared
    # partitions skipped
    gen = np.random.default_rng(101)
    ctx = [int(c) for c in gen.integers(1, 600, size=300)]
    ctx[:40] = [400 + i for i in range(40)]
    spec = W.Spec("b300", B=300, N=16, K=4, H=64, ctx=ctx, seed=101)
    w = W.make(spec)
    groups = repoint(w, [(0, list(range(1, 30)), 20), (30, list(range(31, 40)), 12)])
    run_prefix(w, groups, 64, "B=300 two groups")


def tiles_per_wave(items, tiles):
    """The library's choice for the group kernel: the fewest tiles per wave
    whose waves fit one per SIMD (1024 on the chip), at most four."""
    for pw in range(1, min(4, tiles)):
        if items * -(-tiles // pw) <= 1024:
            return pw
    return min(4, tiles)


# (members, shared blocks): K = 8 KV heads, G = 8, partition 32, so
# items = 8 * shared blocks / 2 and tiles = members / 2
TILING = [(8, 80, 2), (12, 96, 3), (8, 130, 4)]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("members,nblk,per_wave", TILING,
                         ids=[f"{pw}tiles" for _, _, pw in TILING])
def test_tiles_per_wave(members, nblk, per_wave, kv):
    items = 8 * (nblk * 16 // 32)
    assert tiles_per_wave(items, -(-members * 8 // 16)) == per_wave
    B = members + 1
    spec = W.Spec("tiling", B=B, N=64, K=8, H=128, kv_dtype=kv,
                  ctx=[nblk * 16 + 40 + 23 * i for i in range(B)], seed=79)
    w = W.make(spec)
    groups = repoint(w, [(0, list(range(2, B)), nblk)])
    run_prefix(w, groups, 32, f"{members} sharers, {nblk} blocks, {per_wave} tiles per wave")


@pytest.mark.parametrize("Hd", [64, 128])
def test_mha_and_head_dim(Hd):
    spec = W.Spec("mha", B=6, N=16, K=16, H=Hd, ctx=[300, 260, 700, 33, 480, 300], seed=71,
                  max_blocks=50)
    w = W.make(spec)
    groups = repoint(w, [(0, [1, 4, 5], 16)])
    run_prefix(w, groups, 32, f"MHA H={Hd}")


# ------------------------------------------------------------- block copy --

@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_copy_blocks_bit_exact(kv):
    spec = W.Spec("copy", B=4, N=8, K=4, H=128, ctx=[100, 200, 50, 300], seed=73, kv_dtype=kv,
                  pool_blocks=60)
    w = W.make(spec)
    src = torch.tensor([3, 17, -1, 40, 8, 70], dtype=torch.int32)   # -1 and 70: skipped
    dst = torch.tensor([50, 51, 52, 53, 54, 55], dtype=torch.int32)
    H.log(f"case copy blocks {kv}")
    kc, vc = pool_bits(w.key_cache), pool_bits(w.value_cache)
    oracle.copy_blocks(kc, vc, src.numpy(), np.where(src.numpy() >= w.num_blocks, -1,
                                                      dst.numpy()).astype(np.int32))
    g = w.to(DEV)
    pkv.paged_kv_copy_blocks(g.key_cache, g.value_cache, src.to(DEV), dst.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(pool_bits(g.key_cache), kc)
    assert np.array_equal(pool_bits(g.value_cache), vc)


def test_copy_on_write_divergence():
    """Three sequences share a partly filled block; the third must write its
    next token there: copy the block, re-point its table, append into the
    copy.  The first two are unchanged; all three match the oracle."""
    spec = W.Spec("cow", B=3, N=32, K=8, H=128, ctx=[37, 37, 38], seed=79, pool_blocks=20,
                  max_blocks=4)
    w = W.make(spec, poison=False)
    bt = w.block_tables
    bt[1, :3] = bt[0, :3]
    bt[2, :3] = bt[0, :3]                      # all three share blocks 0..2 (block 2 holds 5 tokens)
    shared = int(bt[0, 2])
    used = set(bt[:, :3].flatten().tolist())
    fresh = next(i for i in range(w.num_blocks) if i not in used)
    g = w.to(DEV)
    out0 = torch.empty((3, spec.N, spec.H), dtype=torch.float32, device=DEV)
    before = dataclasses.replace(g, context_lens=torch.tensor([37, 37, 37], dtype=torch.int32,
                                                              device=DEV))
    # one fixed partition: each sequence's result is independent of the others'
    H.gpu_decode(out0, before, w, partition=1024, max_context_len=38)
    pkv.paged_kv_copy_blocks(g.key_cache, g.value_cache,
                             torch.tensor([shared], dtype=torch.int32, device=DEV),
                             torch.tensor([fresh], dtype=torch.int32, device=DEV))
    g.block_tables[2, 2] = fresh
    k_new = w.k_new[2:3].to(DEV)
    v_new = w.v_new[2:3].to(DEV)
    pkv.paged_kv_append(k_new, v_new, torch.tensor([fresh * 16 + 5], device=DEV),
                        g.key_cache, g.value_cache)
    out = torch.empty_like(out0)
    H.gpu_decode(out, g, w, partition=1024, max_context_len=38)
    torch.cuda.synchronize()
    assert torch.equal(out[:2], out0[:2]), "the other sharers' results changed"
    # oracle: same steps on host copies
    kc, vc = bits(w.key_cache), bits(w.value_cache)
    oracle.copy_blocks(kc, vc, np.array([shared], np.int32), np.array([fresh], np.int32))
    oracle.append(bits(w.k_new[2:3]), bits(w.v_new[2:3]),
                  np.array([fresh * 16 + 5], np.int64), kc, vc)
    tables = bt.numpy().astype(np.int32).copy()
    tables[2, 2] = fresh
    ref = oracle.decode(bits(w.q), kc, vc, tables, np.array([37, 37, 38], np.int32), w.scale)
    assert np.array_equal(pool_bits(g.key_cache), kc) and np.array_equal(pool_bits(g.value_cache), vc)
    H.assert_parity(out.cpu().numpy(), ref, "copy-on-write divergence")
