"""Full-size workloads, in the launch configuration the benchmark times
(library-chosen partitions; 512-token partitions for the 128K-context case).

The append is checked bit for bit on the whole pools.  Attention is checked
on every output row (every sequence, query token and head) against the fp64
oracle run over the whole batch, plus the property that every output is
finite (the block tails are NaN-poisoned).  Each case logs its maximum
absolute and row-relative errors."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_100_amd import workloads as W

import gpu_harness as H
from _util import oracle_inputs, pool_bits

pytestmark = pytest.mark.gpu

FULL = ["llama3_8b_b64_ctx8k", "llama2_13b_b1_ctx1k", "llama2_13b_b64_ctx1k",
        "llama2_13b_b256_ctx1k", "llama3_70b_ragged_b100", "llama3_70b_long_b4_ctx128k",
        "llama3_8b_b64_ctx8k_fp8", "llama3_70b_ragged_b100_fp8",
        "llama3_8b_b64_ctx8k_spec4", "llama3_70b_b64_ctx4k_spec6"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    H.log(f"case {name} (full size)")
    with H.Timer("generate"):
        w = W.make(name)
    multi = w.spec.queries > 1
    with H.Timer("gpu step"):
        if multi:
            out, g = H.gpu_step_mq(w, partition=w.spec.partition_size)
        else:
            out, g = H.gpu_step(w, partition=w.spec.partition_size)
    assert torch.isfinite(out).all(), "non-finite output"
    with H.Timer("oracle append + compare pools"):
        inp = oracle_inputs(w)
        H.oracle_append(w, inp)
        assert np.array_equal(pool_bits(g.key_cache), inp["key_cache"]), \
            "key cache differs after append"
        assert np.array_equal(pool_bits(g.value_cache), inp["value_cache"]), \
            "value cache differs after append"
        del g
        torch.cuda.empty_cache()
    with H.Timer("oracle, every row"):
        if multi:
            ref = oracle.decode_multi(inp["q"], inp["key_cache"], inp["value_cache"],
                                      inp["block_tables"], inp["context_lens"], w.scale,
                                      w.k_scale, w.v_scale)
        else:
            ref = H.oracle_decode(w, inp)
    H.assert_parity(out.numpy(), ref, f"{name} every row")


@pytest.mark.parametrize("piece", [128, 256])
@pytest.mark.parametrize("name", ["llama3_70b_ragged_b100", "llama3_70b_ragged_b100_fp8"])
def test_full_size_shared_prefix(name, piece):
    """The ragged mix through the shared-prefix call as the benchmark's
    prefix mode runs it (its 20 sharers' 62 shared blocks read once, in
    128-token pieces; also 256): every row against the oracle and against
    plain decode of the same pools."""
    import paged_kv_cache_100_amd as pkv
    H.log(f"case {name} shared prefix (full size), {piece}-token pieces")
    with H.Timer("generate"):
        w = W.make(name)
    s = w.spec
    dev = "cuda:0"
    out, g = H.gpu_step(w)           # append, then plain decode
    shared = len(w.shared_blocks) * s.bs
    seq_group = torch.full((s.B,), -1, dtype=torch.int32)
    seq_group[w.sharer_ids] = 0
    members = torch.tensor([w.sharer_ids], dtype=torch.int32)
    tokens = torch.tensor([shared], dtype=torch.int32)
    got = torch.full((s.B, s.N, s.H), float("nan"), dtype=torch.float32, device=dev)
    with H.Timer("gpu prefix decode"):
        pkv.paged_decode_attention_prefix(got, g.q, g.key_cache, g.value_cache, g.block_tables,
                                          g.context_lens, w.scale, s.K, s.bs, piece,
                                          seq_group.to(dev), members.to(dev), tokens.to(dev),
                                          max_prefix_tokens=shared, k_scale=w.k_scale,
                                          v_scale=w.v_scale, max_context_len=w.max_context_len)
        torch.cuda.synchronize()
    got = got.cpu()
    assert torch.isfinite(got).all(), "non-finite output"
    H.assert_parity(got.numpy(), out.numpy().astype(np.float64), f"{name} prefix vs plain")
    inp = oracle_inputs(w)
    H.oracle_append(w, inp)
    del g
    torch.cuda.empty_cache()
    with H.Timer("oracle, every row"):
        ref = H.oracle_decode(w, inp)
    H.assert_parity(got.numpy(), ref, f"{name} prefix every row")


def test_full_size_window():
    """Llama-3-8B, B 64 x 8k, with a 4,096-token sliding window, as the
    benchmark's `--window 4096` runs it (token-balanced schedule): every row
    against the oracle's windowed decode."""
    name, window = "llama3_8b_b64_ctx8k", 4096
    H.log(f"case {name} window {window} (full size)")
    with H.Timer("generate"):
        w = W.make(name)
    g = w.to("cuda:0")
    H.gpu_append(g, w)
    out = torch.full(g.q.shape, float("nan"), dtype=torch.float32, device="cuda:0")
    with H.Timer("gpu window decode"):
        H.gpu_decode_window(out, g, w, window, partition=0)
        torch.cuda.synchronize()
    got = out.cpu().numpy()
    del g
    torch.cuda.empty_cache()
    inp = oracle_inputs(w)
    H.oracle_append(w, inp)
    with H.Timer("oracle windowed decode, all rows"):
        ref = H.oracle_decode_window(w, inp, window)
    H.assert_parity(got, ref, f"{name} window {window}")
