"""GPU parity of the FP8 KV pools (OCP E4M3 codes, one scale per pool).

* The append is bit exact against the oracle's quantisation for every one of
  the 65536 bf16 bit patterns (NaN, infinities, zeros of both signs,
  subnormals, values past the clamp, ties), at several pool scales.
* Decode matches the fp64 oracle on poisoned small workloads (several
  chunks, partitions and ragged tails), context edges, every group size,
  a sharp softmax, and pools holding every finite code.
* With unit scales, the FP8 decode agrees with the bf16 decode over the same
  values widened to bf16 up to fp32 summation order (the two formats assign
  head dims to matrix-core k-steps differently); the widening itself is exact.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_100_amd as pkv
from paged_kv_cache_100_amd import workloads as W

import gpu_harness as H
from _util import bits, pool_bits

pytestmark = pytest.mark.gpu


def fp8(spec, **kw):
    return dataclasses.replace(spec, kv_dtype="fp8", **kw)


def run_case(w, partition=0, what=""):
    H.log(f"case {what}: B={w.spec.B} N={w.spec.N} K={w.spec.K} H={w.spec.H} "
          f"partition={partition} k_scale={w.k_scale:.6g} v_scale={w.v_scale:.6g} "
          f"ctx={w.context_lens.tolist()[:12]}")
    ref, inp = H.oracle_step(w)
    out, g = H.gpu_step(w, partition=partition)
    H.assert_append_exact(g, inp, what)
    H.assert_parity(out.numpy(), ref, what)
    return out, ref


def all_bf16_patterns(T, K, Hd, roll=0):
    pats = np.roll(np.arange(65536, dtype=np.uint16), roll).view(np.int16)
    return torch.from_numpy(pats.copy()).view(torch.bfloat16).reshape(T, K, Hd)


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.0123, 3.0e-3), (7.5, 0.02),
                                             (2.0 ** -20, 1.0e5)])
def test_append_every_bf16_pattern(k_scale, v_scale):
    T, K, Hd = 16, 32, 128                       # 65536 values per pool
    k = all_bf16_patterns(T, K, Hd)
    v = all_bf16_patterns(T, K, Hd, roll=12345)
    slots = torch.tensor([16 * j + (5 * j) % 16 for j in range(T)] , dtype=torch.int64)
    nb = T + 1                                   # the last block is never written
    kc = torch.full((nb, K, 16, Hd), 0x5A, dtype=torch.uint8)
    vc = torch.full((nb, K, Hd, 16), 0xA5, dtype=torch.uint8)
    H.log(f"case append all bf16 patterns: k_scale={k_scale} v_scale={v_scale}")
    kc_ref, vc_ref = kc.numpy().copy(), vc.numpy().copy()
    oracle.append_fp8(bits(k), bits(v), slots.numpy(), kc_ref, vc_ref, k_scale, v_scale)
    kg, vg = kc.cuda(), vc.cuda()
    pkv.paged_kv_append_fp8(k.cuda(), v.cuda(), slots.cuda(), kg, vg, k_scale, v_scale)
    torch.cuda.synchronize()
    assert np.array_equal(pool_bits(kg), kc_ref), "key codes differ"
    assert np.array_equal(pool_bits(vg), vc_ref), "value codes differ"


def test_append_accepts_float8_pools():
    w = W.make(W.small("tiny_fp8"))
    g = w.to("cuda:0")
    kf = g.key_cache.view(torch.float8_e4m3fn)
    vf = g.value_cache.view(torch.float8_e4m3fn)
    pkv.paged_kv_append_fp8(g.k_new, g.v_new, g.slot_mapping, kf, vf, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    inp = {"key_cache": pool_bits(w.key_cache), "value_cache": pool_bits(w.value_cache)}
    H.oracle_append(w, inp)
    assert np.array_equal(pool_bits(kf), inp["key_cache"])
    assert np.array_equal(pool_bits(vf), inp["value_cache"])


@pytest.mark.parametrize("name", ["tiny_fp8", "llama3_8b_b64_ctx8k_fp8",
                                  "llama3_70b_ragged_b100_fp8"])
@pytest.mark.parametrize("partition", [0, 64])
def test_small_variants(name, partition):
    w = W.make(W.small(name))
    run_case(w, partition=partition, what=f"{name} small part {partition}")


EDGE_CTX = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1024]


@pytest.mark.parametrize("partition", [0, 32, 512])
@pytest.mark.parametrize("shape", [(8, 2, 64), (32, 8, 128)], ids=["g4h64", "g4h128"])
def test_context_edges(shape, partition):
    N, K, Hd = shape
    spec = fp8(W.Spec("edges", B=len(EDGE_CTX), N=N, K=K, H=Hd, ctx=list(EDGE_CTX),
                      max_blocks=70, seed=7))
    run_case(W.make(spec), partition=partition, what=f"fp8 edges {shape} part {partition}")


@pytest.mark.parametrize("N,K", [(16, 16), (16, 4), (16, 1), (24, 2)],
                         ids=["mha", "g4", "mqa_g16", "g12"])
@pytest.mark.parametrize("Hd", [64, 128])
def test_group_sizes(N, K, Hd):
    spec = fp8(W.Spec("groups", B=3, N=N, K=K, H=Hd, ctx=[300, 47, 129], seed=11))
    run_case(W.make(spec), what=f"fp8 N={N} K={K} H={Hd}")


def test_sharp_softmax():
    spec = fp8(W.Spec("sharp", B=4, N=16, K=2, H=128, ctx=[5, 100, 700, 2000], key_scale=8.0,
                      seed=13))
    run_case(W.make(spec), what="fp8 keys x8")


def random_finite_codes(shape, gen):
    """Uniform over the 254 finite E4M3 codes (every code but 0x7F and 0xFF)."""
    c = torch.randint(0, 254, shape, generator=gen, dtype=torch.int32)
    c = c + (c >= 0x7F).to(torch.int32)
    return c.to(torch.uint8)


@pytest.mark.parametrize("partition", [0, 128])
@pytest.mark.parametrize("Hd", [64, 128])
def test_every_finite_code(Hd, partition):
    spec = fp8(W.Spec("codes", B=4, N=16, K=4, H=Hd, ctx=[300, 1, 77, 1024], seed=43))
    w = W.make(spec, poison=False)
    gen = torch.Generator().manual_seed(44)
    w.key_cache = random_finite_codes(tuple(w.key_cache.shape), gen)
    w.value_cache = random_finite_codes(tuple(w.value_cache.shape), gen)
    w.k_scale = float(np.float32(1.5 / 448.0))
    w.v_scale = float(np.float32(1.0 / 448.0))
    run_case(w, partition=partition, what=f"fp8 every code H={Hd} part {partition}")


@pytest.mark.parametrize("partition", [0, 32, 1024])
def test_unit_scale_fp8_matches_widened_bf16(partition):
    spec = fp8(W.Spec("widen", B=5, N=32, K=8, H=128, ctx=[1000, 37, 1024, 513, 64], seed=47))
    w = W.make(spec, poison=False)
    gen = torch.Generator().manual_seed(48)
    w.key_cache = random_finite_codes(tuple(w.key_cache.shape), gen)
    w.value_cache = random_finite_codes(tuple(w.value_cache.shape), gen)
    w.k_scale = w.v_scale = 1.0
    scale = float(np.float32(1.0 / 4096.0))      # keeps scores of codes up to 448 moderate
    w.scale = scale
    g = w.to("cuda:0")
    out8 = torch.empty(g.q.shape, dtype=torch.float32, device="cuda:0")
    H.gpu_decode(out8, g, w, partition=partition)
    wb = dataclasses.replace(w, kv_dtype="bf16", spec=dataclasses.replace(w.spec, kv_dtype="bf16"))
    wb.key_cache = w.key_cache.view(torch.float8_e4m3fn).to(torch.bfloat16)
    wb.value_cache = w.value_cache.view(torch.float8_e4m3fn).to(torch.bfloat16)
    gb = wb.to("cuda:0")
    out16 = torch.empty_like(out8)
    H.gpu_decode(out16, gb, wb, partition=partition)
    torch.cuda.synchronize()
    abs_err, rel, zero_ok = H.errors(out8.cpu().numpy(), out16.cpu().numpy())
    H.log(f"case widen part {partition}: max abs {abs_err:.3e}, row rel {rel:.3e}")
    assert torch.isfinite(out8).all()
    assert rel < 1e-5 and zero_ok


def test_rejects_bad_scales():
    w = W.make(W.small("tiny_fp8"))
    g = w.to("cuda:0")
    out = torch.empty(g.q.shape, dtype=torch.float32, device="cuda:0")
    for ks, vs in [(0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (1.0, float("nan")),
                   (1e-45, 1.0)]:
        with pytest.raises(pkv.PagedKVError):
            pkv.paged_kv_append_fp8(g.k_new, g.v_new, g.slot_mapping, g.key_cache,
                                    g.value_cache, ks, vs)
        with pytest.raises(pkv.PagedKVError):
            pkv.paged_decode_attention_fp8(out, g.q, g.key_cache, g.value_cache,
                                           g.block_tables, g.context_lens, w.scale, ks, vs,
                                           w.spec.K, w.spec.bs)
