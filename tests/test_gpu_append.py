"""GPU parity of the slot-mapped append on its own ("Week 11. Inference",
step 2: the new token's key and value are written to the cache; the lesson's
Build-It step 1 writes them at the next position, here its slot).

The kernels run one wave per (token, KV head); these cases check them against
the oracle's append on whole pools that start out random (so a stray write
anywhere shows): both head dims, one to forty KV heads, token-head counts
that leave the last four-wave workgroup partly empty, a batch of the 13B
B 256 shape, negative slots (padding: skipped), slots at and past the end of
the pools (skipped by the library; the oracle rejects them, so it is given
the other tokens only), and FP8 pools at several scales.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_100_amd as pkv
import oracle

import gpu_harness as H
from _util import bits, pool_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def random_pools(nb, K, Hd, gen, fp8):
    if fp8:
        kc = torch.randint(0, 256, (nb, K, 16, Hd), dtype=torch.uint8, generator=gen)
        vc = torch.randint(0, 256, (nb, K, Hd, 16), dtype=torch.uint8, generator=gen)
    else:
        kc = torch.randint(-32768, 32768, (nb, K, 16, Hd), dtype=torch.int32,
                           generator=gen).to(torch.int16).view(torch.bfloat16)
        vc = torch.randint(-32768, 32768, (nb, K, Hd, 16), dtype=torch.int32,
                           generator=gen).to(torch.int16).view(torch.bfloat16)
    return kc, vc


def run(T, K, Hd, nb, seed, fp8=False, scales=(1.0, 1.0), special=()):
    """T tokens at distinct random slots (``special`` overrides some: index,
    slot), appended on the GPU and by the oracle; the pools must match."""
    gen = torch.Generator().manual_seed(seed)
    k = torch.randn((T, K, Hd), generator=gen).to(torch.bfloat16)
    v = torch.randn((T, K, Hd), generator=gen).to(torch.bfloat16)
    slots = torch.randperm(nb * 16, generator=gen)[:T].to(torch.int64)
    for i, s in special:
        slots[i] = s
    kc, vc = random_pools(nb, K, Hd, gen, fp8)
    H.log(f"case append T={T} K={K} H={Hd} nb={nb} fp8={fp8} special={list(special)}")
    kc_ref, vc_ref = pool_bits(kc).copy(), pool_bits(vc).copy()
    inside = (slots < nb * 16).numpy()
    ks, vs = bits(k)[inside], bits(v)[inside]
    sl = slots.numpy()[inside]
    if fp8:
        oracle.append_fp8(ks, vs, sl, kc_ref, vc_ref, *scales)
    else:
        oracle.append(ks, vs, sl, kc_ref, vc_ref)
    gk, gv, gs = k.to(DEV), v.to(DEV), slots.to(DEV)
    gkc, gvc = kc.to(DEV), vc.to(DEV)
    if fp8:
        pkv.paged_kv_append_fp8(gk, gv, gs, gkc, gvc, *scales)
    else:
        pkv.paged_kv_append(gk, gv, gs, gkc, gvc)
    torch.cuda.synchronize()
    assert np.array_equal(pool_bits(gkc), kc_ref), "key pool differs from the oracle's append"
    assert np.array_equal(pool_bits(gvc), vc_ref), "value pool differs from the oracle's append"


@pytest.mark.parametrize("Hd", [64, 128])
@pytest.mark.parametrize("T,K", [(1, 1), (3, 1), (5, 3), (64, 8), (100, 8), (7, 40)])
def test_shapes(T, K, Hd):
    run(T, K, Hd, nb=max(8, T), seed=500 + T * 7 + K)


def test_thirteen_b_batch_shape():
    # 256 tokens x 40 KV heads (10,240 token heads, 2,560 workgroups)
    run(256, 40, 128, nb=300, seed=517)


@pytest.mark.parametrize("Hd", [64, 128])
def test_negative_and_out_of_pool_slots(Hd):
    nb = 6
    run(9, 2, Hd, nb, seed=523, special=[(0, -1), (3, -7), (4, nb * 16), (6, nb * 16 + 5),
                                         (8, 1 << 40)])


@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.0123, 3.0e-3), (7.5, 0.02)])
@pytest.mark.parametrize("Hd", [64, 128])
def test_fp8_pools(Hd, scales):
    nb = 10
    run(37, 5, Hd, nb, seed=541, fp8=True, scales=scales,
        special=[(2, -1), (5, nb * 16)])
