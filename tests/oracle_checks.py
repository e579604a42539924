"""Checks that pin the CPU oracle to things other than itself.

Each ``check_*`` function raises AssertionError (or ValueError from the
oracle's own argument checks) when the oracle library ``lib`` is wrong, and
returns None otherwise.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` runs them on deliberately broken copies of the
oracle's C source to show that every plausible slip fails at least one.

What each check compares against:
  * the pure-Python brute force (``oracle/brute.py``), an independent
    statement of the definition;
  * torch's CPU float64 ``scaled_dot_product_attention`` (a library routine)
    on K/V gathered into contiguous form -- the contiguous cache of the
    "Optimización de la inferencia" lesson, Build-It steps 1-2;
  * closed forms: one cached token returns its V; equal keys return the
    mean of V; shifting every key by one vector, or V by a constant, moves the
    output as the algebra says;
  * invariances of paging: relabelling physical blocks, and sharing prefix
    blocks instead of copying them, change nothing ("CS336 Lecture 10:
    Inference", part 6; PagedAttention section of the lesson);
  * GQA equals MHA with each KV head repeated N/K times ("CS336 Lecture 10:
    Inference", part 3);
  * the KV-cache sizes printed on the pages (``tests/golden``).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import brute

from _util import bits_to_f64

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "kv_cache_facts.json")
SPARE_BLOCKS = 2   # unreferenced pool blocks, so a wrong index stays inside the arrays


def to_bf16_bits(x) -> np.ndarray:
    """Round float values to bf16 (round-to-nearest-even via torch) -> bits."""
    t = torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


class Case:
    """A small paged decode problem with its tables drawn from a permutation."""

    def __init__(self, seed, B=3, N=4, K=2, H=8, bs=4, ctx=None, max_ctx=40,
                 grid=False, key_mult=1.0):
        rng = np.random.default_rng(seed)
        self.B, self.N, self.K, self.H, self.bs = B, N, K, H, bs
        self.ctx = (np.array(ctx, np.int32) if ctx is not None
                    else rng.integers(1, max_ctx + 1, B).astype(np.int32))
        nblk = [-(-int(c) // bs) for c in self.ctx]
        self.max_blocks = max([1] + nblk)
        pool = sum(nblk) + 3
        self.num_blocks = pool + SPARE_BLOCKS
        perm = rng.permutation(pool)
        self.tables = np.full((B, self.max_blocks), -1, np.int32)
        i = 0
        for b in range(B):
            for j in range(nblk[b]):
                self.tables[b, j] = perm[i]
                i += 1

        def draw(shape, mult=1.0):
            if grid:   # multiples of 1/8 in [-4, 4]: sums with small integers stay exact
                return to_bf16_bits(rng.integers(-32, 33, shape) / 8.0 * mult)
            return to_bf16_bits(rng.standard_normal(shape) * mult)

        self.q = draw((B, N, H))
        self.kc = draw((self.num_blocks, K, bs, H), key_mult)
        self.vc = draw((self.num_blocks, K, H, bs))
        self.scale = float(np.float32(1.0 / math.sqrt(H)))

    def args(self):
        return (self.q, self.kc, self.vc, self.tables, self.ctx, self.scale)

    def decode(self, lib):
        return oracle.decode(*self.args(), lib=lib)

    def brute(self, scale=None):
        q = bits_to_f64(self.q).tolist()
        kc = bits_to_f64(self.kc).tolist()
        vc = bits_to_f64(self.vc).tolist()
        return np.array(brute.paged_decode(q, kc, vc, self.tables.tolist(), self.ctx.tolist(),
                                           self.scale if scale is None else scale))

    def contiguous(self):
        """K, V gathered per sequence into [ctx, K, H] float64 arrays."""
        kf, vf = bits_to_f64(self.kc), bits_to_f64(self.vc)
        out = []
        for b in range(self.B):
            t = np.arange(self.ctx[b])
            p = self.tables[b, t // self.bs]
            o = t % self.bs
            out.append((kf[p, :, o, :], vf[p, :, :, o]))   # both [ctx, K, H]
        return out


def assert_close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- decode ----

def check_brute_force(lib):
    for seed, (N, K, bs, H) in enumerate([(4, 2, 4, 8), (4, 4, 16, 8), (6, 1, 4, 4),
                                           (8, 2, 16, 16)]):
        c = Case(seed, N=N, K=K, bs=bs, H=H, max_ctx=40)
        assert_close(c.decode(lib), c.brute(), 1e-12, f"brute force (N={N},K={K},bs={bs})")


def check_library_sdpa(lib):
    c = Case(11, B=4, N=8, K=2, H=16, bs=16, max_ctx=70)
    got = c.decode(lib)
    G = c.N // c.K
    for b, (k, v) in enumerate(c.contiguous()):
        q = torch.from_numpy(bits_to_f64(c.q[b]))[:, None, :]                   # [N, 1, H]
        kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)   # [N, ctx, H]
        vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, scale=c.scale)
        assert_close(got[b], ref[:, 0, :].numpy(), 1e-12, f"library SDPA, sequence {b}")


def check_single_token_returns_v(lib):
    c = Case(21, B=4, N=4, K=2, H=8, bs=4, ctx=[1, 1, 1, 1])
    got = c.decode(lib)
    vf = bits_to_f64(c.vc)
    for b in range(c.B):
        for n in range(c.N):
            want = vf[c.tables[b, 0], n // (c.N // c.K), :, 0]
            assert np.array_equal(got[b, n], want), "context length 1 must return V exactly"


def check_equal_keys_mean_v(lib):
    c = Case(31, B=2, N=4, K=2, H=8, bs=4, ctx=[13, 29])
    c.kc[:] = c.kc[0, 0, 0][None, None, None, :]   # every key equal
    got = c.decode(lib)
    for b, (k, v) in enumerate(c.contiguous()):
        for n in range(c.N):
            g = n // (c.N // c.K)
            assert_close(got[b, n], v[:, g, :].mean(axis=0), 1e-13, "equal keys -> mean of V")


def check_empty_context(lib):
    c = Case(41, B=3, ctx=[0, 5, 0])
    got = c.decode(lib)
    assert np.all(got[0] == 0) and np.all(got[2] == 0), "context 0 must give zeros"
    assert np.all(np.isfinite(got[1]))


def check_block_permutation(lib):
    c = Case(51, B=3, N=4, K=2, H=8, bs=4, max_ctx=30)
    base = c.decode(lib)
    rng = np.random.default_rng(5)
    relabel = rng.permutation(c.num_blocks)            # old id -> new id
    kc, vc = np.empty_like(c.kc), np.empty_like(c.vc)
    kc[relabel], vc[relabel] = c.kc, c.vc
    tables = np.where(c.tables >= 0, relabel[np.maximum(c.tables, 0)], -1).astype(np.int32)
    got = oracle.decode(c.q, kc, vc, tables, c.ctx, c.scale, lib=lib)
    assert np.array_equal(got, base), "relabelling physical blocks changed the output"


def check_prefix_sharing(lib):
    """Sequences 1 and 2 reuse sequence 0's first three blocks (shared) versus
    private copies of them: identical outputs."""
    c = Case(61, B=3, N=4, K=2, H=8, bs=4, ctx=[12, 21, 17])
    shared = c.tables[0, :3].copy()
    for b in (1, 2):   # give them private copies first, equal to the shared blocks
        c.kc[c.tables[b, :3]] = c.kc[shared]
        c.vc[c.tables[b, :3]] = c.vc[shared]
    private = c.decode(lib)
    t2 = c.tables.copy()
    t2[1, :3] = shared
    t2[2, :3] = shared
    got = oracle.decode(c.q, c.kc, c.vc, t2, c.ctx, c.scale, lib=lib)
    assert np.array_equal(got, private), "shared prefix blocks differ from private copies"


def check_gqa_is_repeated_mha(lib):
    c = Case(71, B=2, N=8, K=2, H=8, bs=4, max_ctx=25)
    G = c.N // c.K
    got = c.decode(lib)
    kc = np.repeat(c.kc, G, axis=1)    # KV head g copied to heads g*G .. g*G+G-1
    vc = np.repeat(c.vc, G, axis=1)
    mha = oracle.decode(c.q, kc, vc, c.tables, c.ctx, c.scale, lib=lib)
    assert np.array_equal(got, mha), "GQA differs from MHA with repeated KV heads"


def check_key_shift(lib):
    c = Case(81, B=2, N=4, K=2, H=8, bs=4, ctx=[9, 23], grid=True)
    base = c.decode(lib)
    shift = np.array([2, -1, 0, 1, -2, 1, 0, -1], np.float64)
    kf = bits_to_f64(c.kc) + shift
    kc = to_bf16_bits(kf)
    assert np.array_equal(bits_to_f64(kc), kf)
    got = oracle.decode(c.q, kc, c.vc, c.tables, c.ctx, c.scale, lib=lib)
    assert_close(got, base, 1e-12, "adding one vector to every key")


def check_value_affine(lib):
    c = Case(91, B=2, N=4, K=2, H=8, bs=4, ctx=[7, 30], grid=True)
    base = c.decode(lib)
    vf = bits_to_f64(c.vc)
    twice = oracle.decode(c.q, c.kc, to_bf16_bits(vf * 2), c.tables, c.ctx, c.scale, lib=lib)
    assert np.array_equal(twice, base * 2), "doubling V must double the output"
    moved = oracle.decode(c.q, c.kc, to_bf16_bits(vf + 3), c.tables, c.ctx, c.scale, lib=lib)
    assert_close(moved, base + 3, 1e-12, "V + 3")
    const = oracle.decode(c.q, c.kc, to_bf16_bits(np.full_like(vf, -1.25)), c.tables, c.ctx,
                          c.scale, lib=lib)
    assert_close(const, np.full_like(base, -1.25), 1e-14, "constant V")


def check_large_logits(lib):
    """Scores near +-1000: only a max-subtracted softmax stays finite."""
    c = Case(101, B=2, N=4, K=2, H=8, bs=4, ctx=[11, 19], key_mult=4.0)
    big = 60.0
    got = oracle.decode(c.q, c.kc, c.vc, c.tables, c.ctx, big, lib=lib)
    assert_close(got, c.brute(scale=big), 1e-9, "large logits")


def check_scale_is_used(lib):
    c = Case(111, B=2, N=4, K=2, H=16, bs=4, ctx=[15, 26])
    got = c.decode(lib)
    exact = c.brute(scale=1.0 / math.sqrt(c.H))     # the pages divide by sqrt(head_dim)
    assert_close(got, exact, 1e-6, "scale 1/sqrt(H)")


def check_split_merge(lib):
    c = Case(121, B=4, N=4, K=2, H=8, bs=4, ctx=[1, 17, 40, 64])
    whole = c.decode(lib)
    for part in (1, 3, 16, 64, 100):
        got = oracle.decode_split(*c.args(), part, lib=lib)
        assert_close(got, whole, 1e-12, f"split into {part}-token pieces")


def check_rows(lib):
    c = Case(131, B=3, N=4, K=2, H=8, bs=4, max_ctx=30)
    whole = c.decode(lib)
    rb = np.array([2, 0, 1, 2], np.int32)
    rn = np.array([3, 1, 0, 0], np.int32)
    got = oracle.decode_rows(rb, rn, *c.args(), lib=lib)
    assert np.array_equal(got, whole[rb, rn]), "row sampling differs from the full decode"


# ---------------------------------------------------------------- append ----

def _append_case(seed):
    rng = np.random.default_rng(seed)
    T, K, H, bs, nb = 5, 2, 8, 4, 9
    k = to_bf16_bits(rng.standard_normal((T, K, H)))
    v = to_bf16_bits(rng.standard_normal((T, K, H)))
    slots = np.array([13, 0, -1, 35, 22], np.int64)
    sentinel = np.uint16(0x7FA1)      # a NaN pattern no input can produce
    kc = np.full((nb, K, bs, H), sentinel, np.uint16)
    vc = np.full((nb, K, H, bs), sentinel, np.uint16)
    return k, v, slots, kc, vc, sentinel


def check_append_vs_brute(lib):
    k, v, slots, kc, vc, sentinel = _append_case(141)
    bk, bv = kc.astype(np.int64).tolist(), vc.astype(np.int64).tolist()
    brute.paged_append(k.astype(np.int64).tolist(), v.astype(np.int64).tolist(),
                       slots.tolist(), bk, bv)
    oracle.append(k, v, slots, kc, vc, lib=lib)
    assert np.array_equal(kc, np.array(bk, np.uint16)), "K append differs from brute force"
    assert np.array_equal(vc, np.array(bv, np.uint16)), "V append differs from brute force"


def check_append_skips_and_untouched(lib):
    k, v, slots, kc, vc, sentinel = _append_case(151)
    oracle.append(k, v, slots, kc, vc, lib=lib)
    bs = kc.shape[2]
    written = {int(s) for s in slots if s >= 0}
    for blk in range(kc.shape[0]):
        for o in range(bs):
            s = blk * bs + o
            if s in written:
                continue
            assert np.all(kc[blk, :, o, :] == sentinel), f"slot {s} of K touched"
            assert np.all(vc[blk, :, :, o] == sentinel), f"slot {s} of V touched"
    i = int(np.nonzero(slots == 35)[0][0])
    assert np.array_equal(kc[35 // bs, :, 35 % bs, :], k[i])
    assert np.array_equal(vc[35 // bs, :, :, 35 % bs], v[i])


def check_append_then_decode_is_contiguous_update(lib):
    """Paged append + decode equals the lesson's contiguous cache: write the new
    K/V at position seq_len, then attend over positions [0, seq_len + 1)."""
    c = Case(161, B=2, N=4, K=2, H=8, bs=4, ctx=[10, 19])
    rng = np.random.default_rng(7)
    k_new = to_bf16_bits(rng.standard_normal((c.B, c.K, c.H)))
    v_new = to_bf16_bits(rng.standard_normal((c.B, c.K, c.H)))
    last = c.ctx - 1
    slots = np.array([c.tables[b, last[b] // c.bs] * c.bs + last[b] % c.bs
                      for b in range(c.B)], np.int64)
    before = c.contiguous()
    oracle.append(k_new, v_new, slots, c.kc, c.vc, lib=lib)
    got = c.decode(lib)
    G = c.N // c.K
    for b in range(c.B):
        k, v = (a.copy() for a in before[b])     # contiguous [ctx, K, H]
        k[last[b]] = bits_to_f64(k_new[b])
        v[last[b]] = bits_to_f64(v_new[b])
        q = torch.from_numpy(bits_to_f64(c.q[b]))[:, None, :]
        kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)
        vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, scale=c.scale)
        assert_close(got[b], ref[:, 0, :].numpy(), 1e-12, "append then decode")


# ------------------------------------------------------------------- FP8 ----
# OCP FP8 E4M3 pools.  torch's float8_e4m3fn dtype is the library routine the
# code table and the rounding are checked against.

def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.int16).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).float().double().numpy()


def check_e4m3_code_table(lib):
    ref = _torch_e4m3_values()
    got = np.array([oracle.e4m3_value(c, lib=lib) for c in range(256)])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"E4M3 value of codes {np.nonzero(~same)[0][:5]} differs from torch"


def _all_bf16_as_tokens():
    """Every bf16 bit pattern, as [512, 1, 128] tokens for a vectorised append."""
    return np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 1, 128)


def check_e4m3_rounding_vs_torch(lib):
    k = _all_bf16_as_tokens()
    with np.errstate(all="ignore"):     # the sweep includes inf and NaN patterns
        _e4m3_rounding_sweep(k, lib)


def _e4m3_rounding_sweep(k, lib):
    x = bits_to_f64(k).astype(np.float32).reshape(-1)
    for scale in (1.0, 2.0 ** -5, 0.75, 1.0 / 3.0):
        kc = np.zeros((512, 1, 1, 128), np.uint8)
        vc = np.zeros((512, 1, 128, 1), np.uint8)
        slots = np.arange(512, dtype=np.int64)
        # block size 1: token i lands in block i
        oracle.append_fp8(k, k, slots, kc, vc, scale, scale, lib=lib)
        got = kc.reshape(-1)
        inv = np.float32(oracle.fp32_inverse(scale))
        y = torch.from_numpy(x * inv).clamp(-448.0, 448.0)
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        nan = np.isnan(x)
        bad = np.nonzero((got != ref) & ~nan)[0]
        assert bad.size == 0, f"scale {scale}: code of {x[bad[:3]]} differs from torch"
        assert np.all(got[nan] == 0xFF), "NaN must store 0xFF"
        assert np.array_equal(vc.reshape(-1), got), "V pool quantised differently from K"


def check_fp8_decode_is_bf16_decode_of_its_values(lib):
    """With power-of-two scales every FP8 value times its scale is a bf16 value:
    decoding the FP8 pools equals decoding bf16 pools holding those values."""
    c = Case(171, B=3, N=8, K=2, H=16, bs=4, max_ctx=40)
    rng = np.random.default_rng(9)
    finite = np.array([i for i in range(256) if (i & 0x7F) != 0x7F], np.uint8)
    kc8 = rng.choice(finite, size=c.kc.shape).astype(np.uint8)
    vc8 = rng.choice(finite, size=c.vc.shape).astype(np.uint8)
    ks, vs = 2.0 ** -4, 2.0 ** 3
    table = _torch_e4m3_values()
    kc16 = to_bf16_bits(table[kc8] * ks)
    vc16 = to_bf16_bits(table[vc8] * vs)
    assert np.array_equal(bits_to_f64(kc16), table[kc8] * ks)
    got = oracle.decode_fp8(c.q, kc8, vc8, c.tables, c.ctx, c.scale, ks, vs, lib=lib)
    ref = oracle.decode(c.q, kc16, vc16, c.tables, c.ctx, c.scale, lib=lib)
    assert np.array_equal(got, ref), "FP8 decode differs from the bf16 decode of its values"
    rb = np.array([2, 0, 1], np.int32)
    rn = np.array([7, 3, 0], np.int32)
    rows = oracle.decode_rows_fp8(rb, rn, c.q, kc8, vc8, c.tables, c.ctx, c.scale, ks, vs,
                                  lib=lib)
    assert np.array_equal(rows, got[rb, rn]), "FP8 row sampling differs from the full decode"


def check_append_fp8_scatter(lib):
    k, v, slots, _, _, _ = _append_case(181)
    T, K, H = k.shape
    nb, bs = 9, 4
    sentinel = np.uint8(0x5A)
    kc = np.full((nb, K, bs, H), sentinel, np.uint8)
    vc = np.full((nb, K, H, bs), sentinel, np.uint8)
    ks, vs = 2.0 ** -5, 0.1
    oracle.append_fp8(k, v, slots, kc, vc, ks, vs, lib=lib)
    for i, s_ in enumerate(slots):
        if s_ < 0:
            continue
        p_, o_ = divmod(int(s_), bs)
        want_k = [oracle.e4m3_quantize(b, oracle.fp32_inverse(ks), lib=lib) for b in k[i].reshape(-1)]
        want_v = [oracle.e4m3_quantize(b, oracle.fp32_inverse(vs), lib=lib) for b in v[i].reshape(-1)]
        assert np.array_equal(kc[p_, :, o_, :].reshape(-1), np.array(want_k, np.uint8))
        assert np.array_equal(vc[p_, :, :, o_].reshape(-1), np.array(want_v, np.uint8))
    written = {int(x) for x in slots if x >= 0}
    for blk in range(nb):
        for o_ in range(bs):
            if blk * bs + o_ not in written:
                assert np.all(kc[blk, :, o_, :] == sentinel) and np.all(vc[blk, :, :, o_] == sentinel)


# ------------------------------------------------------------ accounting ----

def check_printed_kv_sizes(lib):
    facts = json.load(open(GOLDEN))
    for f in facts["facts"]:
        got = oracle.kv_cache_bytes(f["layers"], f["kv_heads"], f["head_dim"], f["tokens"],
                                    f["bytes"], lib=lib)
        assert got == f["exact"], f"{f['id']}: {got} != {f['exact']}"
        shown = got / f["unit"]
        assert abs(shown - f["printed"]) <= f["rel_tol"] * f["printed"] + 1e-12, \
            f"{f['id']}: {shown} does not round to the printed {f['printed']}"
    for r in facts["gqa_reduction"]:
        mha = oracle.kv_cache_bytes(1, r["N"], 128, 1, 2, lib=lib)
        gqa = oracle.kv_cache_bytes(1, r["K"], 128, 1, 2, lib=lib)
        assert mha == r["factor"] * gqa


# ----------------------------------------------------------- multi-query ----
# Q query tokens per sequence, q and out [B, Q, N, H].

def _multi_case(seed, Q, **kw):
    c = Case(seed, **kw)
    rng = np.random.default_rng(seed + 1000)
    c.Q = Q
    c.qm = to_bf16_bits(rng.standard_normal((c.B, Q, c.N, c.H)))
    return c


def check_multi_brute_force(lib):
    for seed, (Q, N, K, bs, H) in enumerate([(3, 4, 2, 4, 8), (5, 6, 1, 4, 4),
                                              (2, 4, 4, 16, 8)]):
        c = _multi_case(300 + seed, Q, N=N, K=K, bs=bs, H=H, max_ctx=30)
        c.ctx = np.maximum(c.ctx, Q).astype(np.int32)      # the Q tokens are in the cache
        got = oracle.decode_multi(c.qm, c.kc, c.vc, c.tables, c.ctx, c.scale, lib=lib)
        ref = np.array(brute.paged_decode_multi(
            bits_to_f64(c.qm).tolist(), bits_to_f64(c.kc).tolist(), bits_to_f64(c.vc).tolist(),
            c.tables.tolist(), c.ctx.tolist(), c.scale))
        assert_close(got, ref, 1e-12, f"multi-query brute force (Q={Q}, N={N}, K={K})")


def check_multi_torch_bottom_right_mask(lib):
    """torch float64 SDPA on the gathered cache with the lesson's mask: key j
    is hidden from query r when j - r >= Sk - Sq + 1 (np.triu with that
    diagonal offset)."""
    Q = 4
    c = _multi_case(311, Q, B=3, N=8, K=2, H=16, bs=4, ctx=[4, 17, 33])
    got = oracle.decode_multi(c.qm, c.kc, c.vc, c.tables, c.ctx, c.scale, lib=lib)
    qf = bits_to_f64(c.qm)
    G = c.N // c.K
    for b, (kb, vb) in enumerate(c.contiguous()):
        Sk = int(c.ctx[b])
        hidden = np.triu(np.ones((Q, Sk), bool), k=Sk - Q + 1)
        qt = torch.from_numpy(qf[b].transpose(1, 0, 2).copy())            # [N, Q, H]
        kt = torch.from_numpy(np.repeat(kb.transpose(1, 0, 2), G, axis=0).copy())  # [N, Sk, H]
        vt = torch.from_numpy(np.repeat(vb.transpose(1, 0, 2), G, axis=0).copy())
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.from_numpy(~hidden), scale=c.scale)
        assert_close(got[b], ref.numpy().transpose(1, 0, 2), 1e-12,
                     f"multi-query vs torch SDPA with the bottom-right mask (seq {b})")


def check_multi_q1_is_decode(lib):
    c = Case(321, B=4, N=8, K=2, H=8, bs=4, max_ctx=50)
    got = oracle.decode_multi(c.q.reshape(c.B, 1, c.N, c.H), c.kc, c.vc, c.tables, c.ctx,
                              c.scale, lib=lib)
    assert np.array_equal(got[:, 0], c.decode(lib)), "Q = 1 differs from single-token decode"


def check_multi_is_sequential_decoding(lib):
    """Verification of Q appended tokens equals decoding them one after
    another: the i-th token's step sees the cache up to and including itself."""
    Q = 5
    c = _multi_case(331, Q, B=3, N=4, K=2, H=8, bs=4, ctx=[5, 23, 40])
    got = oracle.decode_multi(c.qm, c.kc, c.vc, c.tables, c.ctx, c.scale, lib=lib)
    for i in range(Q):
        step = oracle.decode(np.ascontiguousarray(c.qm[:, i]), c.kc, c.vc, c.tables,
                             (c.ctx - (Q - 1 - i)).astype(np.int32), c.scale, lib=lib)
        assert np.array_equal(got[:, i], step), f"query {i} differs from its sequential step"


def check_multi_rows_and_fp8(lib):
    Q = 3
    c = _multi_case(341, Q, B=3, N=6, K=3, H=8, bs=4, ctx=[3, 20, 31])
    full = oracle.decode_multi(c.qm, c.kc, c.vc, c.tables, c.ctx, c.scale, lib=lib)
    rb = np.array([2, 0, 1, 2], np.int32)
    ri = np.array([0, 2, 1, 2], np.int32)
    rn = np.array([5, 0, 3, 1], np.int32)
    rows = oracle.decode_multi_rows(rb, ri, rn, c.qm, c.kc, c.vc, c.tables, c.ctx, c.scale,
                                    lib=lib)
    assert np.array_equal(rows, full[rb, ri, rn]), "sampled rows differ from the full result"
    rng = np.random.default_rng(342)
    finite = np.array([i for i in range(256) if (i & 0x7F) != 0x7F], np.uint8)
    kc8 = rng.choice(finite, size=c.kc.shape).astype(np.uint8)
    vc8 = rng.choice(finite, size=c.vc.shape).astype(np.uint8)
    got = oracle.decode_multi(c.qm[:, :1], kc8, vc8, c.tables, c.ctx, c.scale, 0.5, 0.25,
                              lib=lib)
    ref = oracle.decode_fp8(np.ascontiguousarray(c.qm[:, 0]), kc8, vc8, c.tables, c.ctx,
                            c.scale, 0.5, 0.25, lib=lib)
    assert np.array_equal(got[:, 0], ref), "FP8 multi-query with Q = 1 differs from FP8 decode"


# ------------------------------------------------------------ block copy ----

def check_copy_blocks_brute_force(lib):
    rng = np.random.default_rng(401)
    nb, K, bs, H = 7, 2, 4, 3
    for dtype in (np.uint16, np.uint8):
        kc = rng.integers(0, np.iinfo(dtype).max, (nb, K, bs, H)).astype(dtype)
        vc = rng.integers(0, np.iinfo(dtype).max, (nb, K, H, bs)).astype(dtype)
        src = np.array([1, 4, -1, 2, 5], np.int32)
        dst = np.array([3, 0, 6, 1, 5], np.int32)     # 1 is copied out before it is overwritten
        kl, vl = kc.tolist(), vc.tolist()
        brute.copy_blocks(kl, vl, src.tolist(), dst.tolist())
        oracle.copy_blocks(kc, vc, src, dst, lib=lib)
        assert np.array_equal(kc, np.array(kl, dtype)), f"key pool copy ({dtype.__name__})"
        assert np.array_equal(vc, np.array(vl, dtype)), f"value pool copy ({dtype.__name__})"


def check_copy_on_write_divergence(lib):
    """Two sequences share a partly filled block; before the second writes its
    next token there, the block is copied and its table re-pointed.  Then the
    first sequence's result is unchanged, and the second's equals what private
    blocks holding the same values give."""
    c = Case(411, B=2, N=4, K=2, H=8, bs=4, ctx=[6, 6])
    kc, vc = c.kc.copy(), c.vc.copy()
    shared = c.tables[0, :2].copy()
    tables = c.tables.copy()
    tables[1, :2] = shared                       # both point at the same two blocks
    ctx = np.array([6, 6], np.int32)
    before0 = oracle.decode(c.q, kc, vc, tables, ctx, c.scale, lib=lib)[0]
    fresh = int(c.num_blocks - 1)                # a spare block no table uses
    oracle.copy_blocks(kc, vc, np.array([shared[1]], np.int32), np.array([fresh], np.int32),
                       lib=lib)
    tables[1, 1] = fresh
    rng = np.random.default_rng(412)
    k_new = to_bf16_bits(rng.standard_normal((1, c.K, c.H)))
    v_new = to_bf16_bits(rng.standard_normal((1, c.K, c.H)))
    oracle.append(k_new, v_new, np.array([fresh * c.bs + 2], np.int64), kc, vc, lib=lib)
    ctx2 = np.array([6, 7], np.int32)
    after = oracle.decode(c.q, kc, vc, tables, ctx2, c.scale, lib=lib)
    assert np.array_equal(after[0], before0), "the other sharer's result changed"
    # reference: private copies of both blocks for sequence 1, new token written there
    kp, vp = c.kc.copy(), c.vc.copy()
    priv = np.array([c.num_blocks - 2, c.num_blocks - 1], np.int32)
    kp[priv] = kp[shared]
    vp[priv] = vp[shared]
    oracle.append(k_new, v_new, np.array([priv[1] * c.bs + 2], np.int64), kp, vp, lib=lib)
    t2 = tables.copy()
    t2[1, :2] = priv
    ref = oracle.decode(c.q, kp, vp, t2, ctx2, c.scale, lib=lib)
    assert np.array_equal(after[1], ref[1]), "diverged sharer differs from private copies"


# --------------------------------------------------------- sliding window ----

def check_window_brute_force(lib):
    for seed, (N, K, bs, H, W) in enumerate([(4, 2, 4, 8, 7), (6, 1, 4, 4, 1),
                                              (4, 4, 16, 8, 20)]):
        c = Case(500 + seed, N=N, K=K, bs=bs, H=H, max_ctx=40)
        got = oracle.decode_window(c.q, c.kc, c.vc, c.tables, c.ctx, c.scale, W, lib=lib)
        ref = np.array(brute.paged_decode_window(
            bits_to_f64(c.q).tolist(), bits_to_f64(c.kc).tolist(), bits_to_f64(c.vc).tolist(),
            c.tables.tolist(), c.ctx.tolist(), c.scale, W))
        assert_close(got, ref, 1e-12, f"sliding window brute force (W={W})")


def check_window_special_cases(lib):
    c = Case(511, B=5, N=4, K=2, H=8, bs=4, ctx=[1, 12, 16, 32, 9])
    full = c.decode(lib)
    wide = oracle.decode_window(c.q, c.kc, c.vc, c.tables, c.ctx, c.scale, 32, lib=lib)
    assert np.array_equal(wide, full), "a window covering the context must be full attention"
    one = oracle.decode_window(c.q, c.kc, c.vc, c.tables, c.ctx, c.scale, 1, lib=lib)
    vf = bits_to_f64(c.vc)
    G = c.N // c.K
    for b in range(c.B):
        t = int(c.ctx[b]) - 1
        p, o = c.tables[b, t // c.bs], t % c.bs
        for n in range(c.N):
            assert np.array_equal(one[b, n], vf[p, n // G, :, o]), "window 1 must return the new V"
    # a window of W equals full attention over a cache whose first ctx - W
    # positions were never there: drop them by shifting the sequence's blocks
    # (block-aligned drops: 0, 4, 8, 24 positions for the first four)
    W = 8
    got = oracle.decode_window(c.q, c.kc, c.vc, c.tables, c.ctx, c.scale, W, lib=lib)
    checked = 0
    for b in range(c.B):
        ctx = int(c.ctx[b])
        drop = max(ctx - W, 0)
        if drop % c.bs:
            continue               # only block-aligned drops are table shifts
        t2 = c.tables.copy()
        t2[b, :t2.shape[1] - drop // c.bs] = c.tables[b, drop // c.bs:]
        cl2 = c.ctx.copy()
        cl2[b] = ctx - drop
        ref = oracle.decode(c.q, c.kc, c.vc, t2, cl2, c.scale, lib=lib)
        assert np.array_equal(got[b], ref[b]), "window differs from the shortened cache"
        checked += 1
    assert checked == 4


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
