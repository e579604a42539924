"""Seeded synthetic inputs for paged-KV decode attention.

This module only draws inputs: random bf16 tensors, context lengths, physical
block assignments and the slot of each step's new token.  It holds none of the
attention or append arithmetic, so both the HIP library's tests and the CPU
oracle can take their inputs from it.  Everything is generated on the CPU with
a seeded ``torch.Generator`` and is identical on every machine.

Workload shapes follow the models the pages discuss (notation of "CS336
Lecture 10: Inference", part 1: B sequences, N query heads, K KV heads, H head
dim):
  * Llama-3-8B layer (N 32, K 8, H 128) at B 64 x 8k context -- the example of
    "Week 11. Inference", steps 2 and 4;
  * Llama-2-13B MHA layer (N = K = 40, H 128) at context 1024, B 1/64/256 --
    the latency/throughput example of "CS336 Lecture 10: Inference", part 2;
  * Llama-3-70B layer (N 64, K 8, H 128) -- the KV-cache memory example of
    the "Optimización de la inferencia" lesson -- as a continuous-batching mix
    of ragged contexts with a shared 1000-token prefix (the prefix-caching
    example of "Week 11. Inference", step 2), and at 128K context.
Pages of 16 tokens follow the PagedAttention section of the same lesson.

Layouts: key_cache [num_blocks][K][bs][H], value_cache [num_blocks][K][H][bs]
(bf16, or uint8 E4M3 codes for FP8 pools); block_tables [B][max_blocks] int32;
context_lens [B] int32 (the step's new tokens included); slot_mapping = block *
bs + offset of each new token's position.  A step appends one token per
sequence (position context_len - 1), or Q tokens for the speculative-verify
workloads (positions context_len - Q .. context_len - 1, whose queries are then
attended together: q [B][Q][N][H], k_new / v_new [B * Q][K][H]).

Poisoning (``poison=True``): cache slots that hold no valid token (block
tails, and the new token's slot before the append) are bf16 NaN (0x7FC0), and
block-table entries past a sequence's last block point at one extra pool
block filled with NaN.  A kernel that reads any of them produces NaN.

FP8 pools (``kv_dtype="fp8"``, the 8-bit cache of "Week 11. Inference",
step 2): the same draws, stored as OCP FP8 E4M3 codes (uint8) with one scale
per pool chosen so that 6 standard deviations map to the largest code, 448:
k_scale = 6 * key_scale / 448, v_scale = 6 / 448 (fp32).  The cached codes
are the drawn values divided by the pool scale, clamped to +-448 and cast
with torch's float8_e4m3fn conversion; poison is the NaN code 0x7F.  The
step's new rows stay bf16 (the append quantises them).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

BF16_NAN_BITS = 0x7FC0
E4M3_NAN_CODE = 0x7F
E4M3_MAX = 448.0
FP8_SIGMAS = 6.0


@dataclasses.dataclass(frozen=True)
class Spec:
    """What to draw.  ``ctx`` is either a list of context lengths or one of
    'uniform' (ctx_lo..ctx_hi) / 'lognormal' (median, sigma, clip)."""
    name: str
    B: int
    N: int
    K: int
    H: int
    bs: int = 16
    ctx: object = 1024
    ctx_lo: int = 1
    ctx_hi: int = 256
    median: float = 2000.0
    sigma: float = 1.0
    max_blocks: Optional[int] = None
    pool_blocks: Optional[int] = None     # None: exactly the blocks needed
    key_scale: float = 1.0
    shared_prefix: int = 0                # tokens of the shared prefix
    sharers: int = 0
    partition_size: int = 0               # 0: the library chooses
    seed: int = 0
    kv_dtype: str = "bf16"                # "bf16" or "fp8" (E4M3 codes, one scale per pool)
    queries: int = 1                      # Q query tokens per sequence (speculative verify)


# The workloads (seed = 1000 + index).
SPECS = {
    "tiny": Spec("tiny", B=4, N=8, K=2, H=64, bs=16, ctx="uniform", ctx_lo=1,
                 ctx_hi=256, max_blocks=16, pool_blocks=128, seed=1001),
    "llama3_8b_b64_ctx8k": Spec("llama3_8b_b64_ctx8k", B=64, N=32, K=8, H=128, bs=16,
                                ctx=8192, seed=1002),
    "llama2_13b_b1_ctx1k": Spec("llama2_13b_b1_ctx1k", B=1, N=40, K=40, H=128, bs=16,
                                ctx=1024, seed=1003),
    "llama2_13b_b64_ctx1k": Spec("llama2_13b_b64_ctx1k", B=64, N=40, K=40, H=128, bs=16,
                                 ctx=1024, seed=1003),
    "llama2_13b_b256_ctx1k": Spec("llama2_13b_b256_ctx1k", B=256, N=40, K=40, H=128, bs=16,
                                  ctx=1024, seed=1003),
    "llama3_70b_ragged_b100": Spec("llama3_70b_ragged_b100", B=100, N=64, K=8, H=128, bs=16,
                                   ctx="lognormal", median=2000.0, sigma=1.0,
                                   ctx_lo=16, ctx_hi=8192, max_blocks=512, key_scale=2.0,
                                   shared_prefix=1000, sharers=20, seed=1004),
    "llama3_70b_long_b4_ctx128k": Spec("llama3_70b_long_b4_ctx128k", B=4, N=64, K=8, H=128,
                                       bs=16, ctx=131072, partition_size=512, seed=1005),
    # Speculative verification: gamma draft tokens plus one, all queried at once.
    # Partition sizes: one wave per (sequence, KV head) fills half the chip and
    # needs no merge (8B); two per pair fill it (70B, three tiles per wave).
    "llama3_8b_b64_ctx8k_spec4": Spec("llama3_8b_b64_ctx8k_spec4", B=64, N=32, K=8, H=128,
                                      bs=16, ctx=8192, queries=4, partition_size=8192,
                                      seed=1006),
    "llama3_70b_b64_ctx4k_spec6": Spec("llama3_70b_b64_ctx4k_spec6", B=64, N=64, K=8, H=128,
                                       bs=16, ctx=4096, queries=6, partition_size=2048,
                                       seed=1007),
}
# The same draws in FP8 pools.
for _name in ("tiny", "llama3_8b_b64_ctx8k", "llama3_70b_ragged_b100"):
    SPECS[_name + "_fp8"] = dataclasses.replace(SPECS[_name], name=_name + "_fp8", kv_dtype="fp8")


@dataclasses.dataclass
class Workload:
    spec: Spec
    q: torch.Tensor              # [B, N, H] bf16 ([B, Q, N, H] with Q > 1 queries)
    k_new: torch.Tensor          # [B * Q, K, H] bf16
    v_new: torch.Tensor          # [B * Q, K, H] bf16
    slot_mapping: torch.Tensor   # [B * Q] int64
    key_cache: torch.Tensor      # [nb, K, bs, H] bf16 or uint8 codes (state before the append)
    value_cache: torch.Tensor    # [nb, K, H, bs] bf16 or uint8 codes
    block_tables: torch.Tensor   # [B, max_blocks] int32
    context_lens: torch.Tensor   # [B] int32
    scale: float                 # fp32 value of 1/sqrt(H)
    sharer_ids: List[int]
    shared_blocks: List[int]
    poison_block: Optional[int]
    kv_dtype: str = "bf16"
    k_scale: float = 1.0         # FP8 pools: a key code c stands for e4m3(c) * k_scale
    v_scale: float = 1.0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.numel() else 0

    @property
    def num_blocks(self) -> int:
        return self.key_cache.shape[0]

    def to(self, device) -> "Workload":
        out = dataclasses.replace(self)
        for f in ("q", "k_new", "v_new", "slot_mapping", "key_cache", "value_cache",
                  "block_tables", "context_lens"):
            setattr(out, f, getattr(self, f).to(device))
        return out


def fp32_scale(H: int) -> float:
    """1/sqrt(H) rounded to fp32, as a Python float."""
    return float(torch.tensor(1.0 / math.sqrt(H), dtype=torch.float32))


def fp8_scales(spec: Spec):
    """(k_scale, v_scale) of a workload's FP8 pools, fp32 values as floats."""
    f32 = lambda x: float(torch.tensor(x, dtype=torch.float32))
    return (f32(FP8_SIGMAS * spec.key_scale / E4M3_MAX), f32(FP8_SIGMAS / E4M3_MAX))


def _e4m3_codes(x: torch.Tensor, scale: float) -> torch.Tensor:
    """Codes of x / scale (clamped to the finite range; NaN stays NaN) as uint8."""
    y = (x.float() / scale).clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def _randn_bf16(shape, gen, mult: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    if mult != 1.0:
        x = x * mult           # a power of two: exact in bf16
    return x


def _context_lengths(spec: Spec, gen) -> List[int]:
    if isinstance(spec.ctx, int):
        return [spec.ctx] * spec.B
    if isinstance(spec.ctx, (list, tuple)):
        assert len(spec.ctx) == spec.B
        return [int(c) for c in spec.ctx]
    if spec.ctx == "uniform":
        return torch.randint(spec.ctx_lo, spec.ctx_hi + 1, (spec.B,), generator=gen).tolist()
    if spec.ctx == "lognormal":
        z = torch.randn(spec.B, generator=gen, dtype=torch.float64)
        raw = torch.exp(math.log(spec.median) + spec.sigma * z)
        return [int(min(max(round(float(x)), spec.ctx_lo), spec.ctx_hi)) for x in raw]
    raise ValueError(f"unknown ctx kind {spec.ctx!r}")


@dataclasses.dataclass
class Layout:
    """The integer part of a workload: contexts, block tables, slots."""
    spec: Spec
    context_lens: List[int]
    blocks_per_seq: List[int]
    block_tables: torch.Tensor   # [B, max_blocks] int32
    slot_mapping: torch.Tensor   # [B] int64
    num_blocks: int              # pool size, including the poison block if any
    sharer_ids: List[int]
    shared_blocks: List[int]
    poison_block: Optional[int]


def _resolve(spec_or_name) -> Spec:
    return SPECS[spec_or_name] if isinstance(spec_or_name, str) else spec_or_name


def _layout(spec: Spec, gen: torch.Generator, poison: bool) -> Layout:
    B, bs = spec.B, spec.bs
    if spec.N % spec.K:
        raise ValueError("N must be a multiple of K")
    ctx = _context_lengths(spec, gen)
    nblk = [-(-c // bs) for c in ctx]
    max_blocks = spec.max_blocks or max([1] + nblk)
    if max(nblk + [0]) > max_blocks:
        raise ValueError("a context does not fit the block table")

    # Sequences sharing the prefix: the first `sharers` in batch order whose
    # new token lies past the prefix.  Only whole blocks are shared; the
    # prefix's partial last block is a private copy in each sharer.
    sharer_ids: List[int] = []
    if spec.sharers:
        sharer_ids = [b for b in range(B) if ctx[b] > spec.shared_prefix][:spec.sharers]
        if len(sharer_ids) < spec.sharers:
            raise ValueError("not enough sequences long enough to share the prefix")
    n_shared = spec.shared_prefix // bs if sharer_ids else 0

    unique = sum(nblk) - max(0, len(sharer_ids) - 1) * n_shared
    pool = spec.pool_blocks if spec.pool_blocks is not None else unique
    if pool < unique:
        raise ValueError("pool too small")
    perm = torch.randperm(pool, generator=gen).tolist()
    need_poison = poison and any(n < max_blocks for n in nblk)
    poison_block = pool if need_poison else None

    tables = torch.full((B, max_blocks), poison_block if need_poison else 0, dtype=torch.int32)
    nxt = 0
    shared_ids: List[int] = []
    for b in range(B):
        for j in range(nblk[b]):
            if shared_ids and b in sharer_ids and j < n_shared:
                tables[b, j] = shared_ids[j]
            else:
                tables[b, j] = perm[nxt]
                nxt += 1
        if sharer_ids and b == sharer_ids[0]:
            shared_ids = tables[b, :n_shared].tolist()

    # The step's new tokens: positions ctx - Q .. ctx - 1 of each sequence
    # (token-major within a sequence); a position below 0 gets slot -1.
    Q = spec.queries
    slots = torch.empty(B * Q, dtype=torch.int64)
    for b in range(B):
        for i in range(Q):
            pos = ctx[b] - Q + i
            slots[b * Q + i] = int(tables[b, pos // bs]) * bs + pos % bs if pos >= 0 else -1
    return Layout(spec=spec, context_lens=ctx, blocks_per_seq=nblk, block_tables=tables,
                  slot_mapping=slots, num_blocks=pool + (1 if need_poison else 0),
                  sharer_ids=sharer_ids, shared_blocks=shared_ids, poison_block=poison_block)


def layout(spec_or_name, poison: bool = True) -> Layout:
    """Only the integer layout of a workload (no values drawn); identical to
    what ``make`` produces for the same arguments."""
    spec = _resolve(spec_or_name)
    return _layout(spec, torch.Generator().manual_seed(spec.seed), poison)


def make(spec_or_name, poison: bool = True) -> Workload:
    """Draw a workload.  Deterministic for a given Spec and ``poison`` flag."""
    spec = _resolve(spec_or_name)
    gen = torch.Generator().manual_seed(spec.seed)
    lay = _layout(spec, gen, poison)
    B, N, K, H, bs = spec.B, spec.N, spec.K, spec.H, spec.bs

    Q = spec.queries
    q = _randn_bf16((B, N, H) if Q == 1 else (B, Q, N, H), gen)
    k_new = _randn_bf16((B * Q, K, H), gen, spec.key_scale)
    v_new = _randn_bf16((B * Q, K, H), gen)
    prefix_k = prefix_v = None
    if lay.sharer_ids:
        prefix_k = _randn_bf16((spec.shared_prefix, K, H), gen, spec.key_scale)
        prefix_v = _randn_bf16((spec.shared_prefix, K, H), gen)

    fp8 = spec.kv_dtype == "fp8"
    if spec.kv_dtype not in ("bf16", "fp8"):
        raise ValueError(f"unknown kv_dtype {spec.kv_dtype!r}")
    k_scale, v_scale = fp8_scales(spec) if fp8 else (1.0, 1.0)
    pool_dtype = torch.uint8 if fp8 else torch.bfloat16
    key_cache = torch.empty((lay.num_blocks, K, bs, H), dtype=pool_dtype)
    value_cache = torch.empty((lay.num_blocks, K, H, bs), dtype=pool_dtype)
    fill_bits = BF16_NAN_BITS if poison else 0
    if fp8:
        key_cache.fill_(E4M3_NAN_CODE if poison else 0)
        value_cache.fill_(E4M3_NAN_CODE if poison else 0)
    else:
        key_cache.view(torch.int16).fill_(fill_bits)
        value_cache.view(torch.int16).fill_(fill_bits)

    for b in range(B):
        nb_b = lay.blocks_per_seq[b]
        n_tok = nb_b * bs
        lk = _randn_bf16((n_tok, K, H), gen, spec.key_scale)
        lv = _randn_bf16((n_tok, K, H), gen)
        if b in lay.sharer_ids:
            lk[:spec.shared_prefix] = prefix_k
            lv[:spec.shared_prefix] = prefix_v
        # Only positions [0, ctx-1) are in the cache before this step's append;
        # the new token's slot and the block tail hold the fill pattern.
        valid = max(lay.context_lens[b] - Q, 0)
        lk[valid:].view(torch.int16).fill_(fill_bits)
        lv[valid:].view(torch.int16).fill_(fill_bits)
        if fp8:
            lk = _e4m3_codes(lk, k_scale)
            lv = _e4m3_codes(lv, v_scale)
        ids = lay.block_tables[b, :nb_b].long()
        key_cache[ids] = lk.view(nb_b, bs, K, H).permute(0, 2, 1, 3)
        value_cache[ids] = lv.view(nb_b, bs, K, H).permute(0, 2, 3, 1)

    return Workload(spec=spec, q=q, k_new=k_new, v_new=v_new, slot_mapping=lay.slot_mapping,
                    key_cache=key_cache, value_cache=value_cache,
                    block_tables=lay.block_tables,
                    context_lens=torch.tensor(lay.context_lens, dtype=torch.int32),
                    scale=fp32_scale(H), sharer_ids=lay.sharer_ids,
                    shared_blocks=lay.shared_blocks, poison_block=lay.poison_block,
                    kv_dtype=spec.kv_dtype, k_scale=k_scale, v_scale=v_scale)


def small(name: str, **overrides) -> Spec:
    """A reduced variant of a named workload the oracle finishes in seconds
    (same heads, head dim and block size; fewer sequences and tokens)."""
    base = SPECS[name]
    key = name[:-len("_fp8")] if name.endswith("_fp8") else name
    defaults = {
        "llama3_8b_b64_ctx8k": dict(B=3, ctx=[700, 1040, 33]),
        "llama2_13b_b1_ctx1k": dict(B=1, ctx=[1024]),
        "llama2_13b_b64_ctx1k": dict(B=4, ctx=[1024, 1024, 1024, 1024]),
        "llama2_13b_b256_ctx1k": dict(B=6, ctx=[1024] * 6),
        "llama3_70b_ragged_b100": dict(B=12, ctx="lognormal", median=300.0,
                                       ctx_hi=1500, max_blocks=96, shared_prefix=200,
                                       sharers=4),
        "llama3_70b_long_b4_ctx128k": dict(B=2, ctx=[2600, 1537]),
        "llama3_8b_b64_ctx8k_spec4": dict(B=3, ctx=[700, 1040, 5]),
        "llama3_70b_b64_ctx4k_spec6": dict(B=3, ctx=[600, 1039, 6]),
        "tiny": dict(),
    }[key]
    defaults.update(overrides)
    return dataclasses.replace(base, name=base.name + "_small", **defaults)
