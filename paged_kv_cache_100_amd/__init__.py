"""Paged-KV decode attention and K/V append for AMD MI355X (gfx950).

A thin Python binding over ``libpagedkv.so`` (C ABI in ``include/pagedkv.h``).
It only checks tensor types, derives the size arguments from tensor shapes,
and passes device pointers and torch's current HIP stream; every step of the
computation runs in the library's HIP kernels.  The library must be built
(``python -m paged_kv_cache_100_amd.build``); without it every call raises.

    paged_kv_append(k, v, slot_mapping, key_cache, value_cache)
    paged_decode_attention(out, q, key_cache, value_cache, block_tables,
                           context_lens, scale, num_kv_heads, block_size)
    paged_kv_append_fp8(k, v, slot_mapping, key_cache, value_cache, k_scale, v_scale)
    paged_decode_attention_fp8(out, q, key_cache, value_cache, block_tables,
                               context_lens, scale, k_scale, v_scale, num_kv_heads,
                               block_size)
    paged_decode_attention_mq(out, q, key_cache, value_cache, block_tables,
                              context_lens, scale, num_kv_heads, block_size, partition)
    paged_decode_attention_prefix(out, q, key_cache, value_cache, block_tables,
                                  context_lens, scale, num_kv_heads, block_size, partition,
                                  seq_group, group_members, prefix_tokens)
    paged_kv_copy_blocks(key_cache, value_cache, src_blocks, dst_blocks)
    paged_decode_attention_window(out, q, key_cache, value_cache, block_tables,
                                  context_lens, scale, num_kv_heads, block_size, window)
    paged_decode_attention_noalloc(out, q, key_cache, value_cache, block_tables,
                                   context_lens, scale, num_kv_heads, block_size)

Layouts: k, v [T, K, H] bf16; slot_mapping [T] int64; key_cache
[num_blocks, K, bs, H]; value_cache [num_blocks, K, H, bs], bs 16 or 32 (bf16, or for the
``_fp8`` calls one-byte OCP FP8 E4M3 codes as uint8 or float8_e4m3fn, one
scale per pool); q [B, N, H] bf16; out [B, N, H] float32; block_tables
[B, max_blocks] int32; context_lens [B] int32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpagedkv.so")

STATUS = {0: "PKV_OK", -1: "PKV_ERR_NULL", -2: "PKV_ERR_SHAPE", -3: "PKV_ERR_UNSUPPORTED",
          -4: "PKV_ERR_ALIGN", -5: "PKV_ERR_WORKSPACE", -6: "PKV_ERR_LAUNCH",
          -7: "PKV_ERR_DEVICE", -8: "PKV_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20     # PKV_NOALLOC_SCRATCH_BYTES

_lib = None


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m paged_kv_cache_100_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    L.paged_kv_append.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i64, P]
    L.paged_kv_append.restype = ctypes.c_int
    L.paged_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.paged_decode_workspace_size.restype = sz
    L.paged_decode_attention.argtypes = [P, P, P, P, P, P, f32, i32, i32, i32, i32, i32, i32,
                                         i32, i64, i32, P, sz, P]
    L.paged_decode_attention.restype = ctypes.c_int
    L.paged_decode_attention_noalloc.argtypes = [P, P, P, P, P, P, f32, i32, i32, i32, i32, i32,
                                                 i32, i32, i64, i32, P]
    L.paged_decode_attention_noalloc.restype = ctypes.c_int
    L.paged_kv_append_fp8.argtypes = [P, P, P, P, P, f32, f32, i32, i32, i32, i32, i64, P]
    L.paged_kv_append_fp8.restype = ctypes.c_int
    L.paged_decode_attention_fp8.argtypes = [P, P, P, P, P, P, f32, f32, f32, i32, i32, i32, i32,
                                             i32, i32, i32, i64, i32, P, sz, P]
    L.paged_decode_attention_fp8.restype = ctypes.c_int
    L.paged_decode_mq_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.paged_decode_mq_workspace_size.restype = sz
    L.paged_decode_prefix_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.paged_decode_prefix_workspace_size.restype = sz
    L.paged_decode_attention_mq.argtypes = [P, P, P, P, P, P, f32, i32, f32, f32, i32, i32, i32,
                                            i32, i32, i32, i32, i32, i64, i32, P, sz, P]
    L.paged_decode_attention_mq.restype = ctypes.c_int
    L.paged_decode_attention_prefix.argtypes = [P, P, P, P, P, P, f32, i32, f32, f32, i32, i32,
                                                i32, i32, i32, i32, i32, i64, i32, P, P, P, i32,
                                                i32, i32, P, sz, P]
    L.paged_decode_attention_prefix.restype = ctypes.c_int
    L.paged_decode_attention_window.argtypes = [P, P, P, P, P, P, f32, i32, f32, f32, i32, i32,
                                                i32, i32, i32, i32, i32, i32, i64, i32, P, sz, P]
    L.paged_decode_attention_window.restype = ctypes.c_int
    L.paged_kv_copy_blocks.argtypes = [P, P, P, P, i32, i32, i32, i32, i64, i32, P]
    L.paged_kv_copy_blocks.restype = ctypes.c_int
    L.pagedkv_stream_read_sink_bytes.argtypes = [sz]
    L.pagedkv_stream_read_sink_bytes.restype = sz
    L.pagedkv_stream_read.argtypes = [P, sz, P, P]
    L.pagedkv_stream_read.restype = ctypes.c_int
    L.pagedkv_stream_copy.argtypes = [P, P, sz, P]
    L.pagedkv_stream_copy.restype = ctypes.c_int
    L.pagedkv_status_string.argtypes = [ctypes.c_int]
    L.pagedkv_status_string.restype = ctypes.c_char_p
    L.pagedkv_version.argtypes = []
    L.pagedkv_version.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().pagedkv_status_string(int(status)).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise PagedKVError(rc, what)


FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _dev(t: torch.Tensor, name: str, dtype) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    allowed = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in allowed:
        raise TypeError(f"{name} must be {' or '.join(map(str, allowed))}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _append_args(k, v, slot_mapping, key_cache, value_cache, cache_dtype):
    pk = _dev(k, "k", torch.bfloat16)
    pv = _dev(v, "v", torch.bfloat16)
    ps = _dev(slot_mapping, "slot_mapping", torch.int64)
    pkc = _dev(key_cache, "key_cache", cache_dtype)
    pvc = _dev(value_cache, "value_cache", cache_dtype)
    if k.dim() != 3 or v.shape != k.shape:
        raise ValueError("k and v must both be [T, K, H]")
    T, K, H = k.shape
    if key_cache.dim() != 4:
        raise ValueError("key_cache must be [num_blocks, K, block_size, H]")
    nb, K2, bs, H2 = key_cache.shape
    if (K2, H2) != (K, H) or value_cache.shape != (nb, K, H, bs):
        raise ValueError("cache shapes do not match k/v ([nb,K,bs,H] and [nb,K,H,bs])")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    return (pk, pv, ps, pkc, pvc), (T, K, H, bs, nb)


def paged_kv_append(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                    key_cache: torch.Tensor, value_cache: torch.Tensor) -> None:
    """Write k[i], v[i] ([T, K, H] bf16) at slot slot_mapping[i] of the caches."""
    ptrs, sizes = _append_args(k, v, slot_mapping, key_cache, value_cache, torch.bfloat16)
    _check(lib().paged_kv_append(*ptrs, *sizes, _stream(k.device)), "paged_kv_append")


def paged_kv_append_fp8(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                        key_cache: torch.Tensor, value_cache: torch.Tensor, k_scale: float,
                        v_scale: float) -> None:
    """Quantise k[i], v[i] ([T, K, H] bf16) into FP8 E4M3 pools (uint8 or
    float8_e4m3fn) at slot slot_mapping[i]; code c in a pool stands for
    e4m3(c) * that pool's scale."""
    ptrs, sizes = _append_args(k, v, slot_mapping, key_cache, value_cache, FP8_DTYPES)
    _check(lib().paged_kv_append_fp8(*ptrs, float(k_scale), float(v_scale), *sizes,
                                     _stream(k.device)), "paged_kv_append_fp8")


def workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                   max_context_len: int, partition: int = 0) -> int:
    return int(lib().paged_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                 max_context_len, partition))


def _decode_args(out, q, key_cache, value_cache, block_tables, context_lens, num_kv_heads,
                 block_size, max_context_len, partition, workspace, cache_dtype,
                 allocate=True):
    po = _dev(out, "out", torch.float32)
    pq = _dev(q, "q", torch.bfloat16)
    pkc = _dev(key_cache, "key_cache", cache_dtype)
    pvc = _dev(value_cache, "value_cache", cache_dtype)
    pbt = _dev(block_tables, "block_tables", torch.int32)
    pcl = _dev(context_lens, "context_lens", torch.int32)
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must both be [B, N, H]")
    B, N, H = q.shape
    if key_cache.dim() != 4:
        raise ValueError("key_cache must be [num_blocks, K, block_size, H]")
    nb, K, bs, H2 = key_cache.shape
    if K != num_kv_heads or bs != block_size or H2 != H or value_cache.shape != (nb, K, H, bs):
        raise ValueError("cache shapes disagree with num_kv_heads / block_size / head_dim")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * block_size
    # the size is only needed to allocate one (the library checks a given one)
    need = (workspace_size(B, N, K, H, max_context_len, partition)
            if B and allocate and workspace is None else 0)
    if need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    pw, wbytes = 0, 0
    if workspace is not None:
        pw = _dev(workspace, "workspace", torch.uint8)
        wbytes = workspace.numel()
    head = (po, pq, pkc, pvc, pbt, pcl)
    tail = (K, bs, B, N, H, max_blocks, int(max_context_len), nb, int(partition), pw, wbytes,
            _stream(q.device))
    return head, tail


def paged_decode_attention(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                           value_cache: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, scale: float, num_kv_heads: int,
                           block_size: int, max_context_len: Optional[int] = None,
                           partition: int = 0,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[b, n] = softmax(scale * q[b, n] . K_b^T) V_b over the paged cache.

    ``max_context_len`` is a host-known bound of ``context_lens``; by default
    the block-table capacity (max_blocks * block_size).  ``partition`` 0 uses
    the token-balanced schedule, P > 0 fixed P-token partitions.
    ``workspace`` (uint8, on the GPU) is allocated here when not given and the
    call needs one.  Returns ``out``.
    """
    head, tail = _decode_args(out, q, key_cache, value_cache, block_tables, context_lens,
                              num_kv_heads, block_size, max_context_len, partition, workspace,
                              torch.bfloat16)
    _check(lib().paged_decode_attention(*head, float(scale), *tail), "paged_decode_attention")
    return out


def paged_decode_attention_noalloc(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                                   value_cache: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, scale: float, num_kv_heads: int,
                                   block_size: int, max_context_len: Optional[int] = None,
                                   partition: int = 0) -> torch.Tensor:
    """``paged_decode_attention`` with no workspace: the library's static
    per-device scratch array serves instead, so neither the library nor this
    wrapper allocates device memory (for graph capture and callers that
    cannot allocate).  Calls that may overlap on one device race."""
    head, tail = _decode_args(out, q, key_cache, value_cache, block_tables, context_lens,
                              num_kv_heads, block_size, max_context_len, partition, None,
                              torch.bfloat16, allocate=False)
    _check(lib().paged_decode_attention_noalloc(*head, float(scale), *tail[:-3], tail[-1]),
           "paged_decode_attention_noalloc")
    return out


def paged_decode_attention_fp8(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                               value_cache: torch.Tensor, block_tables: torch.Tensor,
                               context_lens: torch.Tensor, scale: float, k_scale: float,
                               v_scale: float, num_kv_heads: int, block_size: int,
                               max_context_len: Optional[int] = None, partition: int = 0,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``paged_decode_attention`` over FP8 E4M3 pools (uint8 or float8_e4m3fn),
    keys being codes times ``k_scale`` and values codes times ``v_scale``."""
    head, tail = _decode_args(out, q, key_cache, value_cache, block_tables, context_lens,
                              num_kv_heads, block_size, max_context_len, partition, workspace,
                              FP8_DTYPES)
    _check(lib().paged_decode_attention_fp8(*head, float(scale), float(k_scale), float(v_scale),
                                            *tail), "paged_decode_attention_fp8")
    return out


KV_BF16, KV_FP8_E4M3 = 0, 1


def prefix_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                          max_context_len: int, partition: int, max_prefix_tokens: int) -> int:
    return int(lib().paged_decode_prefix_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                        head_dim, max_context_len, partition,
                                                        max_prefix_tokens))


def mq_workspace_size(num_seqs: int, num_queries: int, num_heads: int, head_dim: int,
                      max_context_len: int, partition: int) -> int:
    return int(lib().paged_decode_mq_workspace_size(num_seqs, num_queries, num_heads, head_dim,
                                                    max_context_len, partition))


def paged_decode_attention_mq(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                              value_cache: torch.Tensor, block_tables: torch.Tensor,
                              context_lens: torch.Tensor, scale: float, num_kv_heads: int,
                              block_size: int, partition: int, k_scale: float = 1.0,
                              v_scale: float = 1.0, max_context_len: Optional[int] = None,
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Q query tokens per sequence (q, out [B, Q, N, H]): token i of sequence b
    attends positions 0 .. ctx_b - Q + i.  bf16 pools, or FP8 E4M3 pools
    (uint8 / float8_e4m3fn) with ``k_scale``, ``v_scale``.  ``partition`` is
    the fixed split size (a multiple of 32 in [32, 1024])."""
    po = _dev(out, "out", torch.float32)
    pq = _dev(q, "q", torch.bfloat16)
    fp8 = key_cache.dtype in FP8_DTYPES
    pool = FP8_DTYPES if fp8 else torch.bfloat16
    pkc = _dev(key_cache, "key_cache", pool)
    pvc = _dev(value_cache, "value_cache", pool)
    pbt = _dev(block_tables, "block_tables", torch.int32)
    pcl = _dev(context_lens, "context_lens", torch.int32)
    if q.dim() != 4 or out.shape != q.shape:
        raise ValueError("q and out must both be [B, Q, N, H]")
    B, Q, N, H = q.shape
    if key_cache.dim() != 4:
        raise ValueError("key_cache must be [num_blocks, K, block_size, H]")
    nb, K, bs, H2 = key_cache.shape
    if K != num_kv_heads or bs != block_size or H2 != H or value_cache.shape != (nb, K, H, bs):
        raise ValueError("cache shapes disagree with num_kv_heads / block_size / head_dim")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * block_size
    need = mq_workspace_size(B, Q, N, H, max_context_len, partition) if B and workspace is None else 0
    if need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    pw, wbytes = 0, 0
    if workspace is not None:
        pw = _dev(workspace, "workspace", torch.uint8)
        wbytes = workspace.numel()
    _check(lib().paged_decode_attention_mq(
        po, pq, pkc, pvc, pbt, pcl, float(scale), KV_FP8_E4M3 if fp8 else KV_BF16,
        float(k_scale), float(v_scale), K, bs, B, Q, N, H, max_blocks, int(max_context_len),
        nb, int(partition), pw, wbytes, _stream(q.device)), "paged_decode_attention_mq")
    return out


def paged_decode_attention_prefix(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                                  value_cache: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, scale: float, num_kv_heads: int,
                                  block_size: int, partition: int, seq_group: torch.Tensor,
                                  group_members: torch.Tensor, prefix_tokens: torch.Tensor,
                                  max_prefix_tokens: Optional[int] = None,
                                  k_scale: float = 1.0, v_scale: float = 1.0,
                                  max_context_len: Optional[int] = None,
                                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``paged_decode_attention`` that reads each shared prefix once for all
    its sharers (in ``partition``-token pieces) and the rest of every context
    on the token-balanced schedule.  seq_group [B] int32 (-1 = none),
    group_members [num_groups, max_members] int32 (-1 padded, lead first),
    prefix_tokens [num_groups] int32; ``max_prefix_tokens`` is a host bound of
    prefix_tokens (default: the block-table capacity)."""
    if max_prefix_tokens is None:
        max_prefix_tokens = block_tables.shape[1] * block_size
    if workspace is None and q.shape[0]:
        mcl = block_tables.shape[1] * block_size if max_context_len is None else max_context_len
        need = prefix_workspace_size(q.shape[0], q.shape[1], num_kv_heads, q.shape[2], mcl,
                                     partition, max_prefix_tokens)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    head, tail = _decode_args(out, q, key_cache, value_cache, block_tables, context_lens,
                              num_kv_heads, block_size, max_context_len, partition, workspace,
                              FP8_DTYPES if key_cache.dtype in FP8_DTYPES else torch.bfloat16)
    fp8 = key_cache.dtype in FP8_DTYPES
    psg = _dev(seq_group, "seq_group", torch.int32)
    if group_members.dim() != 2 or prefix_tokens.shape != (group_members.shape[0],):
        raise ValueError("group_members must be [num_groups, max_members] and prefix_tokens "
                         "[num_groups]")
    pgm = _dev(group_members, "group_members", torch.int32)
    ppt = _dev(prefix_tokens, "prefix_tokens", torch.int32)
    if seq_group.shape != (q.shape[0],):
        raise ValueError("seq_group must be [B]")
    num_groups, max_members = group_members.shape
    K, bs, B, N, H, max_blocks, mcl, nb, part, pw, wbytes, stream = tail
    _check(lib().paged_decode_attention_prefix(
        *head, float(scale), KV_FP8_E4M3 if fp8 else KV_BF16, float(k_scale), float(v_scale),
        K, bs, B, N, H, max_blocks, mcl, nb, part, psg, pgm, ppt, num_groups, max_members,
        int(max_prefix_tokens), pw, wbytes, stream), "paged_decode_attention_prefix")
    return out


def paged_decode_attention_window(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                                  value_cache: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, scale: float, num_kv_heads: int,
                                  block_size: int, window: int, k_scale: float = 1.0,
                                  v_scale: float = 1.0, max_context_len: Optional[int] = None,
                                  partition: int = 0,
                                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sliding-window decode: each query attends the last ``window`` positions
    of its sequence (the new token included); bf16 or FP8 pools."""
    fp8 = key_cache.dtype in FP8_DTYPES
    head, tail = _decode_args(out, q, key_cache, value_cache, block_tables, context_lens,
                              num_kv_heads, block_size, max_context_len, partition, workspace,
                              FP8_DTYPES if fp8 else torch.bfloat16)
    _check(lib().paged_decode_attention_window(
        *head, float(scale), KV_FP8_E4M3 if fp8 else KV_BF16, float(k_scale), float(v_scale),
        int(window), *tail), "paged_decode_attention_window")
    return out


def paged_kv_copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor,
                         src_blocks: torch.Tensor, dst_blocks: torch.Tensor) -> None:
    """Copy-on-write split: block dst_blocks[i] becomes a bit copy of block
    src_blocks[i] (every head of both pools; bf16 or FP8 pools).  No block may
    appear in two pairs."""
    fp8 = key_cache.dtype in FP8_DTYPES
    pool = FP8_DTYPES if fp8 else torch.bfloat16
    pkc = _dev(key_cache, "key_cache", pool)
    pvc = _dev(value_cache, "value_cache", pool)
    ps = _dev(src_blocks, "src_blocks", torch.int32)
    pd = _dev(dst_blocks, "dst_blocks", torch.int32)
    if src_blocks.shape != dst_blocks.shape or src_blocks.dim() != 1:
        raise ValueError("src_blocks and dst_blocks must both be [num_pairs]")
    nb, K, bs, H = key_cache.shape
    if value_cache.shape != (nb, K, H, bs):
        raise ValueError("cache shapes disagree ([nb,K,bs,H] and [nb,K,H,bs])")
    _check(lib().paged_kv_copy_blocks(pkc, pvc, ps, pd, src_blocks.shape[0], K, H, bs, nb,
                                      KV_FP8_E4M3 if fp8 else KV_BF16,
                                      _stream(key_cache.device)), "paged_kv_copy_blocks")


def stream_read(src: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Measurement helper: read ``src`` once with 16-byte loads (no result)."""
    nbytes = src.numel() * src.element_size()
    if not (src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous GPU tensor")
    need = int(lib().pagedkv_stream_read_sink_bytes(nbytes))
    if sink is None:
        sink = torch.empty(need, dtype=torch.uint8, device=src.device)
    if sink.numel() * sink.element_size() < need:
        raise ValueError("sink too small")
    _check(lib().pagedkv_stream_read(src.data_ptr(), nbytes, sink.data_ptr(),
                                     _stream(src.device)), "pagedkv_stream_read")
    return sink


def stream_copy(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Measurement helper: copy ``src`` into ``dst`` with 16-byte accesses."""
    nbytes = src.numel() * src.element_size()
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous GPU tensors")
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check(lib().pagedkv_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                     _stream(src.device)), "pagedkv_stream_copy")
    return dst


def version() -> str:
    v = lib().pagedkv_version()
    return f"{v >> 16}.{v & 0xFFFF}"
