"""CPU reference ("oracle") for paged-KV decode attention and append.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library under ``paged_kv_cache_100_amd`` and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
output rows), compiled with gcc into ``liboracle.so`` next to it.  This module
only marshals numpy arrays into that library.  ``brute.py`` holds a second,
pure-Python statement of the same definition for tiny inputs, and the
KV-cache size formula is ``kv_cache_bytes`` below (also computed in C).

bf16 tensors cross this boundary as ``numpy.uint16`` arrays of raw bit
patterns, so no rounding happens on the way in.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
facts printed on the pages (``tests/golden/``), closed forms, the pure-Python
brute force, a library attention routine (torch CPU float64) and invariants,
and a mutation test shows that each plausible slip in ``oracle.c`` fails at
least one of those checks.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``src`` with gcc (-O2, OpenMP) into the shared library ``out``."""
    stale = not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src)
    if force or stale:
        tmp = out + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                        "-Wall", "-Wextra", "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


def load_library(path: str) -> ctypes.CDLL:
    """Open a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.oracle_append.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i64]
    lib.oracle_append.restype = i32
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, f32,
                                  i32, i32, i32, i32, i32, i32, i64, P, i32]
    lib.oracle_decode.restype = i32
    lib.oracle_decode_rows.argtypes = [P, P, P, i32, P, P, P, P, P, f32,
                                       i32, i32, i32, i32, i32, i32, i64, P, i32]
    lib.oracle_decode_rows.restype = i32
    lib.oracle_decode_split.argtypes = [P, P, P, P, P, P, f32,
                                        i32, i32, i32, i32, i32, i32, i64, i32,
                                        P, P, P, i32]
    lib.oracle_decode_split.restype = i32
    lib.oracle_kv_cache_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.oracle_kv_cache_bytes.restype = i64
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_quantize.argtypes = [ctypes.c_uint16, f32]
    lib.oracle_e4m3_quantize.restype = ctypes.c_uint8
    lib.oracle_append_fp8.argtypes = [P, P, P, P, P, f32, f32, i32, i32, i32, i32, i64]
    lib.oracle_append_fp8.restype = i32
    lib.oracle_decode_fp8.argtypes = [P, P, P, P, f32, f32, P, P, f32,
                                      i32, i32, i32, i32, i32, i32, i64, P, i32]
    lib.oracle_decode_fp8.restype = i32
    lib.oracle_decode_rows_fp8.argtypes = [P, P, P, i32, P, P, P, f32, f32, P, P, f32,
                                           i32, i32, i32, i32, i32, i32, i64, P, i32]
    lib.oracle_decode_rows_fp8.restype = i32
    lib.oracle_decode_multi.argtypes = [P, P, P, P, i32, f32, f32, P, P, f32,
                                        i32, i32, i32, i32, i32, i32, i32, i64, P, i32]
    lib.oracle_decode_multi.restype = i32
    lib.oracle_decode_multi_rows.argtypes = [P, P, P, P, i32, P, P, P, i32, f32, f32, P, P, f32,
                                             i32, i32, i32, i32, i32, i32, i32, i64, P, i32]
    lib.oracle_decode_multi_rows.restype = i32
    lib.oracle_copy_blocks.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i64]
    lib.oracle_copy_blocks.restype = i32
    lib.oracle_decode_window.argtypes = [P, P, P, P, i32, f32, f32, P, P, f32, i32,
                                         i32, i32, i32, i32, i32, i32, i64, P, i32]
    lib.oracle_decode_window.restype = i32
    return lib


_default_lib = None


def _load():
    global _default_lib
    if _default_lib is None:
        _default_lib = load_library(build())
    return _default_lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def num_threads() -> int:
    """Threads the OpenMP loops use (OMP_NUM_THREADS, else the affinity set)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def append(k, v, slot_mapping, key_cache, value_cache, lib=None) -> None:
    """Bit copy of new K/V rows into the paged pools, in place.

    k, v: uint16 [T, K, H]; slot_mapping: int64 [T] (negative = skip);
    key_cache: uint16 [num_blocks, K, bs, H]; value_cache: uint16
    [num_blocks, K, H, bs].  Raises ValueError on a slot outside the pool.
    """
    k = _as(k, np.uint16)
    v = _as(v, np.uint16)
    slot_mapping = _as(slot_mapping, np.int64)
    if not (key_cache.flags.c_contiguous and value_cache.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous (written in place)")
    if key_cache.dtype != np.uint16 or value_cache.dtype != np.uint16:
        raise TypeError("caches must be uint16 bit patterns")
    T, K, H = k.shape
    nb, K2, bs, H2 = key_cache.shape
    if (K2, H2) != (K, H) or value_cache.shape != (nb, K, H, bs) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must have one entry per token")
    rc = (lib or _load()).oracle_append(_ptr(k), _ptr(v), _ptr(slot_mapping),
                                        _ptr(key_cache), _ptr(value_cache), T, K, H, bs, nb)
    if rc:
        raise ValueError("slot outside the pool")


def _decode_args(q, key_cache, value_cache, block_tables, context_lens, cache_dtype=np.uint16):
    q = _as(q, np.uint16)
    key_cache = _as(key_cache, cache_dtype)
    value_cache = _as(value_cache, cache_dtype)
    block_tables = _as(block_tables, np.int32)
    context_lens = _as(context_lens, np.int32)
    B, N, H = q.shape
    nb, K, bs, H2 = key_cache.shape
    if H2 != H or value_cache.shape != (nb, K, H, bs):
        raise ValueError("cache shape mismatch")
    if block_tables.ndim != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("table shape mismatch")
    return q, key_cache, value_cache, block_tables, context_lens, (B, N, H, nb, K, bs)


def _scratch(context_lens):
    stride = max(1, int(context_lens.max()) if context_lens.size else 1)
    return np.empty((num_threads() + 1) * stride, np.float64), stride


def decode(q, key_cache, value_cache, block_tables, context_lens, scale,
           lib=None) -> np.ndarray:
    """softmax(q K^T * scale) V per (sequence, query head), float64 [B, N, H].

    ``scale`` is an fp32 value (the library receives fp32); it is widened to
    double exactly.  A sequence with context length 0 yields zeros.
    """
    q, kc, vc, bt, cl, (B, N, H, nb, K, bs) = _decode_args(
        q, key_cache, value_cache, block_tables, context_lens)
    out = np.zeros((B, N, H), np.float64)
    scratch, stride = _scratch(cl)
    rc = (lib or _load()).oracle_decode(
        _ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(cl), float(np.float32(scale)),
        B, N, K, H, bs, bt.shape[1], nb, _ptr(scratch), stride)
    if rc:
        raise ValueError("invalid decode arguments (block id, shape or context)")
    return out


def decode_rows(rows_b, rows_n, q, key_cache, value_cache, block_tables, context_lens,
                scale, lib=None) -> np.ndarray:
    """Rows (rows_b[r], rows_n[r]) of ``decode`` only, float64 [R, H]."""
    q, kc, vc, bt, cl, (B, N, H, nb, K, bs) = _decode_args(
        q, key_cache, value_cache, block_tables, context_lens)
    rb = _as(rows_b, np.int32)
    rn = _as(rows_n, np.int32)
    R = rb.shape[0]
    out = np.zeros((R, H), np.float64)
    scratch, stride = _scratch(cl)
    rc = (lib or _load()).oracle_decode_rows(
        _ptr(out), _ptr(rb), _ptr(rn), R, _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(cl),
        float(np.float32(scale)), B, N, K, H, bs, bt.shape[1], nb, _ptr(scratch), stride)
    if rc:
        raise ValueError("invalid decode arguments (row, block id, shape or context)")
    return out


def decode_split(q, key_cache, value_cache, block_tables, context_lens, scale,
                 part: int, lib=None) -> np.ndarray:
    """``decode`` computed piecewise over ``part``-token pieces + log-sum-exp merge."""
    q, kc, vc, bt, cl, (B, N, H, nb, K, bs) = _decode_args(
        q, key_cache, value_cache, block_tables, context_lens)
    out = np.zeros((B, N, H), np.float64)
    max_pieces = max(1, -(-int(cl.max()) // part) if B else 1)
    pm = np.empty(max_pieces, np.float64)
    pl = np.empty(max_pieces, np.float64)
    po = np.empty((max_pieces, H), np.float64)
    rc = (lib or _load()).oracle_decode_split(
        _ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(cl), float(np.float32(scale)),
        B, N, K, H, bs, bt.shape[1], nb, part, _ptr(pm), _ptr(pl), _ptr(po), max_pieces)
    if rc:
        raise ValueError("invalid decode arguments")
    return out


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int,
                   bytes_per_value: int = 2, lib=None) -> int:
    """2 * L * K * H * S * bytes (KV-cache size formula), computed by the C oracle."""
    return int((lib or _load()).oracle_kv_cache_bytes(layers, kv_heads, head_dim, tokens,
                                                      bytes_per_value))


# ---------------------------------------------------------------- FP8 ----
# OCP FP8 E4M3 pools: uint8 codes; a code c stands for e4m3_value(c) * scale.

def fp32_inverse(scale: float) -> float:
    """1/scale rounded to fp32 (the inverse the append multiplies by)."""
    return float(np.float32(1.0) / np.float32(scale))


def e4m3_value(code: int, lib=None) -> float:
    """Exact value of an E4M3 code (NaN for 0x7F / 0xFF)."""
    return float((lib or _load()).oracle_e4m3_value(int(code) & 0xFF))


def e4m3_quantize(bits: int, inv_scale: float, lib=None) -> int:
    """Code stored for the bf16 value with these bits, given the fp32 inverse scale."""
    return int((lib or _load()).oracle_e4m3_quantize(int(bits) & 0xFFFF, float(inv_scale)))


def append_fp8(k, v, slot_mapping, key_cache, value_cache, k_scale, v_scale, lib=None) -> None:
    """Quantise new K/V rows (bf16 bits) into FP8 pools (uint8 codes), in place."""
    k = _as(k, np.uint16)
    v = _as(v, np.uint16)
    slot_mapping = _as(slot_mapping, np.int64)
    if not (key_cache.flags.c_contiguous and value_cache.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous (written in place)")
    if key_cache.dtype != np.uint8 or value_cache.dtype != np.uint8:
        raise TypeError("FP8 caches must be uint8 codes")
    T, K, H = k.shape
    nb, K2, bs, H2 = key_cache.shape
    if (K2, H2) != (K, H) or value_cache.shape != (nb, K, H, bs) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    rc = (lib or _load()).oracle_append_fp8(
        _ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(key_cache), _ptr(value_cache),
        fp32_inverse(k_scale), fp32_inverse(v_scale), T, K, H, bs, nb)
    if rc:
        raise ValueError("slot outside the pool")


def decode_fp8(q, key_cache, value_cache, block_tables, context_lens, scale, k_scale, v_scale,
               lib=None) -> np.ndarray:
    """``decode`` over FP8 pools, float64 [B, N, H]."""
    q, kc, vc, bt, cl, (B, N, H, nb, K, bs) = _decode_args(
        q, key_cache, value_cache, block_tables, context_lens, np.uint8)
    out = np.zeros((B, N, H), np.float64)
    scratch, stride = _scratch(cl)
    rc = (lib or _load()).oracle_decode_fp8(
        _ptr(out), _ptr(q), _ptr(kc), _ptr(vc), float(np.float32(k_scale)),
        float(np.float32(v_scale)), _ptr(bt), _ptr(cl), float(np.float32(scale)),
        B, N, K, H, bs, bt.shape[1], nb, _ptr(scratch), stride)
    if rc:
        raise ValueError("invalid decode arguments (block id, shape or context)")
    return out


def decode_rows_fp8(rows_b, rows_n, q, key_cache, value_cache, block_tables, context_lens,
                    scale, k_scale, v_scale, lib=None) -> np.ndarray:
    """Rows (rows_b[r], rows_n[r]) of ``decode_fp8`` only, float64 [R, H]."""
    q, kc, vc, bt, cl, (B, N, H, nb, K, bs) = _decode_args(
        q, key_cache, value_cache, block_tables, context_lens, np.uint8)
    rb = _as(rows_b, np.int32)
    rn = _as(rows_n, np.int32)
    R = rb.shape[0]
    out = np.zeros((R, H), np.float64)
    scratch, stride = _scratch(cl)
    rc = (lib or _load()).oracle_decode_rows_fp8(
        _ptr(out), _ptr(rb), _ptr(rn), R, _ptr(q), _ptr(kc), _ptr(vc),
        float(np.float32(k_scale)), float(np.float32(v_scale)), _ptr(bt), _ptr(cl),
        float(np.float32(scale)), B, N, K, H, bs, bt.shape[1], nb, _ptr(scratch), stride)
    if rc:
        raise ValueError("invalid decode arguments (row, block id, shape or context)")
    return out


# ------------------------------------------------------- multi-query ----
# Q query tokens per sequence (speculative verification): q, out [B, Q, N, H];
# query i sees positions 0 .. ctx - Q + i (bottom-right causal mask).

_KV_DTYPES = {np.dtype(np.uint16): 0, np.dtype(np.uint8): 1}


def _multi_args(q, key_cache, value_cache, block_tables, context_lens):
    q = _as(q, np.uint16)
    if q.ndim != 4:
        raise ValueError("q must be [B, Q, N, H]")
    B, Q, N, H = q.shape
    kc = np.ascontiguousarray(key_cache)
    if kc.dtype not in _KV_DTYPES:
        raise TypeError("pools must be uint16 (bf16 bits) or uint8 (E4M3 codes)")
    _, kc, vc, bt, cl, (_, _, _, nb, K, bs) = _decode_args(
        q.reshape(B, Q * N, H), kc, value_cache, block_tables, context_lens, kc.dtype.type)
    return q, kc, vc, bt, cl, (B, Q, N, H, nb, K, bs), _KV_DTYPES[kc.dtype]


def decode_multi(q, key_cache, value_cache, block_tables, context_lens, scale,
                 k_scale: float = 1.0, v_scale: float = 1.0, lib=None) -> np.ndarray:
    """Q query tokens per sequence over bf16 or FP8 pools, float64 [B, Q, N, H]."""
    q, kc, vc, bt, cl, (B, Q, N, H, nb, K, bs), dt = _multi_args(
        q, key_cache, value_cache, block_tables, context_lens)
    out = np.zeros((B, Q, N, H), np.float64)
    scratch, stride = _scratch(cl)
    rc = (lib or _load()).oracle_decode_multi(
        _ptr(out), _ptr(q), _ptr(kc), _ptr(vc), dt, float(np.float32(k_scale)),
        float(np.float32(v_scale)), _ptr(bt), _ptr(cl), float(np.float32(scale)),
        B, Q, N, K, H, bs, bt.shape[1], nb, _ptr(scratch), stride)
    if rc:
        raise ValueError("invalid decode arguments (block id, shape or context)")
    return out


def decode_multi_rows(rows_b, rows_i, rows_n, q, key_cache, value_cache, block_tables,
                      context_lens, scale, k_scale: float = 1.0, v_scale: float = 1.0,
                      lib=None) -> np.ndarray:
    """Rows (rows_b[r], rows_i[r], rows_n[r]) of ``decode_multi`` only, float64 [R, H]."""
    q, kc, vc, bt, cl, (B, Q, N, H, nb, K, bs), dt = _multi_args(
        q, key_cache, value_cache, block_tables, context_lens)
    rb, ri, rn = _as(rows_b, np.int32), _as(rows_i, np.int32), _as(rows_n, np.int32)
    R = rb.shape[0]
    out = np.zeros((R, H), np.float64)
    scratch, stride = _scratch(cl)
    rc = (lib or _load()).oracle_decode_multi_rows(
        _ptr(out), _ptr(rb), _ptr(ri), _ptr(rn), R, _ptr(q), _ptr(kc), _ptr(vc), dt,
        float(np.float32(k_scale)), float(np.float32(v_scale)), _ptr(bt), _ptr(cl),
        float(np.float32(scale)), B, Q, N, K, H, bs, bt.shape[1], nb, _ptr(scratch), stride)
    if rc:
        raise ValueError("invalid decode arguments (row, block id, shape or context)")
    return out


# ------------------------------------------------------- block copy ----

def copy_blocks(key_cache, value_cache, src, dst, lib=None) -> None:
    """Copy whole physical blocks src[i] -> dst[i] (all heads, both pools), in
    place and in pair order; bf16 (uint16) or E4M3 (uint8) pools."""
    if not (key_cache.flags.c_contiguous and value_cache.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous (written in place)")
    if key_cache.dtype != value_cache.dtype or key_cache.dtype not in (np.uint16, np.uint8):
        raise TypeError("pools must both be uint16 (bf16 bits) or uint8 (E4M3 codes)")
    nb, K, bs, H = key_cache.shape
    if value_cache.shape != (nb, K, H, bs):
        raise ValueError("shape mismatch")
    src = _as(src, np.int32)
    dst = _as(dst, np.int32)
    if src.shape != dst.shape:
        raise ValueError("src and dst differ in length")
    rc = (lib or _load()).oracle_copy_blocks(
        _ptr(key_cache), _ptr(value_cache), _ptr(src), _ptr(dst), src.shape[0], K, H, bs,
        key_cache.dtype.itemsize, nb)
    if rc:
        raise ValueError("block id outside the pool")


# ---------------------------------------------------- sliding window ----

def decode_window(q, key_cache, value_cache, block_tables, context_lens, scale, window: int,
                  k_scale: float = 1.0, v_scale: float = 1.0, lib=None) -> np.ndarray:
    """Each sequence's query attends its last ``window`` positions only
    (positions max(0, ctx - window) .. ctx - 1); bf16 or FP8 pools;
    float64 [B, N, H]."""
    kc = np.ascontiguousarray(key_cache)
    if kc.dtype not in _KV_DTYPES:
        raise TypeError("pools must be uint16 (bf16 bits) or uint8 (E4M3 codes)")
    q, kc, vc, bt, cl, (B, N, H, nb, K, bs) = _decode_args(
        q, kc, value_cache, block_tables, context_lens, kc.dtype.type)
    out = np.zeros((B, N, H), np.float64)
    scratch, stride = _scratch(cl)
    rc = (lib or _load()).oracle_decode_window(
        _ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _KV_DTYPES[kc.dtype], float(np.float32(k_scale)),
        float(np.float32(v_scale)), _ptr(bt), _ptr(cl), float(np.float32(scale)), int(window),
        B, N, K, H, bs, bt.shape[1], nb, _ptr(scratch), stride)
    if rc:
        raise ValueError("invalid decode arguments (window, block id, shape or context)")
    return out
