"""Small conversions shared by the tests (no attention arithmetic here)."""
import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 array of its bit patterns (copy, CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bits(x) -> np.ndarray:
    """float values (exactly representable in bf16) -> uint16 bit patterns."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not exactly representable in bf16")
    return (u >> 16).astype(np.uint16)


def pool_bits(t: torch.Tensor) -> np.ndarray:
    """A KV pool as the oracle takes it: uint16 bf16 bits, or uint8 FP8 codes."""
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.detach().cpu().contiguous().view(torch.uint8).numpy().copy()
    return bits(t)


def oracle_inputs(w):
    """numpy views of a workload's decode inputs in the oracle's types."""
    return dict(q=bits(w.q), key_cache=pool_bits(w.key_cache),
                value_cache=pool_bits(w.value_cache),
                block_tables=w.block_tables.numpy().astype(np.int32),
                context_lens=w.context_lens.numpy().astype(np.int32))
