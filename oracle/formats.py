"""Exact widening of stored numbers to float64 (oracle side).

bf16 and fp16 values widen exactly to float64; a 4-bit KV value is
``d * (n - 8)`` with ``d`` the block's fp16 scale and ``n`` the 4-bit code,
which float64 holds exactly.  The 4-bit cache is the one the single-RTX-3090
DFlash note keeps for 128K of context (section "128K context in 24 GB"); the
pages name the format but do not spell it out, so the block layout read here
is: 32 consecutive head-dim values per block, one fp16 scale per block, code
of value 2t in the low nibble of byte t and of value 2t+1 in the high nibble.
"""
import numpy as np


def widen_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def widen_fp16(bits: np.ndarray) -> np.ndarray:
    """uint16 IEEE-half bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def q4_decode(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """4-bit rows -> float64 values.

    ``codes``: uint8 ``[..., D/2]``; ``scale_bits``: uint16 ``[..., D/32]``.
    Value i of a row is ``scale[i // 32] * (code_i - 8)``.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    lo = (codes & 0x0F).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    n = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.int64)
    n[..., 0::2] = lo
    n[..., 1::2] = hi
    d = widen_fp16(scale_bits)
    d_per_value = np.repeat(d, 32, axis=-1)
    return d_per_value * (n - 8).astype(np.float64)


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return widen_f32(x)
    if dtype == "bf16":
        return widen_bf16(x)
    raise ValueError(dtype)
