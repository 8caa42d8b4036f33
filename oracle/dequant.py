"""Dequantization of integer codes to bf16 (oracle; test infrastructure only).

EntroLLM runs its models on the uint8/uint4 codes, which implies mapping a
code back to a real weight with the tensor's scale and zero point
(gist.science technical summary, Methodology item 1 and Experimental results;
EntroLLM abstract v4 on shd-paper.top).  The output precision is not on the
pages; reading: one IEEE float32 product, then round to nearest even to bf16.

    v  = f32(q - zp)            exact: |q - zp| < 2^8
    p  = f32(scale) * v         one float32 multiply, round to nearest even
    bf = RNE_bf16(p)            u = bits(p); u += 0x7FFF + ((u >> 16) & 1); u >>= 16
"""
from __future__ import annotations

import numpy as np


def dequant_f32(q: np.ndarray, scale: float, zero_point: int) -> np.ndarray:
    """``f32(scale) * f32(q - zp)`` as float32 (a single rounded product)."""
    v = (np.asarray(q, dtype=np.int64) - int(zero_point)).astype(np.float32)
    return np.float32(scale) * v


def f32_to_bf16_rne(p: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.asarray(p, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def dequant_bf16(q: np.ndarray, scale: float, zero_point: int) -> np.ndarray:
    """bf16 bits (uint16) of every code, same shape as ``q``."""
    return f32_to_bf16_rne(dequant_f32(q, scale, zero_point))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
