"""Per-tensor quantizers of the oracle (test infrastructure only).

EntroLLM quantizes each weight tensor as a whole ("tensor-level") and picks,
per layer, between two schemes, which the pages name unsigned and asymmetric
(EntroLLM abstract v4 on shd-paper.top; gist.science technical summary,
Methodology item 1).  The earlier abstract (papers.pytorch.kr) calls the pair
symmetric and asymmetric and says the choice is made from the layer's weight
distribution to optimize compressibility.

The pages give no formulas.  Readings used here:

* asymmetric: min-max affine.  ``s = f32((max - min) / Q)``,
  ``zp = clamp(rint(-min / s), 0, Q)``, ``q = clamp(rint(w / s) + zp, 0, Q)``.
* unsigned: a symmetric range stored as unsigned codes.
  ``s = f32(m / (2^(b-1) - 1))`` with ``m = max|w|`` (or a clip value),
  ``zp = 2^(b-1)``, ``q = clamp(rint(w / s) + zp, 0, Q)``.
* mixed selection: quantize both ways and keep the scheme whose codes have
  the lower empirical entropy; ties go to asymmetric.
* arithmetic in float64 on the float32 weights; the scale is rounded to
  float32 and that float32 value is used everywhere after; ``rint`` rounds
  half to even.
* degenerate tensors (max == min, or m == 0): ``s = 1``, zp as above.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Quantized:
    q: np.ndarray        # uint8 codes, same shape as the weight
    scale: np.float32
    zero_point: int
    scheme: str          # "asymmetric" | "unsigned"
    bits: int


def quantize_asymmetric(w: np.ndarray, bits: int) -> Quantized:
    """Min-max affine quantization of a whole tensor to ``bits``-bit codes."""
    Q = (1 << bits) - 1
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    lo = float(w64.min())
    hi = float(w64.max())
    if hi == lo:
        s = np.float32(1.0)
        zp = 0
    else:
        s = np.float32((hi - lo) / Q)
        zp = int(np.clip(np.rint(-lo / float(s)), 0, Q))
    q = np.clip(np.rint(w64 / float(s)) + zp, 0, Q).astype(np.uint8)
    return Quantized(q, s, zp, "asymmetric", bits)


def quantize_unsigned(w: np.ndarray, bits: int, clip: float | None = None) -> Quantized:
    """Symmetric-range quantization stored as unsigned codes (zero point 2^(b-1)).

    ``clip`` replaces ``max|w|`` as the range end when given.
    """
    Q = (1 << bits) - 1
    half = 1 << (bits - 1)
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    m = float(np.abs(w64).max()) if clip is None else float(clip)
    if m == 0.0:
        s = np.float32(1.0)
    else:
        s = np.float32(m / (half - 1))
    q = np.clip(np.rint(w64 / float(s)) + half, 0, Q).astype(np.uint8)
    return Quantized(q, s, half, "unsigned", bits)


def histogram(q: np.ndarray, bits: int) -> np.ndarray:
    """Counts of every code value ``0 .. 2^bits - 1`` (int64)."""
    return np.bincount(np.asarray(q, dtype=np.uint8).ravel(), minlength=1 << bits).astype(np.int64)


def entropy_bits(counts: np.ndarray) -> float:
    """Empirical entropy ``-sum p log2 p`` (bits per symbol) of a histogram."""
    c = np.asarray(counts, dtype=np.float64)
    n = c.sum()
    p = c[c > 0] / n
    return float(-(p * np.log2(p)).sum())


def quantize_mixed(w: np.ndarray, bits: int) -> Quantized:
    """Per-tensor choice between the two schemes: lower code entropy wins."""
    a = quantize_asymmetric(w, bits)
    u = quantize_unsigned(w, bits)
    ha = entropy_bits(histogram(a.q, bits))
    hu = entropy_bits(histogram(u.q, bits))
    return u if hu < ha else a


def dequant_f64(qz: Quantized) -> np.ndarray:
    """``scale * (q - zp)`` in float64 (for quantizer error checks only)."""
    return float(qz.scale) * (qz.q.astype(np.float64) - qz.zero_point)
